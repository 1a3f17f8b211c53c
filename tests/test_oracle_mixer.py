"""Pins of the oracle's mixer (oracle.mixer_prefill, oracle.mixer_step): the layer core with
the bias-free in- and out-projections and the group RMSNorm around it (hyper.ai summary,
section "方法"; neurohive, section "Архитектура"). The core (conv1d, ssd_scan,
state_update_tokens) and group_rmsnorm are pinned in their own modules; the products are
numpy matmuls. These tests pin what the composition adds, against other code paths:

- zeroing the z rows of w_in gives out = 0 exactly (SiLU(0) = 0 gates everything, the norm
  of a zero group is zero): z is the first column block and the gate is applied;
- with identity projections (d_model = E, w_in = I, w_out = [I; 0]) the mixer is the core
  and the norm applied to the column blocks of hidden taken by hand;
- a prefill of L tokens followed by a step of T tokens equals a prefill of L + T tokens
  (outputs, conv history and state);
- causality: changing one token leaves every earlier output bitwise unchanged;
- io "bf16" rounds exactly the stored intermediates: with bf16-exact inputs and identity
  projections it equals the core with its own bf16 rounding.
"""
import numpy as np

import oracle
import seeded_inputs as si

H, G = 4, 2
DI = H * 64
CC = DI + 2 * G * 128
E = DI + CC + H


def cfg(cid, io="f32", seqlen=40):
    return si.Config(cid=cid, name=f"mixer{cid}", batch=2, seqlen=seqlen, nheads=H, ngroups=G, chunk=64,
                     io=io, h0_std=0.2)


def setup(c, d_model):
    p = si.draw_params(c)
    w = si.draw_mixer_weights(c, d_model)
    hid = si.draw_hidden(c, d_model)
    return p, w, hid, si.draw_conv_state(c), si.draw_h0(c)


def run(c, p, w, hid, cs, h0, **kw):
    return oracle.mixer_prefill(hid, w["w_in"], p["conv_w"], p["conv_b"], cs, p["dt_bias"], p["A"], p["D"], h0,
                                w["norm_w"], w["w_out"], nheads=H, ngroups=G, io=c.io, **kw)


def test_zero_z_rows_give_zero_output():
    c = cfg(950)
    p, w, hid, cs, h0 = setup(c, 64)
    w = dict(w, w_in=w["w_in"].copy())
    w["w_in"][:DI] = 0
    out, _, _ = run(c, p, w, hid, cs, h0)
    assert np.all(out == 0)
    w2 = dict(w, w_in=w["w_in"].copy())
    w2["w_in"][:DI] = 1e-3   # not zero: not zero out
    out2, _, _ = run(c, p, w2, hid, cs, h0)
    assert np.abs(out2).max() > 0


def test_identity_projections_reduce_to_the_core():
    c = cfg(951)
    p, w, _, cs, h0 = setup(c, E)
    hid = si.draw_hidden(c, E)
    w_in = np.eye(E, dtype=np.float32)
    w_out = np.zeros((E, DI), dtype=np.float32)
    w_out[:DI] = np.eye(DI, dtype=np.float32)
    out, hist, hf = oracle.mixer_prefill(hid, w_in, p["conv_w"], p["conv_b"], cs, p["dt_bias"], p["A"], p["D"],
                                         h0, w["norm_w"], w_out, nheads=H, ngroups=G)
    z, xbc, dt = hid[..., :DI], hid[..., DI:DI + CC], hid[..., DI + CC:]
    xr, hist_r = oracle.conv1d(xbc, p["conv_w"], p["conv_b"], cs)
    x, Bm, Cm = oracle.split_xbc(xr, H, G)
    y, hf_r = oracle.ssd_scan(x, Bm, Cm, dt, p["dt_bias"], p["A"], p["D"], z, h0, ngroups=G)
    yn = oracle.group_rmsnorm(y, w["norm_w"], ngroups=G)
    np.testing.assert_array_equal(out[..., DI:], 0)
    np.testing.assert_allclose(out[..., :DI], yn, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(hist, hist_r)
    np.testing.assert_array_equal(hf, hf_r)


def test_prefill_then_step_equals_longer_prefill():
    L, T, DM = 37, 3, 64
    c = cfg(952, seqlen=L + T)
    p, w, hid, cs, h0 = setup(c, DM)
    whole, hist, hf = run(c, p, w, hid, cs, h0)
    first, hist1, hf1 = run(c, p, w, hid[:, :L], cs, h0)
    step, hist2, hf2 = oracle.mixer_step(hid[:, L:], w["w_in"], p["conv_w"], p["conv_b"], hist1, p["dt_bias"],
                                         p["A"], p["D"], hf1, w["norm_w"], w["w_out"], nheads=H, ngroups=G)
    np.testing.assert_allclose(np.concatenate([first, step], 1), whole, rtol=1e-9, atol=1e-11)
    np.testing.assert_array_equal(hist2, hist)
    np.testing.assert_allclose(hf2, hf, rtol=1e-9, atol=1e-12)


def test_causality():
    c = cfg(953)
    p, w, hid, cs, h0 = setup(c, 64)
    out, _, _ = run(c, p, w, hid, cs, h0)
    hid2 = hid.copy()
    hid2[:, 25] += 1.0
    out2, _, _ = run(c, p, w, hid2, cs, h0)
    np.testing.assert_array_equal(out2[:, :25], out[:, :25])
    assert not np.array_equal(out2[:, 25], out[:, 25])


def test_bf16_rounds_the_stored_intermediates():
    """Identity projections in bf16 mode: zx = hidden is bf16-exact already, so the mixer
    equals conv1d -> round -> ssd_scan -> round -> group_rmsnorm -> round, projected by w_out."""
    c = cfg(954, io="bf16")
    p, w, _, cs, h0 = setup(c, E)
    hid = si.draw_hidden(c, E)
    w_in = np.eye(E, dtype=np.float32)
    w_out = np.zeros((E, DI), dtype=np.float32)
    w_out[:DI] = np.eye(DI, dtype=np.float32)
    out, _, _ = oracle.mixer_prefill(hid, w_in, p["conv_w"], p["conv_b"], cs, p["dt_bias"], p["A"], p["D"], h0,
                                     w["norm_w"], w_out, nheads=H, ngroups=G, io="bf16")
    z, xbc, dt = hid[..., :DI], hid[..., DI:DI + CC], hid[..., DI + CC:]
    xr, _ = oracle.conv1d(xbc, p["conv_w"], p["conv_b"], cs)
    x, Bm, Cm = oracle.split_xbc(oracle.round_bf16(xr), H, G)
    y, _ = oracle.ssd_scan(x, Bm, Cm, dt, p["dt_bias"], p["A"], p["D"], z, h0, ngroups=G)
    yn = oracle.round_bf16(oracle.group_rmsnorm(oracle.round_bf16(y), w["norm_w"], ngroups=G))
    np.testing.assert_allclose(out[..., :DI], yn, rtol=1e-13, atol=1e-13)
    assert np.all(yn == oracle.round_bf16(yn))
