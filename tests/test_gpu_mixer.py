"""Parity of the mixer calls (mamba2_mixer_prefill, mamba2_mixer_step) with the oracle's
mixer_prefill / mixer_step (hyper.ai summary, section "方法"; neurohive, section
"Архитектура": bias-free projections and RMSNorm around the Mamba-2 layer).

The oracle rounds to bf16 exactly the intermediates the library stores in bf16, so the
bar is the layer core's: max error <= 2e-2 * rms (bf16) or 1e-5 * rms (f32) on the output,
the state and the conv history (which holds projected rows, so it is not bitwise). Cases: the fused chunk-64 prefill with a
ragged tail, the chunk-128 path, fp32 io, the step with 1 and 3 tokens in both io types, a
prefill followed by a step, and the 12B-shape 8192-token call the benchmark times, checked
stage by stage on sampled rows and on two full heads through the documented workspace.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_helpers import assert_close, dev, dev32, empty, host, torch

pytestmark = pytest.mark.gpu

m2 = pytest.importorskip("state_space_sequence_causal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")


def case(cid, B, L, H, G, DM, io="bf16", chunk=64):
    c = si.Config(cid=cid, name=f"mixer{cid}", batch=B, seqlen=L, nheads=H, ngroups=G, chunk=chunk, io=io,
                  h0_std=0.2)
    return c, si.draw_params(c), si.draw_mixer_weights(c, DM), si.draw_hidden(c, DM), si.draw_conv_state(c), \
        si.draw_h0(c)


def gpu_prefill(c, p, w, hid, cs0, h0, workspace=None):
    t = torch()
    B, L, DM = hid.shape
    cs = dev(cs0, c.io)
    hf = t.empty((B, c.nheads, 128, 64), dtype=t.float32, device="cuda")
    out = empty((B, L, DM), c.io)
    m2.mamba2_mixer_prefill(dev(hid, c.io), dev(w["w_in"], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cs,
                            dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), dev32(h0), hf, dev32(w["norm_w"]),
                            dev(w["w_out"], c.io), out, ngroups=c.ngroups, chunk=c.chunk, workspace=workspace)
    t.cuda.synchronize()
    return host(out), host(cs), host(hf)


def gpu_step(c, p, w, hid, cs0, h0):
    t = torch()
    B, T, DM = hid.shape
    cs, ss = dev(cs0, c.io), dev32(h0)
    out = empty((B, T, DM), c.io)
    m2.mamba2_mixer_step(dev(hid, c.io), dev(w["w_in"], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cs,
                         dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), ss, dev32(w["norm_w"]),
                         dev(w["w_out"], c.io), out, ngroups=c.ngroups)
    t.cuda.synchronize()
    return host(out), host(cs), host(ss)


def ref_prefill(c, p, w, hid, cs0, h0):
    return oracle.mixer_prefill(hid, w["w_in"], p["conv_w"], p["conv_b"], cs0, p["dt_bias"], p["A"], p["D"], h0,
                                w["norm_w"], w["w_out"], nheads=c.nheads, ngroups=c.ngroups, io=c.io)


def ref_step(c, p, w, hid, cs0, h0):
    return oracle.mixer_step(hid, w["w_in"], p["conv_w"], p["conv_b"], cs0, p["dt_bias"], p["A"], p["D"], h0,
                             w["norm_w"], w["w_out"], nheads=c.nheads, ngroups=c.ngroups, io=c.io)


def check(got, ref, io, what):
    (out, cs, st), (ro, rcs, rst) = got, ref
    e1 = assert_close(out, ro, io, f"{what} out")
    e2 = assert_close(st, rst, io, f"{what} state", rounded=False)
    # the history holds the last raw xBC rows: GEMM outputs rounded to io, so a value near a
    # rounding boundary may land on the neighbouring grid point
    assert_close(cs, rcs, io, f"{what} conv_state")
    print(f"{what}: out {e1:.2e} state {e2:.2e}", flush=True)


@pytest.mark.parametrize("cid,B,L,H,G,DM,io,chunk", [
    (960, 2, 200, 8, 2, 256, "bf16", 64),
    (961, 1, 300, 16, 8, 512, "bf16", 128),
    (962, 1, 130, 4, 1, 128, "f32", 64),
    (963, 1, 2, 4, 1, 128, "bf16", 64),
])
def test_prefill(cid, B, L, H, G, DM, io, chunk):
    c, p, w, hid, cs0, h0 = case(cid, B, L, H, G, DM, io, chunk)
    print(f"mixer prefill: B{B} L{L} H{H} G{G} d_model {DM} {io} chunk {chunk}", flush=True)
    check(gpu_prefill(c, p, w, hid, cs0, h0), ref_prefill(c, p, w, hid, cs0, h0), io, f"prefill {cid}")


@pytest.mark.parametrize("cid,B,T,io", [(964, 3, 1, "bf16"), (965, 3, 3, "bf16"), (966, 2, 2, "f32"),
                                        (967, 64, 1, "bf16")])
def test_step(cid, B, T, io):
    c, p, w, hid, cs0, h0 = case(cid, B, T, 16, 8, 256, io)
    print(f"mixer step: B{B} T{T} {io}", flush=True)
    check(gpu_step(c, p, w, hid, cs0, h0), ref_step(c, p, w, hid, cs0, h0), io, f"step {cid}")


def test_prefill_then_step():
    """A 70-token prefill, then a 3-token step from the caches it left, against the
    oracle's 73-token prefill."""
    L, T = 70, 3
    c, p, w, hid, cs0, h0 = case(968, 2, L + T, 8, 2, 256)
    first, cs1, h1 = gpu_prefill(c, p, w, hid[:, :L], cs0, h0)
    out2, cs2, h2 = gpu_step(c, p, w, hid[:, L:], cs1, h1)     # the caches' exact values
    ro, rcs, rh = ref_prefill(c, p, w, hid, cs0, h0)
    assert_close(np.concatenate([first, out2], 1), ro, "bf16", "prefill + step out")
    assert_close(h2, rh, "bf16", "prefill + step state", rounded=False)
    assert_close(cs2, rcs, "bf16", "prefill + step conv_state")


def test_12b_shape_8k_stage_by_stage():
    """The call the benchmark times (12B shape: 160 heads, 8 groups, d_model 5120, 8192
    tokens, chunk 64, bf16). The workspace keeps every stage: the projected rows [8192][Es]
    (z | xBC | dt_raw), the core's output and the normalised output (each [8192][10240]).
    Sampled rows check both projections and the norm against the oracle on the GPU's own
    stage inputs; two whole heads (groups 0 and 7) check the layer core on its inputs."""
    t = torch()
    H, G, DM, L = 160, 8, 5120, 8192
    c = si.Config(cid=969, name="mixer-12b-8k", batch=1, seqlen=L, nheads=H, ngroups=G, chunk=64, io="bf16")
    p, w, hid = si.draw_params(c), si.draw_mixer_weights(c, DM), si.draw_hidden(c, DM)
    d = m2.make_dims(1, L, H, G, 64, m2.MAMBA2_BF16)
    ws = t.empty(m2.mamba2_mixer_prefill_workspace_bytes(d, DM), dtype=t.uint8, device="cuda")
    print("mixer 12B 8k: running", flush=True)
    out, _, hf = gpu_prefill(c, p, w, hid, np.zeros((1, 3, c.conv_channels), np.float32),
                             np.zeros((1, H, 128, 64), np.float32), workspace=ws)
    DI, CC = H * 64, c.conv_channels
    E = DI + CC + H
    Es = -(-E // 8) * 8
    a256 = lambda v: -(-v // 256) * 256
    zx = host(ws[:L * Es * 2].view(t.bfloat16).view(L, Es))
    yoff = a256(L * Es * 2)
    yc = host(ws[yoff:yoff + L * DI * 2].view(t.bfloat16).view(L, DI))
    noff = yoff + a256(L * DI * 2)
    ynr = host(ws[noff:noff + L * DI * 2].view(t.bfloat16).view(L, DI))
    rows = np.array([0, 1, 63, 64, 1000, 4095, 4096, 6000, 8190, 8191])
    h = hid[0, rows]
    proj = oracle.round_bf16(oracle._project(h, w["w_in"]))
    assert_close(zx[rows, :E], proj, "bf16", "in-projection")
    yn = oracle.round_bf16(oracle.group_rmsnorm(yc[rows], w["norm_w"], ngroups=G))
    assert_close(ynr[rows], yn, "bf16", "group RMSNorm")
    assert_close(out[0, rows], oracle._project(ynr[rows], w["w_out"]), "bf16", "out-projection")
    # the layer core on two heads, from the GPU's projected rows
    for hh in (0, H - 1):
        g = hh // (H // G)
        xs = slice(hh * 64, hh * 64 + 64)
        bs = slice(DI + g * 128, DI + g * 128 + 128)
        cs_ = slice(DI + G * 128 + g * 128, DI + G * 128 + g * 128 + 128)
        raw = zx[:, DI:DI + CC]
        chans = np.concatenate([raw[:, xs], raw[:, bs], raw[:, cs_]], 1)[None]
        wsel = np.concatenate([p["conv_w"][xs], p["conv_w"][bs], p["conv_w"][cs_]])
        bsel = np.concatenate([p["conv_b"][xs], p["conv_b"][bs], p["conv_b"][cs_]])
        conv, _ = oracle.conv1d(chans, wsel, bsel)
        conv = oracle.round_bf16(conv)
        z = zx[None, :, xs]
        y, hr = oracle.ssd_scan(conv[..., :64], conv[..., 64:192], conv[..., 192:], zx[None, :, DI + CC + hh:DI + CC + hh + 1],
                                p["dt_bias"][hh:hh + 1], p["A"][hh:hh + 1], p["D"][hh:hh + 1], z, None, ngroups=1)
        e1 = assert_close(yc[:, xs], y[0], "bf16", f"core y head {hh}")
        e2 = assert_close(hf[0, hh], hr[0, 0], "bf16", f"core state head {hh}", rounded=False)
        print(f"head {hh}: y {e1:.2e} state {e2:.2e}", flush=True)


def test_prefill_seqlen_zero_and_strided_hidden():
    """seqlen 0 carries h0 into h_final and leaves the conv history alone; a hidden tensor
    that is a column view of a wider one (row stride 384 for d_model 256) gives the bits of
    the same rows stored densely."""
    t = torch()
    c, p, w, hid, cs0, h0 = case(970, 2, 90, 8, 2, 256)
    # seqlen 0
    hf = t.empty((2, 8, 128, 64), dtype=t.float32, device="cuda")
    cs = dev(cs0, "bf16")
    out0 = empty((2, 0, 256), "bf16")
    m2.mamba2_mixer_prefill(empty((2, 0, 256), "bf16"), dev(w["w_in"], "bf16"), dev32(p["conv_w"]),
                            dev32(p["conv_b"]), cs, dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), dev32(h0), hf,
                            dev32(w["norm_w"]), dev(w["w_out"], "bf16"), out0, ngroups=2, chunk=64)
    t.cuda.synchronize()
    np.testing.assert_array_equal(host(hf), np.asarray(h0, np.float32))
    np.testing.assert_array_equal(host(cs), cs0)
    # strided hidden
    dense = gpu_prefill(c, p, w, hid, cs0, h0)
    wide = np.zeros((2, 90, 384), np.float32)
    wide[..., 64:320] = hid
    hv = dev(wide, "bf16")[..., 64:320]
    cs2 = dev(cs0, "bf16")
    hf2 = t.empty((2, 8, 128, 64), dtype=t.float32, device="cuda")
    out2 = empty((2, 90, 256), "bf16")
    m2.mamba2_mixer_prefill(hv, dev(w["w_in"], "bf16"), dev32(p["conv_w"]), dev32(p["conv_b"]), cs2,
                            dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), dev32(h0), hf2, dev32(w["norm_w"]),
                            dev(w["w_out"], "bf16"), out2, ngroups=2, chunk=64)
    t.cuda.synchronize()
    for g, r in zip((host(out2), host(cs2), host(hf2)), dense):
        np.testing.assert_array_equal(g, r)


def test_deterministic():
    c, p, w, hid, cs0, h0 = case(971, 1, 150, 8, 2, 256)
    a = gpu_prefill(c, p, w, hid, cs0, h0)
    b = gpu_prefill(c, p, w, hid, cs0, h0)
    for g, r in zip(a, b):
        np.testing.assert_array_equal(g, r)
