"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The pages print no worked example, so the oracle is pinned by closed forms,
textbook special cases computed with numpy library routines, invariants of the
recurrence, and the brute-force unrolled form (oracle/brute.py). Each test
names the mistake it is there to catch.

Recurrence (benchmark spec of the Mamba-2 core; Mamba-2 block of the
Nemotron-Nano-2 report, hyper.ai summary section "方法"):
    h_t = exp(dt_t A) h_{t-1} + dt_t B_t x_t^T,  y_t = C_t h_t + D x_t,  gated by SiLU(z).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.brute import ssd_brute
import seeded_inputs as si

HERE = os.path.dirname(os.path.abspath(__file__))


def softplus(v):
    return np.logaddexp(0.0, v)


def silu(v):
    return v / (1.0 + np.exp(-v))


def rand_case(seed, B=2, L=29, H=4, G=2, P=8, N=6, W=4, A_scale=1.0, with_h0=True):
    r = np.random.default_rng(seed)
    c = dict(
        x=r.standard_normal((B, L, H * P)),
        Bm=r.standard_normal((B, L, G * N)) / np.sqrt(N),
        Cm=r.standard_normal((B, L, G * N)) / np.sqrt(N),
        dt_raw=r.standard_normal((B, L, H)),
        dt_bias=np.log(np.expm1(np.exp(r.uniform(np.log(1e-2), np.log(0.5), H)))),
        A=-np.exp(r.uniform(0, np.log(16), H)) * A_scale,
        D=r.standard_normal(H),
        z=r.standard_normal((B, L, H * P)),
        h0=r.standard_normal((B, H, N, P)) * 0.3 if with_h0 else None,
    )
    return c, dict(B=B, L=L, H=H, G=G, P=P, N=N, W=W)


def scan(c, s, **kw):
    return oracle.ssd_scan(c["x"], c["Bm"], c["Cm"], c["dt_raw"], c["dt_bias"], c["A"], c["D"],
                           c["z"], c["h0"], ngroups=s["G"], **kw)


# --------------------------------------------------------------------------- golden shapes
def test_golden_shapes_define_configs():
    """The config table's Mamba-2 shapes are the ones the pages state."""
    facts = {f["name"]: f["value"] for f in json.load(open(os.path.join(HERE, "golden", "mamba2_shapes.json")))["facts"]}
    for cid, cfg in si.WORKLOADS.items():
        assert cfg.headdim == facts["headdim"]
        assert cfg.dstate == facts["dstate"]
        assert cfg.conv_width == facts["conv_width"]
        if cid != 0:
            assert cfg.ngroups == facts["ngroups"]
    c1 = si.PREFILL_12B_8K
    assert c1.d_inner == facts["expand"] * facts["hidden_12b"]
    assert c1.seqlen == facts["pretrain_seqlen"]
    assert si.PREFILL_12B_128K.seqlen == facts["max_context"]
    for cid in (2, 4):
        assert facts["mamba_heads_9b_min"] <= si.WORKLOADS[cid].nheads <= facts["mamba_heads_9b_max"]
    assert si.PREFILL_12B_8K.conv_channels == 10240 + 2 * 8 * 128


# --------------------------------------------------------------------------- conv
def test_conv_impulse_gives_reversed_taps():
    """Catches a flipped tap order or an off-by-one in the causal window."""
    r = np.random.default_rng(1)
    Cc, W, L, t0 = 5, 4, 12, 4
    w = r.uniform(-0.5, 0.5, (Cc, W))
    b = r.uniform(-0.1, 0.1, Cc)
    u = np.zeros((1, L, Cc))
    u[0, t0, :] = 1.0
    out, _ = oracle.conv1d(u, w, b)
    for t in range(L):
        k = t - t0  # lag
        v = b + (w[:, W - 1 - k] if 0 <= k < W else 0.0)
        np.testing.assert_allclose(out[0, t], silu(v), rtol=0, atol=1e-15)


def test_conv_identity_taps_is_silu():
    r = np.random.default_rng(2)
    u = r.standard_normal((2, 9, 7))
    w = np.zeros((7, 4))
    w[:, 3] = 1.0
    out, _ = oracle.conv1d(u, w, None, r.standard_normal((2, 3, 7)))
    np.testing.assert_allclose(out, silu(u), rtol=1e-15, atol=0)


def test_conv_ramp_closed_form():
    """u_t = t+1 on every channel: for t >= W-1, v_t = bias + (t+2-W) sum_k w_k + sum_k k w_k."""
    r = np.random.default_rng(3)
    Cc, W, L = 6, 4, 20
    w = r.uniform(-0.5, 0.5, (Cc, W))
    b = r.uniform(-0.1, 0.1, Cc)
    u = np.broadcast_to(np.arange(1, L + 1, dtype=np.float64)[None, :, None], (1, L, Cc)).copy()
    out, _ = oracle.conv1d(u, w, b)
    k = np.arange(W)
    for t in range(W - 1, L):
        v = b + (t + 2 - W) * w.sum(1) + (w * k).sum(1)
        np.testing.assert_allclose(out[0, t], silu(v), rtol=1e-14)


@pytest.mark.parametrize("L1", [0, 1, 2, 3, 7])
def test_conv_state_handoff(L1):
    """conv over [0,L) equals conv over [0,L1) then [L1,L) through the returned history,
    and the history is the last W-1 raw inputs (drawing on the old history when L < W-1)."""
    r = np.random.default_rng(10 + L1)
    B, L, Cc, W = 2, 11, 5, 4
    u = r.standard_normal((B, L, Cc))
    w = r.uniform(-0.5, 0.5, (Cc, W))
    b = r.uniform(-0.1, 0.1, Cc)
    s0 = r.standard_normal((B, W - 1, Cc))
    full, sf = oracle.conv1d(u, w, b, s0)
    if L1 > 0:
        a, s1 = oracle.conv1d(u[:, :L1], w, b, s0)
        ext = np.concatenate([s0, u[:, :L1]], axis=1)
        np.testing.assert_array_equal(s1, ext[:, -(W - 1):])
    else:
        a, s1 = np.zeros((B, 0, Cc)), s0
    c, s2 = oracle.conv1d(u[:, L1:], w, b, s1)
    np.testing.assert_allclose(np.concatenate([a, c], 1), full, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(s2, sf)
    np.testing.assert_array_equal(sf, u[:, -(W - 1):])


# --------------------------------------------------------------------------- scan closed forms
def test_A_zero_is_cumulative_sum():
    """A = 0: h_t = h0 + sum_{s<=t} dt_s B_s x_s^T (numpy cumsum). Catches B/C swapped,
    a transposed state, a wrong softplus (dt_raw spans +-30), a missing gate or D term."""
    c, s = rand_case(4, L=23)
    c["A"] = np.zeros(s["H"])
    c["dt_raw"] = c["dt_raw"] * 10.0
    y, hf = scan(c, s)
    B, L, H, G, P, N = (s[k] for k in "B L H G P N".split())
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            dt = softplus(c["dt_raw"][b, :, h] + c["dt_bias"][h])
            X = c["x"][b, :, h * P:(h + 1) * P]
            Bg = c["Bm"][b, :, g * N:(g + 1) * N]
            Cg = c["Cm"][b, :, g * N:(g + 1) * N]
            outer = dt[:, None, None] * Bg[:, :, None] * X[:, None, :]     # [L][N][P]
            hs = c["h0"][b, h][None] + np.cumsum(outer, axis=0)
            yy = np.einsum("tn,tnp->tp", Cg, hs) + c["D"][h] * X
            yy *= silu(c["z"][b, :, h * P:(h + 1) * P])
            np.testing.assert_allclose(y[b, :, h * P:(h + 1) * P], yy, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(hf[b, h], hs[-1], rtol=1e-12, atol=1e-12)


def test_scalar_geometric_series():
    """N = P = H = G = 1, constant inputs: h_t = a^{t+1} h0 + dt b x (1 - a^{t+1}) / (1 - a)."""
    L = 40
    dt_raw, bias, A = 0.3, -0.2, -0.7
    bb, cc, xx, h0, Dv = 0.8, -1.3, 0.6, 2.0, 0.25
    dt = np.log1p(np.exp(dt_raw + bias))
    a = np.exp(dt * A)
    y, hf = oracle.ssd_scan(np.full((1, L, 1), xx), np.full((1, L, 1), bb), np.full((1, L, 1), cc),
                            np.full((1, L, 1), dt_raw), np.array([bias]), np.array([A]),
                            np.array([Dv]), None, np.array([[[[h0]]]]), ngroups=1)
    t = np.arange(L) + 1
    h = a ** t * h0 + dt * bb * xx * (1 - a ** t) / (1 - a)
    np.testing.assert_allclose(y[0, :, 0], cc * h + Dv * xx, rtol=1e-13)
    np.testing.assert_allclose(hf[0, 0, 0, 0], h[-1], rtol=1e-13)


def test_zero_input_is_pure_decay():
    """x = 0: h_t = exp(A sum_{r<=t} dt_r) h0 exactly; catches a sign error in the decay."""
    c, s = rand_case(5, L=17)
    c["x"] = np.zeros_like(c["x"])
    c["z"] = None
    y, hf = scan(c, s)
    B, L, H, G, P, N = (s[k] for k in "B L H G P N".split())
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            dt = softplus(c["dt_raw"][b, :, h] + c["dt_bias"][h])
            dec = np.exp(c["A"][h] * np.cumsum(dt))
            Cg = c["Cm"][b, :, g * N:(g + 1) * N]
            yy = dec[:, None] * (Cg @ c["h0"][b, h])
            np.testing.assert_allclose(y[b, :, h * P:(h + 1) * P], yy, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(hf[b, h], dec[-1] * c["h0"][b, h], rtol=1e-12)


@pytest.mark.parametrize("which", ["B", "C"])
def test_B_or_C_zero_leaves_skip_and_gate(which):
    """B = 0 (h0 = 0) or C = 0: out = D x * SiLU(z). Catches a dropped D term or gate."""
    c, s = rand_case(6, with_h0=(which == "C"))
    c["Bm" if which == "B" else "Cm"] = np.zeros_like(c["Bm"])
    y, _ = scan(c, s)
    H, P = s["H"], s["P"]
    Dx = np.repeat(c["D"], P)[None, None, :] * c["x"]
    np.testing.assert_allclose(y, Dx * silu(c["z"]), rtol=1e-14, atol=1e-15)


def test_A_D_zero_is_causal_masked_matmul():
    """A = D = 0, h0 = 0, no gate: Y = (tril(C B^T) * dt^T) X, computed with numpy matmul."""
    c, s = rand_case(7, L=31, with_h0=False)
    c["A"] = np.zeros(s["H"])
    y, _ = oracle.ssd_scan(c["x"], c["Bm"], c["Cm"], c["dt_raw"], c["dt_bias"], c["A"], None,
                           None, None, ngroups=s["G"])
    B, H, G, P, N = (s[k] for k in "B H G P N".split())
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            dt = softplus(c["dt_raw"][b, :, h] + c["dt_bias"][h])
            M = np.tril(c["Cm"][b, :, g * N:(g + 1) * N] @ c["Bm"][b, :, g * N:(g + 1) * N].T) * dt[None, :]
            np.testing.assert_allclose(y[b, :, h * P:(h + 1) * P], M @ c["x"][b, :, h * P:(h + 1) * P],
                                       rtol=1e-12, atol=1e-13)


def test_contiguous_head_to_group_map():
    """G = 2, H = 4: zeroing group 1's B (h0 = 0) silences exactly heads 2 and 3 (g = h // (H/G))."""
    c, s = rand_case(8, with_h0=False)
    N = s["N"]
    c["Bm"][:, :, N:2 * N] = 0.0
    y, _ = scan(c, s)
    P = s["P"]
    Dx = np.repeat(c["D"], P)[None, None, :] * c["x"] * silu(c["z"])
    np.testing.assert_allclose(y[:, :, 2 * P:], Dx[:, :, 2 * P:], rtol=1e-14, atol=1e-15)
    assert np.abs(y[:, :, :2 * P] - Dx[:, :, :2 * P]).max() > 1e-3


# --------------------------------------------------------------------------- three forms agree
@pytest.mark.parametrize("Q", [1, 3, 5, 8, 29, 64])
def test_sequential_equals_chunked(Q):
    """O1 = O2 for chunk lengths that divide L and that do not (L = 29)."""
    c, s = rand_case(9)
    y1, h1 = scan(c, s)
    y2, h2 = oracle.ssd_chunked(c["x"], c["Bm"], c["Cm"], c["dt_raw"], c["dt_bias"], c["A"], c["D"],
                                c["z"], c["h0"], ngroups=s["G"], chunk=Q)
    scale = np.sqrt(np.mean(y1 ** 2))
    assert np.abs(y1 - y2).max() <= 1e-12 * scale
    assert np.abs(h1 - h2).max() <= 1e-12 * np.sqrt(np.mean(h1 ** 2))


def test_sequential_equals_brute_force():
    """O1 = O3 (explicit running products, no exp of sums)."""
    c, s = rand_case(11, L=19)
    y1, _ = scan(c, s)
    y3 = ssd_brute(c["x"], c["Bm"], c["Cm"], c["dt_raw"], c["dt_bias"], c["A"], c["D"], c["z"],
                   c["h0"], ngroups=s["G"])
    np.testing.assert_allclose(y1, y3, rtol=1e-11, atol=1e-13)


def test_chunked_equals_brute_force_strong_decay():
    """Strong decay (|A| up to 160): the chunked log-decay differences still agree with products."""
    c, s = rand_case(12, L=21, A_scale=10.0)
    y2, _ = oracle.ssd_chunked(c["x"], c["Bm"], c["Cm"], c["dt_raw"], c["dt_bias"], c["A"], c["D"],
                               c["z"], c["h0"], ngroups=s["G"], chunk=8)
    y3 = ssd_brute(c["x"], c["Bm"], c["Cm"], c["dt_raw"], c["dt_bias"], c["A"], c["D"], c["z"],
                   c["h0"], ngroups=s["G"])
    np.testing.assert_allclose(y2, y3, rtol=1e-10, atol=1e-13)


# --------------------------------------------------------------------------- invariants
def _layer_inputs(seed, B=2, L=13, H=4, G=2, P=8, N=6, W=4):
    r = np.random.default_rng(seed)
    Cc = H * P + 2 * G * N
    return dict(
        u=r.standard_normal((B, L, Cc)), w=r.uniform(-0.5, 0.5, (Cc, W)), b=r.uniform(-0.1, 0.1, Cc),
        cs=r.standard_normal((B, W - 1, Cc)), z=r.standard_normal((B, L, H * P)),
        dt_raw=r.standard_normal((B, L, H)), dt_bias=np.log(np.expm1(np.exp(r.uniform(-4, -1, H)))),
        A=-np.exp(r.uniform(0, 2.7, H)), D=r.standard_normal(H), h0=r.standard_normal((B, H, N, P)) * 0.2,
    ), dict(B=B, L=L, H=H, G=G, P=P, N=N, W=W)


def _prefill(d, s, t0, t1, cs, h0):
    xbc, cs2 = oracle.conv1d(d["u"][:, t0:t1], d["w"], d["b"], cs)
    x, Bm, Cm = oracle.split_xbc(xbc, s["H"], s["G"], s["P"], s["N"])
    y, hf = oracle.ssd_scan(x, Bm, Cm, d["dt_raw"][:, t0:t1], d["dt_bias"], d["A"], d["D"],
                            d["z"][:, t0:t1], h0, ngroups=s["G"])
    return y, cs2, hf


def test_prefill_len1_equals_state_update():
    d, s = _layer_inputs(20, L=1)
    y, cs, hf = _prefill(d, s, 0, 1, d["cs"], d["h0"])
    y2, cs2, ss2 = oracle.state_update(d["u"][:, 0], d["w"], d["b"], d["cs"], d["dt_raw"][:, 0],
                                       d["dt_bias"], d["A"], d["D"], d["z"][:, 0], d["h0"],
                                       nheads=s["H"], ngroups=s["G"], headdim=s["P"], dstate=s["N"])
    np.testing.assert_allclose(y2, y[:, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(cs2, cs)
    np.testing.assert_allclose(ss2, hf, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("L1", [1, 5, 9])
def test_split_prefill_and_decode_handoff(L1):
    """prefill(L1) -> (conv_state, h) -> prefill(rest) equals prefill(L); and prefill(L1)
    followed by L-L1 decode steps equals it too."""
    d, s = _layer_inputs(21)
    L = s["L"]
    y, csf, hff = _prefill(d, s, 0, L, d["cs"], d["h0"])
    ya, csa, ha = _prefill(d, s, 0, L1, d["cs"], d["h0"])
    yb, csb, hb = _prefill(d, s, L1, L, csa, ha)
    np.testing.assert_allclose(np.concatenate([ya, yb], 1), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hb, hff, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(csb, csf)
    cs, ss = csa, ha
    for t in range(L1, L):
        yt, cs, ss = oracle.state_update(d["u"][:, t], d["w"], d["b"], cs, d["dt_raw"][:, t],
                                         d["dt_bias"], d["A"], d["D"], d["z"][:, t], ss,
                                         nheads=s["H"], ngroups=s["G"], headdim=s["P"], dstate=s["N"])
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ss, hff, rtol=1e-12, atol=1e-13)


def test_causality():
    c, s = rand_case(13)
    y, _ = scan(c, s)
    t0 = 11
    c["x"][:, t0] += 5.0
    c["dt_raw"][:, t0] += 1.0
    c["Bm"][:, t0] *= -2.0
    y2, _ = scan(c, s)
    np.testing.assert_array_equal(y2[:, :t0], y[:, :t0])
    assert np.abs(y2[:, t0] - y[:, t0]).max() > 1e-6


def test_batch_independence():
    c, s = rand_case(14, B=3)
    y, hf = scan(c, s)
    perm = [2, 0, 1]
    cp = {k: (v[perm] if (v is not None and v.ndim >= 3) else v) for k, v in c.items()}
    y2, hf2 = scan(cp, s)
    np.testing.assert_array_equal(y2, y[perm])
    np.testing.assert_array_equal(hf2, hf[perm])


def test_group_sharing_identical_groups_equals_one_group():
    c, s = rand_case(15, G=1)
    y1, h1 = scan(c, s)
    c2 = dict(c)
    c2["Bm"] = np.concatenate([c["Bm"], c["Bm"]], axis=2)
    c2["Cm"] = np.concatenate([c["Cm"], c["Cm"]], axis=2)
    y2, h2 = oracle.ssd_scan(c2["x"], c2["Bm"], c2["Cm"], c["dt_raw"], c["dt_bias"], c["A"], c["D"],
                             c["z"], c["h0"], ngroups=2)
    np.testing.assert_array_equal(y2, y1)
    np.testing.assert_array_equal(h2, h1)


def test_linear_in_x():
    """For fixed dt, B, C and no gate, with h0 = 0, y is linear in x."""
    c, s = rand_case(16, with_h0=False)
    c["z"] = None
    ya, _ = scan(c, s)
    x2 = np.random.default_rng(99).standard_normal(c["x"].shape)
    cb = dict(c, x=x2)
    yb, _ = scan(cb, s)
    cc = dict(c, x=2.0 * c["x"] - 3.0 * x2)
    yc, _ = scan(cc, s)
    np.testing.assert_allclose(yc, 2.0 * ya - 3.0 * yb, rtol=1e-11, atol=1e-12)


def test_head_subset_matches_full():
    c, s = rand_case(17)
    y, hf = scan(c, s)
    ys, hs = scan(c, s, heads=[3, 1])
    P = s["P"]
    for h in (1, 3):
        np.testing.assert_array_equal(ys[:, :, h * P:(h + 1) * P], y[:, :, h * P:(h + 1) * P])
        np.testing.assert_array_equal(hs[:, h], hf[:, h])
    assert np.all(ys[:, :, 0:P] == 0)


def test_threads_do_not_change_results():
    c, s = rand_case(18)
    y1, _ = scan(c, s, nthreads=1)
    y4, _ = scan(c, s, nthreads=4)
    np.testing.assert_array_equal(y1, y4)


def test_one_head_per_group_sublayer_matches_full():
    """The long-workload parity tests run the oracle on a sub-layer made of one head per
    group (its x, z, dt columns and every group's B and C). The recurrence is per head, so
    that sub-layer must reproduce the full layer's outputs for those heads exactly."""
    c, s = rand_case(19, H=8, G=4)
    y, hf = scan(c, s)
    P, N, G = s["P"], s["N"], s["G"]
    heads = [1, 2, 4, 7]
    cols = np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])
    sub = dict(c, x=c["x"][..., cols], z=c["z"][..., cols], dt_raw=c["dt_raw"][..., heads],
               dt_bias=c["dt_bias"][heads], A=c["A"][heads], D=c["D"][heads], h0=c["h0"][:, heads])
    ys, hs = scan(sub, dict(s, H=len(heads)))
    np.testing.assert_array_equal(ys, y[..., cols])
    np.testing.assert_array_equal(hs, hf[:, heads])
