"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Bar: max |gpu - oracle| <= 2e-2 * rms(oracle) for bf16 io with fp32 state and
<= 1e-5 * rms(oracle) for all-fp32, per output tensor, where an output stored in
the io type is allowed, on top, the rounding of its exact value to that type
(half an ulp at the value: no implementation can do better, and with heavy-tailed
outputs -- max/rms of 14 to 60 here -- that rounding alone exceeds 2e-2 * rms).
fp32 states get no such allowance; conv caches must match bitwise.
Each ABI call is checked on identical inputs (the oracle reads the exact
values the GPU read). Sizes span several chunks and a ragged last chunk; the
full-size workloads are checked on a head subset that covers every group.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_helpers import TOL, assert_close, compute_err, dev, dev32, empty, host, torch

pytestmark = pytest.mark.gpu

m2 = pytest.importorskip("state_space_sequence_causal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")


def small(cid, **kw):
    base = dict(cid=cid, name=f"case{cid}", batch=2, seqlen=300, nheads=16, ngroups=8, chunk=128,
                io="bf16", h0_std=0.5)
    base.update(kw)
    return si.Config(**base)


# --------------------------------------------------------------------------- prefill scan
def gpu_prefill(cfg, inp, chunk=None, z=True, D=True, h0=True, inplace=False, guard=0):
    t = torch()
    io, B, L, H, G = cfg.io, cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    xbc = dev(inp["xbc"], io)
    x, Bm, Cm = xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:]
    zt = dev(inp["z"], io) if z else None
    dt = dev(inp["dt_raw"], io)
    h0t = dev32(inp["h0"]) if h0 else None
    if inplace:
        hf = h0t
    else:
        hf = t.empty((B, H, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda")
    ybuf = empty(B * L * di + guard, io)
    if guard:
        ybuf[B * L * di:] = 12345.0
    y = ybuf[:B * L * di].view(B, L, di)
    m2.mamba2_ssd_prefill(x, Bm, Cm, dt, dev32(inp["dt_bias"]), dev32(inp["A"]),
                          dev32(inp["D"]) if D else None, zt, h0t, hf, y, ngroups=G,
                          chunk=chunk or cfg.chunk)
    t.cuda.synchronize()
    if guard:
        assert bool((ybuf[B * L * di:] == 12345.0).all()), "write past the end of y"
    return host(y), host(hf)


def oracle_prefill(cfg, inp, z=True, D=True, h0=True, heads=None):
    x, Bm, Cm = oracle.split_xbc(inp["xbc"], cfg.nheads, cfg.ngroups)
    return oracle.ssd_scan(x, Bm, Cm, inp["dt_raw"], inp["dt_bias"], inp["A"],
                           inp["D"] if D else None, inp["z"] if z else None,
                           inp["h0"] if h0 else None, ngroups=cfg.ngroups, heads=heads)


def check_prefill(cfg, **kw):
    inp = si.draw_prefill(cfg)
    heads = kw.pop("heads", None)
    yg, hg = gpu_prefill(cfg, inp, **kw)
    okw = {k: v for k, v in kw.items() if k in ("z", "D", "h0")}
    yr, hr = oracle_prefill(cfg, inp, heads=heads, **okw)
    if heads is not None:
        P = cfg.headdim
        cols = np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])
        yg, yr = yg[..., cols], yr[..., cols]
        hg, hr = hg[:, heads], hr[:, heads]
    ey = assert_close(yg, yr, cfg.io, f"{cfg.name} y")
    eh = assert_close(hg, hr, cfg.io, f"{cfg.name} h_final", rounded=False)
    print(f"{cfg.name}: y err/rms {ey:.2e}, h_final err/rms {eh:.2e}")
    return yg, hg


def test_prefill_tiny_f32_config():
    """All-fp32 tiny layer (B=1, L=256, 4 heads, 1 group, chunk 64)."""
    check_prefill(si.TINY_F32)


def test_prefill_f32_ragged_with_state():
    check_prefill(small(101, io="f32", chunk=64, seqlen=197, nheads=8, ngroups=2))


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_prefill_bf16_ragged_multichunk(chunk):
    check_prefill(small(102, chunk=chunk, seqlen=600))


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("opts", [dict(z=False), dict(D=False), dict(h0=False),
                                  dict(z=False, D=False, h0=False)])
def test_prefill_optional_operands(opts, chunk):
    check_prefill(small(103, seqlen=160, chunk=chunk), **opts)


@pytest.mark.parametrize("chunk", [64, 128])
def test_prefill_inplace_state(chunk):
    check_prefill(small(104, seqlen=129, chunk=chunk), inplace=True)


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("L", [1, 2, 31, 63, 64, 65, 128, 129])
def test_prefill_short_and_boundary_lengths(L, chunk):
    check_prefill(small(105, seqlen=L, batch=3, nheads=8, ngroups=2, chunk=chunk))


def test_prefill_len0_passes_state_through():
    cfg = small(106, seqlen=0)
    inp = si.draw_prefill(cfg)
    _, hg = gpu_prefill(cfg, inp)
    np.testing.assert_array_equal(hg, inp["h0"].astype(np.float64))


@pytest.mark.parametrize("chunk", [64, 128])
def test_prefill_one_group_many_heads(chunk):
    check_prefill(small(107, nheads=12, ngroups=1, seqlen=140, chunk=chunk))


def test_prefill_no_write_past_y():
    cfg = small(108, seqlen=77)
    inp = si.draw_prefill(cfg)
    gpu_prefill(cfg, inp, guard=4096)


def test_prefill_chunk_invariance_and_determinism():
    """Chunk 64 and 128 both meet the bar against the oracle (so they agree within twice
    it), and a repeated run is bitwise identical (no atomics, fixed reduction order)."""
    cfg = small(109, seqlen=512)
    inp = si.draw_prefill(cfg)
    yr, hr = oracle_prefill(cfg, inp)
    y64, h64 = gpu_prefill(cfg, inp, chunk=64)
    y128, h128 = gpu_prefill(cfg, inp, chunk=128)
    y256, h256 = gpu_prefill(cfg, inp, chunk=256)
    y128b, h128b = gpu_prefill(cfg, inp, chunk=128)
    y64b, h64b = gpu_prefill(cfg, inp, chunk=64)
    for yg, hg, q in ((y64, h64, 64), (y128, h128, 128), (y256, h256, 256)):
        assert_close(yg, yr, "bf16", f"chunk {q} y")
        assert_close(hg, hr, "bf16", f"chunk {q} h_final", rounded=False)
    assert compute_err(y64, y128, "bf16") <= 2 * TOL["bf16"]
    np.testing.assert_array_equal(y128, y128b)
    np.testing.assert_array_equal(h128, h128b)
    np.testing.assert_array_equal(y64, y64b)
    np.testing.assert_array_equal(h64, h64b)


@pytest.mark.parametrize("chunk", [64, 128])
def test_prefill_12b_8k_full_size_head_subset(chunk):
    """The 12B-shape 8k prefill at full size, with the benchmark's chunk of 64 and with 128,
    checked on 9 heads spanning all 8 groups."""
    cfg = si.PREFILL_12B_8K
    check_prefill(dataclasses.replace(cfg, chunk=chunk), heads=[0, 21, 40, 63, 77, 99, 118, 139, 159])


# --------------------------------------------------------------------------- conv1d
def gpu_conv(u_np, w, b, cs_np, io):
    t = torch()
    u = dev(u_np, io)
    out = empty(u.shape, io)
    cs = dev(cs_np, io) if cs_np is not None else None
    m2.mamba2_conv1d(u, dev32(w), dev32(b) if b is not None else None, cs, out)
    t.cuda.synchronize()
    return host(out), (host(cs) if cs is not None else None)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 2, 3, 64, 200])
@pytest.mark.parametrize("hist", [True, False])
def test_conv1d(io, L, hist):
    cfg = small(110, io=io, seqlen=L, nheads=8, ngroups=2)
    p = si.draw_params(cfg)
    u = si.draw_xbc(cfg)
    cs = si.draw_conv_state(cfg) if hist else None
    og, csg = gpu_conv(u, p["conv_w"], p["conv_b"], cs, io)
    orf, csr = oracle.conv1d(u, p["conv_w"], p["conv_b"], cs)
    assert_close(og, orf, io, f"conv L={L}")
    if hist:
        np.testing.assert_array_equal(csg, csr)


def test_conv1d_12b_channels_no_bias():
    cfg = si.config(si.PREFILL_12B_8K, seqlen=300)
    p = si.draw_params(cfg)
    u = si.draw_xbc(cfg)
    og, _ = gpu_conv(u, p["conv_w"], None, None, "bf16")
    orf, _ = oracle.conv1d(u, p["conv_w"], None, None)
    assert_close(og, orf, "bf16", "conv 12B")


# --------------------------------------------------------------------------- decode
def gpu_decode(cfg, params, step_inp, conv_state, ssm_state, z=True, D=True, bias=True):
    t = torch()
    io = cfg.io
    u = dev(step_inp["xbc"][:, 0], io)
    zt = dev(step_inp["z"][:, 0], io) if z else None
    dt = dev(step_inp["dt_raw"][:, 0], io)
    cs = dev(conv_state, io)
    ss = dev32(ssm_state)
    y = empty((cfg.batch, cfg.d_inner), io)
    m2.mamba2_state_update(u, dev32(params["conv_w"]), dev32(params["conv_b"]) if bias else None, cs, dt,
                           dev32(params["dt_bias"]), dev32(params["A"]), dev32(params["D"]) if D else None,
                           zt, ss, y, ngroups=cfg.ngroups)
    t.cuda.synchronize()
    return host(y), host(cs), host(ss)


def oracle_decode(cfg, params, step_inp, conv_state, ssm_state, z=True, D=True, bias=True):
    return oracle.state_update(step_inp["xbc"][:, 0], params["conv_w"], params["conv_b"] if bias else None,
                               conv_state, step_inp["dt_raw"][:, 0], params["dt_bias"], params["A"],
                               params["D"] if D else None, step_inp["z"][:, 0] if z else None,
                               ssm_state, nheads=cfg.nheads, ngroups=cfg.ngroups)


def check_decode(cfg, **opts):
    params = si.draw_params(cfg)
    step = si.draw_decode_step(cfg, 0)
    cs0, ss0 = si.draw_conv_state(cfg), si.draw_h0(cfg)
    yg, csg, ssg = gpu_decode(cfg, params, step, cs0, ss0, **opts)
    yr, csr, ssr = oracle_decode(cfg, params, step, cs0, ss0, **opts)
    np.testing.assert_array_equal(csg, csr)
    ey = assert_close(yg, yr, cfg.io, f"{cfg.name} y")
    es = assert_close(ssg, ssr, cfg.io, f"{cfg.name} state", rounded=False)
    print(f"{cfg.name}: y err/rms {ey:.2e}, state err/rms {es:.2e}")


def test_decode_9b_batch64_full():
    """The 9B-shape decode step (B=64, 128 heads, 8 groups), every output checked."""
    check_decode(si.DECODE_9B_B64)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_small(io):
    check_decode(small(111, io=io, seqlen=1, batch=3, nheads=12, ngroups=3))


def test_decode_12b_shape_20_heads_per_group():
    check_decode(small(112, seqlen=1, batch=2, nheads=160, ngroups=8))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_one_group_80_heads(io):
    """80 heads in one group: the group's conv channels exceed one pass of the workgroup's
    threads and each wave streams five heads."""
    check_decode(small(114, io=io, seqlen=1, batch=2, nheads=80, ngroups=1))


@pytest.mark.parametrize("opts", [dict(z=False), dict(D=False), dict(bias=False),
                                  dict(z=False, D=False, bias=False)])
def test_decode_optional_operands(opts):
    check_decode(small(115, seqlen=1, batch=3, nheads=16, ngroups=2), **opts)


# --------------------------------------------------------------------------- chained paths
def test_chained_conv_then_scan_f32():
    """conv1d -> ssd_prefill on device equals the oracle's conv -> scan end to end."""
    t = torch()
    cfg = si.TINY_F32
    inp = si.draw_prefill(cfg)
    cs = si.draw_conv_state(cfg)
    u = dev(inp["xbc"], "f32")
    xbc = empty(u.shape, "f32")
    csd = dev(cs, "f32")
    m2.mamba2_conv1d(u, dev32(inp["conv_w"]), dev32(inp["conv_b"]), csd, xbc)
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    y = empty((1, cfg.seqlen, di), "f32")
    hf = t.empty((1, cfg.nheads, 128, 64), dtype=t.float32, device="cuda")
    m2.mamba2_ssd_prefill(xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:], dev(inp["dt_raw"], "f32"),
                          dev32(inp["dt_bias"]), dev32(inp["A"]), dev32(inp["D"]), dev(inp["z"], "f32"),
                          None, hf, y, ngroups=cfg.ngroups, chunk=64)
    t.cuda.synchronize()
    xr, csr = oracle.conv1d(inp["xbc"], inp["conv_w"], inp["conv_b"], cs)
    x, Bm, Cm = oracle.split_xbc(xr, cfg.nheads, cfg.ngroups)
    yr, hr = oracle.ssd_scan(x, Bm, Cm, inp["dt_raw"], inp["dt_bias"], inp["A"], inp["D"], inp["z"],
                             None, ngroups=cfg.ngroups)
    assert_close(host(y), yr, "f32", "chained y")
    assert_close(host(hf), hr, "f32", "chained h", rounded=False)
    np.testing.assert_array_equal(host(csd), csr)


def test_prefill_then_decode_handoff():
    """prefill(L0) on device, then k decode steps carrying (conv_state, ssm_state), checked
    against the oracle fed the same values: its scan runs on the device's bf16 conv output
    for the prefill part and its decode steps run from the oracle's own prefill state."""
    t = torch()
    cfg = small(113, batch=2, seqlen=136, nheads=16, ngroups=8, h0_std=0.0)
    k = 8
    inp = si.draw_prefill(cfg)
    L0 = cfg.seqlen - k
    io, di, gn = cfg.io, cfg.d_inner, cfg.ngroups * cfg.dstate
    w, b = dev32(inp["conv_w"]), dev32(inp["conv_b"])
    dtb, A, D = dev32(inp["dt_bias"]), dev32(inp["A"]), dev32(inp["D"])
    u = dev(inp["xbc"][:, :L0], io)
    xbc = empty(u.shape, io)
    cs = t.zeros((cfg.batch, 3, cfg.conv_channels), dtype=u.dtype, device="cuda")
    m2.mamba2_conv1d(u, w, b, cs, xbc)
    y = empty((cfg.batch, L0, di), io)
    hs = t.empty((cfg.batch, cfg.nheads, 128, 64), dtype=t.float32, device="cuda")
    m2.mamba2_ssd_prefill(xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:],
                          dev(inp["dt_raw"][:, :L0], io), dtb, A, D, dev(inp["z"][:, :L0], io),
                          None, hs, y, ngroups=cfg.ngroups, chunk=cfg.chunk)
    ys = []
    for s in range(L0, cfg.seqlen):
        yt = empty((cfg.batch, di), io)
        m2.mamba2_state_update(dev(inp["xbc"][:, s], io), w, b, cs, dev(inp["dt_raw"][:, s], io), dtb, A,
                               D, dev(inp["z"][:, s], io), hs, yt, ngroups=cfg.ngroups)
        ys.append(host(yt))
    t.cuda.synchronize()

    x_dev = host(xbc)
    xo, Bo, Co = oracle.split_xbc(x_dev, cfg.nheads, cfg.ngroups)
    yr, hr = oracle.ssd_scan(xo, Bo, Co, inp["dt_raw"][:, :L0], inp["dt_bias"], inp["A"], inp["D"],
                             inp["z"][:, :L0], None, ngroups=cfg.ngroups)
    assert_close(host(y), yr, io, "prefill part")
    _, csr = oracle.conv1d(inp["xbc"][:, :L0], inp["conv_w"], inp["conv_b"], None)
    yts = []
    for s in range(L0, cfg.seqlen):
        ytr, csr, hr = oracle.state_update(inp["xbc"][:, s], inp["conv_w"], inp["conv_b"], csr,
                                           inp["dt_raw"][:, s], inp["dt_bias"], inp["A"], inp["D"],
                                           inp["z"][:, s], hr, nheads=cfg.nheads, ngroups=cfg.ngroups)
        yts.append(ytr)
    assert_close(np.stack(ys, 1), np.stack(yts, 1), io, "decode tail")
    assert_close(host(hs), hr, io, "state after decode", rounded=False)
    np.testing.assert_array_equal(host(cs), csr)
