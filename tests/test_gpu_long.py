"""Full-size parity of the long workloads: the 128k-token 12B prefill (chunk 256), one
GPU's 16384-token share of it with an incoming state and history (the per-GPU part of a
context-parallel split), and the 9B generation run (batch 8, 8192-token prefill, then 16384
decode steps carrying the conv and SSM states). Every call runs at its real shape on all heads; the oracle checks one head
per group (the recurrence is per head, so a head's outputs depend only on its own x, z, dt
and its group's B and C) on every token and every decode step.

Inputs are drawn and uploaded in slabs so that host memory stays a few GB above the
device copies.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_helpers import assert_close, empty, host, torch

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

m2 = pytest.importorskip("state_space_sequence_causal_amd")

SLAB = 16384


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(dst, a: np.ndarray):
    """Copy a host float32 array (exact in bf16) into the bf16 device tensor ``dst``."""
    t = torch()
    bits = si.bf16_bits(a).view(np.int16)
    dst.copy_(t.from_numpy(bits).view(t.bfloat16))


def dev32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def head_cols(heads, P=64):
    return np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])


def sub_channels(cfg, heads):
    """Conv/xBC channel indices of the sub-layer made of ``heads``: their x columns, then
    every group's B and C columns."""
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    return np.concatenate([head_cols(heads), np.arange(di, di + 2 * gn)])


def sub_params(p, heads, chans):
    return {"A": p["A"][heads], "dt_bias": p["dt_bias"][heads], "D": p["D"][heads],
            "conv_w": p["conv_w"][chans], "conv_b": p["conv_b"][chans]}


def one_head_per_group(cfg):
    """Head g * (H/G) + (7 g mod H/G) of each group g: one per group, at varied positions."""
    hpg = cfg.nheads // cfg.ngroups
    return [g * hpg + (7 * g) % hpg for g in range(cfg.ngroups)]


def test_prefill_12b_128k_chunk256():
    """12B shape, L = 131072, chunk 256, dt log-uniform: y on every token of one head per
    group and those heads' final states."""
    t = torch()
    cfg = si.PREFILL_12B_128K
    B, L, H, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    di, gn, Cc = cfg.d_inner, G * cfg.dstate, cfg.conv_channels
    heads = one_head_per_group(cfg)
    chans = sub_channels(cfg, heads)
    p = si.draw_params(cfg)
    xbc = empty((B, L, Cc), "bf16")
    z = empty((B, L, di), "bf16")
    dt = empty((B, L, H), "bf16")
    sub_x = np.empty((B, L, len(chans)))
    sub_z = np.empty((B, L, len(heads) * 64))
    sub_dt = np.empty((B, L, len(heads)))
    for t0 in range(0, L, SLAB):
        t1 = min(L, t0 + SLAB)
        a = si.draw_xbc(cfg, t0, t1)
        to_dev(xbc[:, t0:t1], a)
        sub_x[:, t0:t1] = a[..., chans]
        a = si.draw_z(cfg, t0, t1)
        to_dev(z[:, t0:t1], a)
        sub_z[:, t0:t1] = a[..., head_cols(heads)]
        a = si.draw_dt_raw(cfg, t0, t1, dt_bias=p["dt_bias"])
        to_dev(dt[:, t0:t1], a)
        sub_dt[:, t0:t1] = a[..., heads]
        del a
    y = empty((B, L, di), "bf16")
    hf = t.empty((B, H, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda")
    m2.mamba2_ssd_prefill(xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:], dt,
                          dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), z, None, hf, y,
                          ngroups=G, chunk=cfg.chunk)
    t.cuda.synchronize()
    cols = t.from_numpy(head_cols(heads)).cuda()
    yg = host(y.index_select(2, cols))
    hg = host(hf[:, heads])
    del xbc, z, y
    sp = sub_params(p, heads, chans)
    n = len(heads)
    yr, hr = oracle.ssd_scan(sub_x[..., :n * 64], sub_x[..., n * 64:n * 64 + gn],
                             sub_x[..., n * 64 + gn:], sub_dt, sp["dt_bias"], sp["A"], sp["D"],
                             sub_z, None, ngroups=G)
    ey = assert_close(yg, yr, "bf16", "128k y")
    eh = assert_close(hg, hr, "bf16", "128k h_final", rounded=False)
    print(f"128k prefill (heads {heads}): y err/rms {ey:.2e}, h_final err/rms {eh:.2e}")


def test_generation_9b_b8_prefill_then_16k_decode_steps():
    """9B shape, batch 8: conv1d + ssd_prefill over 8192 tokens, then 16384 state updates
    with fresh inputs each step. The oracle scans the device's conv output for the prefill
    (identical inputs per call), then runs the decode tokens as one conv + scan from its own
    prefill state and the raw conv history."""
    t = torch()
    cfg = si.GENERATE_9B_B8
    B, L, H, G, K = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, cfg.decode_steps
    di, gn, Cc = cfg.d_inner, G * cfg.dstate, cfg.conv_channels
    heads = one_head_per_group(cfg)
    chans = sub_channels(cfg, heads)
    n = len(heads)
    p = si.draw_params(cfg)
    w, b = dev32(p["conv_w"]), dev32(p["conv_b"])
    dtb, A, D = dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"])

    # ---- prefill
    inp = si.draw_prefill(cfg)
    u = empty((B, L, Cc), "bf16")
    to_dev(u, inp["xbc"])
    z = empty((B, L, di), "bf16")
    to_dev(z, inp["z"])
    dt = empty((B, L, H), "bf16")
    to_dev(dt, inp["dt_raw"])
    raw_tail = inp["xbc"][:, L - 3:].astype(np.float64)          # conv history after prefill
    sub_z = inp["z"][..., head_cols(heads)].astype(np.float64)
    sub_dt = inp["dt_raw"][..., heads].astype(np.float64)
    del inp
    xbc = empty((B, L, Cc), "bf16")
    cs = t.zeros((B, 3, Cc), dtype=t.bfloat16, device="cuda")
    m2.mamba2_conv1d(u, w, b, cs, xbc)
    y = empty((B, L, di), "bf16")
    state = t.empty((B, H, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda")
    m2.mamba2_ssd_prefill(xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:], dt, dtb, A, D, z,
                          None, state, y, ngroups=G, chunk=cfg.chunk)
    t.cuda.synchronize()
    cols = t.from_numpy(head_cols(heads)).cuda()
    y_pre = host(y.index_select(2, cols))
    h_pre = host(state[:, heads])
    cs_pre = host(cs)
    sub_xbc = host(xbc.index_select(2, t.from_numpy(chans).cuda()))
    del u, z, dt, xbc, y

    # ---- decode
    ud = empty((K, B, Cc), "bf16")
    zd = empty((K, B, di), "bf16")
    dtd = empty((K, B, H), "bf16")
    sub_u_dec = np.empty((B, K, len(chans)))
    sub_z_dec = np.empty((B, K, n * 64))
    sub_dt_dec = np.empty((B, K, n))
    for k0 in range(0, K, 2048):
        k1 = min(K, k0 + 2048)
        d = si.draw_decode_steps(cfg, k0, k1)
        to_dev(ud[k0:k1], d["xbc"])
        to_dev(zd[k0:k1], d["z"])
        to_dev(dtd[k0:k1], d["dt_raw"])
        sub_u_dec[:, k0:k1] = d["xbc"][..., chans].transpose(1, 0, 2)
        sub_z_dec[:, k0:k1] = d["z"][..., head_cols(heads)].transpose(1, 0, 2)
        sub_dt_dec[:, k0:k1] = d["dt_raw"][..., heads].transpose(1, 0, 2)
        del d
    last3 = host(ud[K - 3:]).transpose(1, 0, 2)
    yd = empty((K, B, di), "bf16")
    for k in range(K):
        m2.mamba2_state_update(ud[k], w, b, cs, dtd[k], dtb, A, D, zd[k], state, yd[k], ngroups=G)
    t.cuda.synchronize()
    y_dec = host(yd.index_select(2, cols)).transpose(1, 0, 2)
    h_end = host(state[:, heads])
    np.testing.assert_array_equal(host(cs), last3)
    del ud, zd, dtd, yd

    # ---- oracle
    np.testing.assert_array_equal(cs_pre, raw_tail)
    sp = sub_params(p, heads, chans)
    yr_pre, hr_pre = oracle.ssd_scan(sub_xbc[..., :n * 64], sub_xbc[..., n * 64:n * 64 + gn],
                                     sub_xbc[..., n * 64 + gn:], sub_dt, sp["dt_bias"], sp["A"],
                                     sp["D"], sub_z, None, ngroups=G)
    e1 = assert_close(y_pre, yr_pre, "bf16", "generation prefill y")
    e2 = assert_close(h_pre, hr_pre, "bf16", "generation prefill state", rounded=False)
    xr, csr = oracle.conv1d(sub_u_dec, sp["conv_w"], sp["conv_b"], raw_tail[..., chans])
    yr_dec, hr_end = oracle.ssd_scan(xr[..., :n * 64], xr[..., n * 64:n * 64 + gn], xr[..., n * 64 + gn:],
                                     sub_dt_dec, sp["dt_bias"], sp["A"], sp["D"], sub_z_dec, hr_pre,
                                     ngroups=G)
    e3 = assert_close(y_dec, yr_dec, "bf16", "generation decode y")
    e4 = assert_close(h_end, hr_end, "bf16", "generation final state", rounded=False)
    print(f"generation (heads {heads}): prefill y {e1:.2e} state {e2:.2e}; "
          f"{K} decode steps y {e3:.2e}, final state {e4:.2e}")


def test_context_parallel_share_12b_16k_with_h0():
    """One GPU's share of the 128k-token sequence split 8 ways: 16384 tokens of the 12B
    shape through the one-call prefill (chunk 64, the conv fused) starting from an incoming
    state h0 ~ N(0, 0.1^2) and a conv history, as the GPU after the first would run it once
    the exchange delivered them. y on every token of one head per group, those heads' final
    states against the oracle's scan from the same state, on the conv outputs the library
    computes (checked against the oracle's conv), and the new history bitwise."""
    t = torch()
    cfg = si.config(si.PREFILL_12B_128K, seqlen=16384, h0_std=0.1)
    B, L, H, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    di, gn, Cc = cfg.d_inner, G * cfg.dstate, cfg.conv_channels
    heads = one_head_per_group(cfg)
    chans = sub_channels(cfg, heads)
    p = si.draw_params(cfg)
    a = si.draw_xbc(cfg)
    xbc = empty((B, L, Cc), "bf16")
    to_dev(xbc, a)
    sub_x = a[..., chans].astype(np.float64)
    del a
    zz = si.draw_z(cfg)
    z = empty((B, L, di), "bf16")
    to_dev(z, zz)
    sub_z = zz[..., head_cols(heads)].astype(np.float64)
    del zz
    dd = si.draw_dt_raw(cfg, dt_bias=p["dt_bias"])
    dt = empty((B, L, H), "bf16")
    to_dev(dt, dd)
    sub_dt = dd[..., heads].astype(np.float64)
    h0 = si.draw_h0(cfg)
    cs0 = si.draw_conv_state(cfg)
    cs = empty((B, 3, Cc), "bf16")
    to_dev(cs, cs0)
    # the scan's inputs as the library computes them: the conv call on the same rows and
    # history (the one call is bitwise equal to it followed by the scan), so the oracle's scan
    # sees the exact bf16 conv outputs the kernels used
    cs_conv = empty((B, 3, Cc), "bf16")
    to_dev(cs_conv, cs0)
    xconv = empty((B, L, Cc), "bf16")
    m2.mamba2_conv1d(xbc, dev32(p["conv_w"]), dev32(p["conv_b"]), cs_conv, xconv)
    t.cuda.synchronize()
    conv = host(xconv.index_select(2, t.from_numpy(chans).cuda()))
    hist_conv = host(cs_conv)
    del xconv
    y = empty((B, L, di), "bf16")
    hf = t.empty((B, H, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda")
    print("context-parallel share: 12B, 16384 tokens, h0 and history", flush=True)
    m2.mamba2_conv_ssd_prefill(xbc, dev32(p["conv_w"]), dev32(p["conv_b"]), cs, dt, dev32(p["dt_bias"]),
                               dev32(p["A"]), dev32(p["D"]), z, dev32(h0), hf, y, ngroups=G, chunk=64)
    t.cuda.synchronize()
    cols = t.from_numpy(head_cols(heads)).cuda()
    yg = host(y.index_select(2, cols))
    hg = host(hf[:, heads])
    csg = host(cs)
    del xbc, z, y
    sp = sub_params(p, heads, chans)
    conv_r, hist = oracle.conv1d(sub_x, sp["conv_w"], sp["conv_b"], cs0[..., chans])
    assert_close(conv, conv_r, "bf16", "16k share conv")
    n = len(heads)
    yr, hr = oracle.ssd_scan(conv[..., :n * 64], conv[..., n * 64:n * 64 + gn], conv[..., n * 64 + gn:], sub_dt,
                             sp["dt_bias"], sp["A"], sp["D"], sub_z, h0[:, heads], ngroups=G)
    ey = assert_close(yg, yr, "bf16", "16k share y")
    eh = assert_close(hg, hr, "bf16", "16k share h_final", rounded=False)
    np.testing.assert_array_equal(csg[..., chans], hist)
    np.testing.assert_array_equal(csg, hist_conv)
    print(f"16k share (heads {heads}): y err/rms {ey:.2e}, h_final err/rms {eh:.2e}")


def test_fused_prefill_12b_128k_chunk64():
    """The call the benchmark times for the 128k-token workload: mamba2_conv_ssd_prefill at
    chunk 64 (the conv inside the scan's kernels) over the raw xBC of the 12B shape, from a
    zero conv history. Each step is checked on identical inputs: the conv call's output on the
    same rows (bitwise what the one call convolves, as test_gpu_conv_prefill shows) against the
    oracle's conv, then y on every token of one head per group and those heads' final states
    against the oracle's scan of that conv output; the new history bitwise."""
    t = torch()
    cfg = si.PREFILL_12B_128K
    B, L, H, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    di, gn, Cc = cfg.d_inner, G * cfg.dstate, cfg.conv_channels
    heads = one_head_per_group(cfg)
    chans = sub_channels(cfg, heads)
    p = si.draw_params(cfg)
    u = empty((B, L, Cc), "bf16")
    z = empty((B, L, di), "bf16")
    dt = empty((B, L, H), "bf16")
    sub_u = np.empty((B, L, len(chans)))
    sub_z = np.empty((B, L, len(heads) * 64))
    sub_dt = np.empty((B, L, len(heads)))
    for t0 in range(0, L, SLAB):
        t1 = min(L, t0 + SLAB)
        a = si.draw_xbc(cfg, t0, t1)
        to_dev(u[:, t0:t1], a)
        sub_u[:, t0:t1] = a[..., chans]
        a = si.draw_z(cfg, t0, t1)
        to_dev(z[:, t0:t1], a)
        sub_z[:, t0:t1] = a[..., head_cols(heads)]
        a = si.draw_dt_raw(cfg, t0, t1, dt_bias=p["dt_bias"])
        to_dev(dt[:, t0:t1], a)
        sub_dt[:, t0:t1] = a[..., heads]
        del a
    last3 = host(u[:, L - 3:])
    w, b = dev32(p["conv_w"]), dev32(p["conv_b"])
    xconv = empty((B, L, Cc), "bf16")
    m2.mamba2_conv1d(u, w, b, None, xconv)
    cs = t.zeros((B, 3, Cc), dtype=t.bfloat16, device="cuda")
    y = empty((B, L, di), "bf16")
    hf = t.empty((B, H, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda")
    print("fused prefill: 12B, 131072 tokens, chunk 64", flush=True)
    m2.mamba2_conv_ssd_prefill(u, w, b, cs, dt, dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), z, None, hf,
                               y, ngroups=G, chunk=64)
    t.cuda.synchronize()
    cols = t.from_numpy(head_cols(heads)).cuda()
    yg = host(y.index_select(2, cols))
    hg = host(hf[:, heads])
    conv = host(xconv.index_select(2, t.from_numpy(chans).cuda()))
    np.testing.assert_array_equal(host(cs), last3)
    del u, z, dt, y, xconv
    sp = sub_params(p, heads, chans)
    n = len(heads)
    xr, _ = oracle.conv1d(sub_u, sp["conv_w"], sp["conv_b"], None)
    del sub_u
    ec = assert_close(conv, xr, "bf16", "128k conv")
    del xr
    yr, hr = oracle.ssd_scan(conv[..., :n * 64], conv[..., n * 64:n * 64 + gn], conv[..., n * 64 + gn:], sub_dt,
                             sp["dt_bias"], sp["A"], sp["D"], sub_z, None, ngroups=G)
    ey = assert_close(yg, yr, "bf16", "128k fused y")
    eh = assert_close(hg, hr, "bf16", "128k fused h_final", rounded=False)
    print(f"128k fused chunk 64 (heads {heads}): conv {ec:.2e}, y err/rms {ey:.2e}, h_final err/rms {eh:.2e}")


def test_fused_prefill_9b_b8_8k_chunk64():
    """The prefill of the generation-shaped run as the benchmark times it: 9B shape, batch 8,
    8192 tokens, mamba2_conv_ssd_prefill at chunk 64 from a zero conv history. On identical
    inputs per step: the conv call's output against the oracle's conv, then y on every token
    of one head per group in all 8 sequences and those heads' final states against the
    oracle's scan of that conv output; the new history bitwise."""
    t = torch()
    cfg = si.GENERATE_9B_B8
    B, L, H, G = cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups
    di, gn, Cc = cfg.d_inner, G * cfg.dstate, cfg.conv_channels
    heads = one_head_per_group(cfg)
    chans = sub_channels(cfg, heads)
    n = len(heads)
    p = si.draw_params(cfg)
    inp = si.draw_prefill(cfg)
    u = empty((B, L, Cc), "bf16")
    to_dev(u, inp["xbc"])
    z = empty((B, L, di), "bf16")
    to_dev(z, inp["z"])
    dt = empty((B, L, H), "bf16")
    to_dev(dt, inp["dt_raw"])
    sub_u = inp["xbc"][..., chans].astype(np.float64)
    sub_z = inp["z"][..., head_cols(heads)].astype(np.float64)
    sub_dt = inp["dt_raw"][..., heads].astype(np.float64)
    last3 = inp["xbc"][:, L - 3:].astype(np.float64)
    del inp
    w, b = dev32(p["conv_w"]), dev32(p["conv_b"])
    xconv = empty((B, L, Cc), "bf16")
    m2.mamba2_conv1d(u, w, b, None, xconv)
    cs = t.zeros((B, 3, Cc), dtype=t.bfloat16, device="cuda")
    y = empty((B, L, di), "bf16")
    hf = t.empty((B, H, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda")
    print("fused prefill: 9B, batch 8, 8192 tokens, chunk 64", flush=True)
    m2.mamba2_conv_ssd_prefill(u, w, b, cs, dt, dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]), z, None, hf,
                               y, ngroups=G, chunk=64)
    t.cuda.synchronize()
    cols = t.from_numpy(head_cols(heads)).cuda()
    yg = host(y.index_select(2, cols))
    hg = host(hf[:, heads])
    conv = host(xconv.index_select(2, t.from_numpy(chans).cuda()))
    np.testing.assert_array_equal(host(cs), last3)
    del u, z, dt, y, xconv
    sp = sub_params(p, heads, chans)
    xr, _ = oracle.conv1d(sub_u, sp["conv_w"], sp["conv_b"], None)
    ec = assert_close(conv, xr, "bf16", "9B b8 conv")
    yr, hr = oracle.ssd_scan(conv[..., :n * 64], conv[..., n * 64:n * 64 + gn], conv[..., n * 64 + gn:], sub_dt,
                             sp["dt_bias"], sp["A"], sp["D"], sub_z, None, ngroups=G)
    ey = assert_close(yg, yr, "bf16", "9B b8 fused y")
    eh = assert_close(hg, hr, "bf16", "9B b8 fused h_final", rounded=False)
    print(f"9B batch 8 fused chunk 64 (heads {heads}): conv {ec:.2e}, y err/rms {ey:.2e}, "
          f"h_final err/rms {eh:.2e}")
