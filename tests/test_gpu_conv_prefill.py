"""Parity of mamba2_conv_ssd_prefill, the conv and the scan in one call.

For bf16 io at chunk 64 the conv runs inside the scan's kernels; the call promises
the results of mamba2_conv1d followed by mamba2_ssd_prefill bit for bit (the same conv
arithmetic, the same rounding of its output to bf16, the same scan). Those two calls
are checked against the fp64 oracle in test_gpu_parity.py; here the one call is
compared with them bitwise on the same inputs (y, h_final and the updated conv
history), over ragged and short lengths, with and without history, bias, D, z and h0,
on strided xBC, at the full 12B 8k size, and for the settings that run the two steps
through the workspace. One case is also checked against the oracle directly.
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


def small(cid, **kw):
    base = dict(cid=cid, name=f"conv_prefill{cid}", batch=2, seqlen=300, nheads=16, ngroups=8,
                chunk=64, io="bf16", h0_std=0.5)
    base.update(kw)
    return si.Config(**base)


def _operands(cfg, inp, cs_np, z, D, h0, bias, pad):
    """Device operands; with pad > 0 the raw xBC is a column view of a wider tensor."""
    t = torch()
    io = cfg.io
    u = dev(inp["xbc"], io)
    if pad:
        wide = empty(u.shape[:-1] + (u.shape[-1] + 2 * pad,), io)
        wide.fill_(7.0)
        wide[..., pad:pad + u.shape[-1]] = u
        u = wide[..., pad:pad + u.shape[-1]]
    return dict(
        u=u, w=dev32(inp["conv_w"]), b=dev32(inp["conv_b"]) if bias else None,
        cs=dev(cs_np, io) if cs_np is not None else None,
        dt=dev(inp["dt_raw"], io), dtb=dev32(inp["dt_bias"]), A=dev32(inp["A"]),
        D=dev32(inp["D"]) if D else None, z=dev(inp["z"], io) if z else None,
        h0=dev32(inp["h0"]) if h0 else None,
        hf=t.empty((cfg.batch, cfg.nheads, cfg.dstate, cfg.headdim), dtype=t.float32, device="cuda"),
        y=empty((cfg.batch, cfg.seqlen, cfg.d_inner), io))


def run_fused(cfg, inp, cs_np, *, chunk=None, z=True, D=True, h0=True, bias=True, pad=0):
    o = _operands(cfg, inp, cs_np, z, D, h0, bias, pad)
    m2.mamba2_conv_ssd_prefill(o["u"], o["w"], o["b"], o["cs"], o["dt"], o["dtb"], o["A"], o["D"],
                               o["z"], o["h0"], o["hf"], o["y"], ngroups=cfg.ngroups,
                               chunk=chunk or cfg.chunk)
    torch().cuda.synchronize()
    return host(o["y"]), host(o["hf"]), None if o["cs"] is None else host(o["cs"])


def run_two_calls(cfg, inp, cs_np, *, chunk=None, z=True, D=True, h0=True, bias=True, pad=0):
    o = _operands(cfg, inp, cs_np, z, D, h0, bias, pad)
    di, gn = cfg.d_inner, cfg.ngroups * cfg.dstate
    xbc = empty((cfg.batch, cfg.seqlen, cfg.conv_channels), cfg.io)
    if cfg.seqlen:
        m2.mamba2_conv1d(o["u"], o["w"], o["b"], o["cs"], xbc)
    m2.mamba2_ssd_prefill(xbc[..., :di], xbc[..., di:di + gn], xbc[..., di + gn:], o["dt"], o["dtb"],
                          o["A"], o["D"], o["z"], o["h0"], o["hf"], o["y"], ngroups=cfg.ngroups,
                          chunk=chunk or cfg.chunk)
    torch().cuda.synchronize()
    return host(o["y"]), host(o["hf"]), None if o["cs"] is None else host(o["cs"])


def check_bitwise(cfg, hist=True, **kw):
    inp = si.draw_prefill(cfg)
    cs = si.draw_conv_state(cfg) if hist else None
    print(f"{cfg.name}: B{cfg.batch} L{cfg.seqlen} H{cfg.nheads} G{cfg.ngroups} chunk "
          f"{kw.get('chunk', cfg.chunk)} {cfg.io} hist={hist} {kw}", flush=True)
    got = run_fused(cfg, inp, cs, **kw)
    ref = run_two_calls(cfg, inp, cs, **kw)
    for name, g, r in zip(("y", "h_final", "conv_state"), got, ref):
        if r is None:
            assert g is None
            continue
        np.testing.assert_array_equal(g, r, err_msg=f"{cfg.name} {name}")
    return got


@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 63, 64, 65, 67, 130, 300])
@pytest.mark.parametrize("hist", [True, False])
def test_fused_equals_two_calls(L, hist):
    check_bitwise(small(301, seqlen=L), hist=hist)


@pytest.mark.parametrize("opts", [dict(z=False), dict(D=False), dict(h0=False), dict(bias=False),
                                  dict(pad=32), dict(z=False, D=False, h0=False, bias=False)])
def test_fused_optional_operands_and_strided_xbc(opts):
    check_bitwise(small(302, seqlen=200), **opts)


def test_fused_one_group_many_heads():
    check_bitwise(small(303, batch=1, seqlen=150, nheads=20, ngroups=1))


def test_fused_two_groups_batch3():
    check_bitwise(small(304, batch=3, seqlen=97, nheads=8, ngroups=2))


@pytest.mark.parametrize("io,chunk", [("bf16", 128), ("bf16", 256), ("f32", 64)])
def test_two_step_settings_through_workspace(io, chunk):
    check_bitwise(small(305, seqlen=270, io=io, chunk=chunk))


def test_fused_12b_8k_full_size():
    """The 12B 8k prefill workload, all heads, with a conv history."""
    check_bitwise(si.PREFILL_12B_8K, chunk=64)


def test_fused_against_oracle():
    """The one call against the oracle's conv -> scan, on the exact inputs."""
    cfg = small(306, seqlen=200)
    inp = si.draw_prefill(cfg)
    cs = si.draw_conv_state(cfg)
    y, hf, csg = run_fused(cfg, inp, cs)
    xr, csr = oracle.conv1d(inp["xbc"], inp["conv_w"], inp["conv_b"], cs)
    # the kernels round the conv output to bf16 before the scan, as the two-call path does
    xr = si.bf16_round(xr)
    x, Bm, Cm = oracle.split_xbc(xr, cfg.nheads, cfg.ngroups)
    yr, hr = oracle.ssd_scan(x, Bm, Cm, inp["dt_raw"], inp["dt_bias"], inp["A"], inp["D"], inp["z"],
                             inp["h0"], ngroups=cfg.ngroups)
    assert_close(y, yr, cfg.io, "fused y")
    assert_close(hf, hr, cfg.io, "fused h_final", rounded=False)
    np.testing.assert_array_equal(csg, csr)


def test_fused_len0_keeps_history_and_state():
    t = torch()
    cfg = small(307, seqlen=0)
    cs = si.draw_conv_state(cfg)
    csd = dev(cs, cfg.io)
    h0 = dev32(si.draw_prefill(small(307, seqlen=1))["h0"])
    hf = t.empty_like(h0)
    u = empty((cfg.batch, 0, cfg.conv_channels), cfg.io)
    dt = empty((cfg.batch, 0, cfg.nheads), cfg.io)
    y = empty((cfg.batch, 0, cfg.d_inner), cfg.io)
    p = si.draw_prefill(small(307, seqlen=1))
    m2.mamba2_conv_ssd_prefill(u, dev32(p["conv_w"]), dev32(p["conv_b"]), csd, dt, dev32(p["dt_bias"]),
                               dev32(p["A"]), dev32(p["D"]), None, h0, hf, y, ngroups=cfg.ngroups, chunk=64)
    t.cuda.synchronize()
    np.testing.assert_array_equal(host(csd), np.asarray(cs, np.float64))
    np.testing.assert_array_equal(host(hf), host(h0))


def test_fused_is_deterministic():
    cfg = small(308, seqlen=500)
    inp = si.draw_prefill(cfg)
    cs = si.draw_conv_state(cfg)
    a = run_fused(cfg, inp, cs)
    b = run_fused(cfg, inp, cs)
    for g, r in zip(a, b):
        np.testing.assert_array_equal(g, r)


def test_profile_call_bitwise_and_cycles():
    """mamba2_conv_ssd_prefill_profile gives the one call's results bit for bit and fills the
    cycle profile: every wave's chunk-loop count is positive, and each phase of a Y or H wave
    is a positive part of its loop."""
    t = torch()
    cfg = small(560, seqlen=700)
    inp = si.draw_prefill(cfg)
    cs0 = si.draw_conv_state(cfg)
    y0, h0_, c0 = run_fused(cfg, inp, cs0)
    o = _operands(cfg, inp, cs0, True, True, True, True, 0)
    d = m2.make_dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, 64, m2.MAMBA2_BF16)
    ws = t.empty(m2.mamba2_conv_ssd_prefill_workspace_bytes(d), dtype=t.uint8, device="cuda")
    cyc = t.zeros(cfg.batch * cfg.nheads * 128, dtype=t.int64, device="cuda")
    m2.mamba2_conv_ssd_prefill_profile(o["u"], o["w"], o["b"], o["cs"], o["dt"], o["dtb"], o["A"], o["D"], o["z"],
                                       o["h0"], o["hf"], o["y"], cyc, ngroups=cfg.ngroups, chunk=64, workspace=ws)
    t.cuda.synchronize()
    np.testing.assert_array_equal(host(o["y"]), y0)
    np.testing.assert_array_equal(host(o["hf"]), h0_)
    np.testing.assert_array_equal(host(o["cs"]), c0)
    c = cyc.view(cfg.batch * cfg.nheads, 16, 8).cpu().numpy()
    assert (c[:, :, 0] > 0).all()
    assert (c[:, :, 1] > 0).all() and (c[:, :, 1] < c[:, :, 0]).all()
    assert (c[:, 0:4, 2] > 0).all() and (c[:, 0:4, 2] < c[:, 0:4, 0]).all()
    assert (c[:, 8:16, 2] > 0).all() and (c[:, 8:16, 2] < c[:, 8:16, 0]).all()
    assert (c[:, :, 4] < c[:, :, 0]).all() and (c[:, :, 5:] == 0).all()
