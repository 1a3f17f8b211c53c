"""mamba2_conv_ssd_prefill_noalloc: the one-call prefill with the library's static device
scratch as its workspace, for callers that cannot allocate. Called through the C ABI, it
must give exactly what mamba2_conv_ssd_prefill gives with a caller workspace (the same
kernels on the same inputs): y, h_final and the new conv history bitwise, on two calls in a
row, the second smaller than the first (the scratch keeps the first call's contents), in
bf16 and in fp32.
"""
import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import dev, dev32, empty, host, torch

pytestmark = pytest.mark.gpu

m2 = pytest.importorskip("state_space_sequence_causal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")


def _case(cfg):
    t = torch()
    io = cfg.io
    inp = si.draw_prefill(cfg)
    cs0 = si.draw_conv_state(cfg)
    ops = dict(u=dev(inp["xbc"], io), w=dev32(inp["conv_w"]), b=dev32(inp["conv_b"]), dt=dev(inp["dt_raw"], io),
               dtb=dev32(inp["dt_bias"]), A=dev32(inp["A"]), D=dev32(inp["D"]), z=dev(inp["z"], io),
               h0=dev32(inp["h0"]))

    def outputs():
        return (dev(cs0, io), t.empty((cfg.batch, cfg.nheads, cfg.dstate, cfg.headdim), dtype=t.float32,
                                      device="cuda"), empty((cfg.batch, cfg.seqlen, cfg.d_inner), io))
    return ops, outputs


def _call(fn, o, cs, hf, y, cfg, **kw):
    fn(o["u"], o["w"], o["b"], cs, o["dt"], o["dtb"], o["A"], o["D"], o["z"], o["h0"], hf, y,
       ngroups=cfg.ngroups, chunk=cfg.chunk, **kw)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(io):
    t = torch()
    big = si.Config(cid=801, name="noalloc-big", batch=2, seqlen=1000, nheads=32, ngroups=8, chunk=64, io=io,
                    h0_std=0.3)
    small = si.Config(cid=802, name="noalloc-small", batch=1, seqlen=300, nheads=16, ngroups=4, chunk=128,
                      io=io, h0_std=0.3)
    for cfg in (big, small):
        print(f"noalloc {io}: batch {cfg.batch}, {cfg.seqlen} tokens, {cfg.nheads} heads", flush=True)
        o, outs = _case(cfg)
        cs_a, hf_a, y_a = outs()
        _call(m2.mamba2_conv_ssd_prefill_noalloc, o, cs_a, hf_a, y_a, cfg)
        cs_b, hf_b, y_b = outs()
        _call(m2.mamba2_conv_ssd_prefill, o, cs_b, hf_b, y_b, cfg)
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(y_a), host(y_b))
        np.testing.assert_array_equal(host(hf_a), host(hf_b))
        np.testing.assert_array_equal(host(cs_a), host(cs_b))
