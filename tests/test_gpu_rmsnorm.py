"""GPU parity of mamba2_group_rmsnorm (the block's RMSNorm of the gated output, taken over
the G contiguous channel groups) against the fp64 oracle, on the seeded stand-in for the
gated output: the full 12B-shape 8k prefill output, fp32 and bf16 io, in place, without a
weight, on strided views, on decode-shaped rows, and with one and with many groups."""
import dataclasses

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_helpers import assert_close, dev, dev32, empty, host, torch

pytestmark = pytest.mark.gpu

m2 = pytest.importorskip("state_space_sequence_causal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")


def small(cid, **kw):
    base = dict(cid=cid, name=f"norm{cid}", batch=2, seqlen=37, nheads=16, ngroups=8, chunk=64,
                io="bf16", h0_std=0.0)
    base.update(kw)
    return si.Config(**base)


def run(cfg, weight=True, inplace=False, eps=1e-5, pad=0):
    t = torch()
    g = si.draw_gated(cfg)
    w = si.draw_norm_weight(cfg) if weight else None
    W = cfg.d_inner
    if pad:
        wide = empty((cfg.batch, cfg.seqlen, W + pad), cfg.io)
        wide.zero_()
        gd = wide[..., :W]
        gd.copy_(dev(g, cfg.io))
    else:
        gd = dev(g, cfg.io)
    out = gd if inplace else empty((cfg.batch, cfg.seqlen, W), cfg.io)
    m2.mamba2_group_rmsnorm(gd, dev32(w) if weight else None, out, ngroups=cfg.ngroups, eps=eps)
    t.cuda.synchronize()
    ref = oracle.group_rmsnorm(g, w, ngroups=cfg.ngroups, eps=eps)
    return host(out), ref


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_rmsnorm_small(io):
    og, ref = run(small(201, io=io))
    assert_close(og, ref, io, f"rmsnorm {io}")


def test_rmsnorm_12b_8k_full():
    """All 8192 x 10240 outputs of the 12B-shape prefill, 8 groups of 1280 channels."""
    cfg = si.PREFILL_12B_8K
    og, ref = run(cfg)
    e = assert_close(og, ref, "bf16", "rmsnorm 12B")
    print(f"rmsnorm 12B: err/rms {e:.2e}")


def test_rmsnorm_in_place_no_weight_strided():
    og, ref = run(small(202), inplace=True)
    assert_close(og, ref, "bf16", "in place")
    og, ref = run(small(203), weight=False)
    assert_close(og, ref, "bf16", "no weight")
    og, ref = run(small(204), pad=64)
    assert_close(og, ref, "bf16", "strided")


@pytest.mark.parametrize("heads,groups", [(16, 1), (8, 8), (20, 4), (64, 1)])
def test_rmsnorm_group_widths(heads, groups):
    og, ref = run(small(205, nheads=heads, ngroups=groups, io="f32"))
    assert_close(og, ref, "f32", f"{heads} heads / {groups} groups")


def test_rmsnorm_decode_rows_and_determinism():
    t = torch()
    cfg = small(206, seqlen=1, batch=5)
    g = si.draw_gated(cfg)[:, 0]
    w = si.draw_norm_weight(cfg)
    gd = dev(g, "bf16")
    o1 = empty((cfg.batch, cfg.d_inner), "bf16")
    o2 = empty((cfg.batch, cfg.d_inner), "bf16")
    m2.mamba2_group_rmsnorm(gd, dev32(w), o1, ngroups=cfg.ngroups)
    m2.mamba2_group_rmsnorm(gd, dev32(w), o2, ngroups=cfg.ngroups)
    t.cuda.synchronize()
    assert_close(host(o1), oracle.group_rmsnorm(g, w, ngroups=cfg.ngroups), "bf16", "decode rows")
    np.testing.assert_array_equal(host(o1), host(o2))
