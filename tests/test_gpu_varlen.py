"""Parity of mamba2_conv_ssd_prefill_varlen: packed sequences of different lengths with
their states in slot pools (continuous batching).

The call promises, per sequence, the bits of mamba2_conv_ssd_prefill on that sequence
alone (batch 1) started from the same state and history (test_gpu_conv_prefill.py ties
that call to the two-call path and the oracle). Here each packed sequence is compared
bitwise with such a call: its y rows, and the final state and conv history left in its
pool entry; entries no sequence owns must be untouched. Cases: ragged and empty
sequences with mixed has_init flags and shuffled entries, default slots and flags,
entries out of range, no pools at all, invalid offsets (clamped: results equal those of
the clamped offsets), a 16-sequence 12B-shape mix of 8192 tokens, and one case against the
oracle directly.
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


def small(cid, H=16, G=8):
    return si.Config(cid=cid, name=f"varlen{cid}", batch=1, seqlen=1, nheads=H, ngroups=G, chunk=64,
                     io="bf16", h0_std=0.5)


def packed(cfg, total):
    big = si.Config(cid=cfg.cid, name=cfg.name, batch=1, seqlen=max(total, 1), nheads=cfg.nheads,
                    ngroups=cfg.ngroups, chunk=64, io="bf16", h0_std=0.5)
    inp = si.draw_prefill(big)
    return {k: (v[0, :total] if k in ("xbc", "z", "dt_raw") else v) for k, v in inp.items()}


def i32(a):
    t = torch()
    return None if a is None else t.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def run_varlen(cfg, inp, cu, slots, has_init, cpool, spool):
    t = torch()
    T = int(inp["xbc"].shape[0])
    cp = dev(cpool, "bf16") if cpool is not None else None
    sp = dev32(spool) if spool is not None else None
    y = empty((T, cfg.d_inner), "bf16")
    y.fill_(0)
    m2.mamba2_conv_ssd_prefill_varlen(
        dev(inp["xbc"], "bf16"), dev32(inp["conv_w"]), dev32(inp["conv_b"]), i32(cu), i32(slots),
        i32(has_init), cp, sp, dev(inp["dt_raw"], "bf16"), dev32(inp["dt_bias"]), dev32(inp["A"]),
        dev32(inp["D"]), dev(inp["z"], "bf16"), y, ngroups=cfg.ngroups)
    t.cuda.synchronize()
    return host(y), None if cp is None else host(cp), None if sp is None else host(sp)


def run_each(cfg, inp, cu, slots, has_init, cpool, spool):
    """The reference: one batch-1 mamba2_conv_ssd_prefill per sequence, from the same entry."""
    t = torch()
    T = int(inp["xbc"].shape[0])
    S = len(cu) - 1
    npool = 0 if spool is None else spool.shape[0]
    y = np.zeros((T, cfg.d_inner))
    cp = None if cpool is None else np.asarray(cpool, np.float64).copy()
    sp = None if spool is None else np.asarray(spool, np.float64).copy()
    w, b = dev32(inp["conv_w"]), dev32(inp["conv_b"])
    dtb, A, D = dev32(inp["dt_bias"]), dev32(inp["A"]), dev32(inp["D"])
    for i in range(S):
        a, e = int(cu[i]), int(cu[i + 1])
        s = i if slots is None else int(slots[i])
        has_slot = 0 <= s < npool
        init = has_slot and has_init is not None and int(has_init[i]) != 0
        cs = dev(cpool[s][None], "bf16") if init else t.zeros((1, 3, cfg.conv_channels), dtype=t.bfloat16,
                                                            device="cuda")
        h0 = dev32(spool[s][None]) if init else None
        hf = t.empty((1, cfg.nheads, 128, 64), dtype=t.float32, device="cuda")
        yi = empty((1, e - a, cfg.d_inner), "bf16")
        m2.mamba2_conv_ssd_prefill(dev(inp["xbc"][None, a:e], "bf16"), w, b, cs, dev(inp["dt_raw"][None, a:e], "bf16"),
                                   dtb, A, D, dev(inp["z"][None, a:e], "bf16"), h0, hf, yi,
                                   ngroups=cfg.ngroups, chunk=64)
        t.cuda.synchronize()
        y[a:e] = host(yi)[0]
        if has_slot:
            cp[s] = host(cs)[0]
            sp[s] = host(hf)[0]
    return y, cp, sp


def check(cfg, lens, slots, has_init, npool, cu=None):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32) if cu is None else np.asarray(cu, np.int32)
    inp = packed(cfg, int(cu[-1]))
    pools = si.draw_pools(cfg, npool) if npool else (None, None)
    print(f"{cfg.name}: H{cfg.nheads} G{cfg.ngroups} lens {list(np.diff(cu))} slots "
          f"{None if slots is None else list(slots)} init {None if has_init is None else list(has_init)} "
          f"npool {npool}", flush=True)
    got = run_varlen(cfg, inp, cu, slots, has_init, *pools)
    ref = run_each(cfg, inp, cu, slots, has_init, *pools)
    for name, g, r in zip(("y", "conv_pool", "ssm_pool"), got, ref):
        if r is None:
            assert g is None
            continue
        np.testing.assert_array_equal(g, r, err_msg=f"{cfg.name} {name}")
    return inp, cu, pools, got


def test_ragged_mixed_init_shuffled_slots():
    cfg = small(401)
    lens = [1, 2, 3, 0, 64, 65, 130, 7, 300]
    check(cfg, lens, si.draw_slots(cfg, len(lens), 14), si.draw_has_init(cfg, len(lens)), 14)


def test_default_slots_and_flags():
    cfg = small(402)
    check(cfg, [70, 5, 128], None, None, 3)


def test_entries_out_of_range_and_all_continuing():
    cfg = small(403)
    check(cfg, [40, 3, 97, 64], np.array([-1, 2, 9, 0], np.int32), np.ones(4, np.int32), 4)


def test_no_pools():
    cfg = small(404)
    check(cfg, [33, 0, 80], None, None, 0)


def test_one_group_twenty_heads():
    cfg = small(405, H=20, G=1)
    check(cfg, [150, 1, 66], np.array([1, 0, 2], np.int32), np.array([1, 0, 1], np.int32), 3)


def test_invalid_offsets_are_clamped():
    """Decreasing, negative and too-large offsets: the call equals the same call with the
    offsets clamped into order (cu'[i] = min(max(0, cu[0..i]), total)), and faults nothing."""
    cfg = small(406)
    total = 200
    bad = np.array([0, 50, 30, -7, 120, 999, 150], np.int32)
    clamped = np.minimum(np.maximum.accumulate(np.maximum(bad, 0)), total).astype(np.int32)
    inp = packed(cfg, total)
    pools = si.draw_pools(cfg, 6)
    slots = np.arange(6, dtype=np.int32)
    hi = np.array([1, 0, 1, 1, 0, 1], np.int32)
    a = run_varlen(cfg, inp, bad, slots, hi, *pools)
    b = run_varlen(cfg, inp, clamped, slots, hi, *pools)
    for g, r in zip(a, b):
        np.testing.assert_array_equal(g, r)


def test_serving_mix_12b_shape():
    """16 sequences of log-uniform lengths summing to 8192 tokens at the 12B shape (160 heads,
    8 groups), half continuing from their entries, in a pool of 40."""
    cfg = si.Config(cid=407, name="varlen-12b-mix", batch=1, seqlen=1, nheads=160, ngroups=8, chunk=64,
                    io="bf16", h0_std=0.1)
    lens = si.draw_lengths(cfg, 16, 16, 2048, 8192)
    check(cfg, lens, si.draw_slots(cfg, 16, 40), si.draw_has_init(cfg, 16), 40)


def test_against_oracle():
    cfg = small(408)
    lens = [90, 0, 1, 64, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.array([2, 5, 0, 4, 1], np.int32)
    hi = np.array([1, 1, 0, 1, 0], np.int32)
    inp = packed(cfg, int(cu[-1]))
    cpool, spool = si.draw_pools(cfg, 6)
    y, cp, sp = run_varlen(cfg, inp, cu, slots, hi, cpool, spool)
    yr, cpr, spr = oracle.conv_ssd_prefill_varlen(inp["xbc"], cu, slots, hi, cpool, spool, inp["conv_w"],
                                                  inp["conv_b"], inp["dt_raw"], inp["dt_bias"], inp["A"],
                                                  inp["D"], inp["z"], nheads=cfg.nheads, ngroups=cfg.ngroups,
                                                  io="bf16")
    assert_close(y, yr, "bf16", "varlen y")
    assert_close(sp, spr, "bf16", "varlen states", rounded=False)
    np.testing.assert_array_equal(cp, cpr)


def test_deterministic():
    cfg = small(409)
    lens = [200, 17, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp = packed(cfg, int(cu[-1]))
    pools = si.draw_pools(cfg, 3)
    a = run_varlen(cfg, inp, cu, None, np.ones(3, np.int32), *pools)
    b = run_varlen(cfg, inp, cu, None, np.ones(3, np.int32), *pools)
    for g, r in zip(a, b):
        np.testing.assert_array_equal(g, r)
