"""Parity of mamba2_state_update_slots: one decode token per request of a continuous
batch whose caches live in pools.

For tokens whose entry is in range the call promises the bits of mamba2_state_update on
that entry's caches (test_gpu_parity.py ties that call to the oracle). Each case gathers
the entries into batch caches, runs mamba2_state_update on the tokens that own one, and
scatters the caches back; the pools and y must match bitwise, tokens without an entry
must get y = 0, and entries no token owns must be untouched. Cases: a small batch with
shuffled entries and two tokens out of range, the 9B-shape batch-64 decode over a pool of
96, and one case against the oracle directly.
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


def case(cfg, slots, npool):
    B = len(slots)
    c = si.Config(cid=cfg.cid, name=cfg.name, batch=B, seqlen=1, nheads=cfg.nheads, ngroups=cfg.ngroups,
                  chunk=64, io=cfg.io, h0_std=0.1)
    p = si.draw_params(c)
    step = si.draw_decode_step(c, 0)
    cpool, spool = si.draw_pools(c, npool)
    return c, p, step, cpool, spool


def run_slots(c, p, step, cpool, spool, slots):
    t = torch()
    cp, sp = dev(cpool, c.io), dev32(spool)
    y = empty((len(slots), c.d_inner), c.io)
    y.fill_(3.0)
    m2.mamba2_state_update_slots(dev(step["xbc"][:, 0], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cp,
                                 dev(step["dt_raw"][:, 0], c.io), dev32(p["dt_bias"]), dev32(p["A"]),
                                 dev32(p["D"]), dev(step["z"][:, 0], c.io), sp,
                                 t.from_numpy(np.asarray(slots, np.int32)).cuda(), y, ngroups=c.ngroups)
    t.cuda.synchronize()
    return host(y), host(cp), host(sp)


def run_gathered(c, p, step, cpool, spool, slots):
    """mamba2_state_update on the tokens that own an entry, caches gathered and scattered."""
    t = torch()
    npool = spool.shape[0]
    own = [b for b, s in enumerate(slots) if 0 <= s < npool]
    y = np.zeros((len(slots), c.d_inner))
    cp, sp = np.asarray(cpool, np.float64).copy(), np.asarray(spool, np.float64).copy()
    if own:
        ent = [int(slots[b]) for b in own]
        cs = dev(cpool[ent], c.io)
        ss = dev32(spool[ent])
        yt = empty((len(own), c.d_inner), c.io)
        m2.mamba2_state_update(dev(step["xbc"][own, 0], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cs,
                               dev(step["dt_raw"][own, 0], c.io), dev32(p["dt_bias"]), dev32(p["A"]),
                               dev32(p["D"]), dev(step["z"][own, 0], c.io), ss, yt, ngroups=c.ngroups)
        t.cuda.synchronize()
        y[own] = host(yt)
        cp[ent], sp[ent] = host(cs), host(ss)
    return y, cp, sp


def check(cfg, slots, npool):
    c, p, step, cpool, spool = case(cfg, slots, npool)
    print(f"{cfg.name}: B{len(slots)} H{cfg.nheads} G{cfg.ngroups} {cfg.io} npool {npool} slots {list(slots)}",
          flush=True)
    got = run_slots(c, p, step, cpool, spool, slots)
    ref = run_gathered(c, p, step, cpool, spool, slots)
    for name, g, r in zip(("y", "conv_pool", "ssm_pool"), got, ref):
        np.testing.assert_array_equal(g, r, err_msg=f"{cfg.name} {name}")
    return c, p, step, cpool, spool, got


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_shuffled_entries_and_tokens_without_one(io):
    cfg = si.Config(cid=501, name="slots-small", batch=1, seqlen=1, nheads=16, ngroups=8, chunk=64, io=io)
    slots = si.draw_slots(cfg, 6, 10).copy()
    slots[2], slots[4] = -1, 12
    check(cfg, slots, 10)


def test_9b_batch64_pool96():
    cfg = si.Config(cid=502, name="slots-9b-b64", batch=1, seqlen=1, nheads=128, ngroups=8, chunk=64, io="bf16")
    check(cfg, si.draw_slots(cfg, 64, 96), 96)


def test_against_oracle():
    cfg = si.Config(cid=503, name="slots-oracle", batch=1, seqlen=1, nheads=16, ngroups=8, chunk=64, io="bf16")
    slots = np.array([3, 0, -1, 5], np.int32)
    c, p, step, cpool, spool = case(cfg, slots, 6)
    y, cp, sp = run_slots(c, p, step, cpool, spool, slots)
    own = [0, 1, 3]
    ent = [3, 0, 5]
    yr, csr, hr = oracle.state_update(step["xbc"][own, 0], p["conv_w"], p["conv_b"], cpool[ent],
                                      step["dt_raw"][own, 0], p["dt_bias"], p["A"], p["D"], step["z"][own, 0],
                                      spool[ent], nheads=c.nheads, ngroups=c.ngroups)
    assert_close(y[own], yr, "bf16", "slots y")
    assert np.all(y[2] == 0)
    assert_close(sp[ent], hr, "bf16", "slots state", rounded=False)
    np.testing.assert_array_equal(cp[ent], csr)
    untouched = [1, 2, 4]
    np.testing.assert_array_equal(sp[untouched], np.asarray(spool, np.float64)[untouched])
