"""Parity of the multi-token decode: mamba2_state_update (and its slot form) with
T = dims->seqlen new tokens per sequence.

The call promises the bits of T one-token calls in order (test_gpu_parity.py ties the
one-token call to the oracle); each case runs both and compares y, the conv cache and the
state bitwise, for T = 2 .. 6 in bf16 and fp32, the 9B-shape batch of 64 at T = 4, one
group of 20 heads, shapes whose one-token calls take the split form with 1, 2 or 4 heads
per workgroup shared by all its waves, the slot form against gather / T-token call /
scatter, and once against the oracle (oracle.state_update_tokens).
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


def inputs(cid, B, T, H=16, G=8, io="bf16"):
    c = si.Config(cid=cid, name=f"dec-tokens{cid}", batch=B, seqlen=1, nheads=H, ngroups=G, chunk=64, io=io,
                  h0_std=0.1)
    p = si.draw_params(c)
    steps = si.draw_decode_steps(c, 0, T)            # [T][B][...]
    tok = {k: np.ascontiguousarray(v.transpose(1, 0, 2)) for k, v in steps.items()}   # [B][T][...]
    return c, p, tok, si.draw_conv_state(c), si.draw_h0(c)


def run_multi(c, p, tok, cs0, h0):
    t = torch()
    cs, hs = dev(cs0, c.io), dev32(h0)
    B, T = tok["xbc"].shape[:2]
    y = empty((B, T, c.d_inner), c.io)
    m2.mamba2_state_update(dev(tok["xbc"], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cs,
                           dev(tok["dt_raw"], c.io), dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]),
                           dev(tok["z"], c.io), hs, y, ngroups=c.ngroups)
    t.cuda.synchronize()
    return host(y), host(cs), host(hs)


def run_single(c, p, tok, cs0, h0):
    t = torch()
    cs, hs = dev(cs0, c.io), dev32(h0)
    B, T = tok["xbc"].shape[:2]
    ys = []
    for k in range(T):
        yk = empty((B, c.d_inner), c.io)
        m2.mamba2_state_update(dev(tok["xbc"][:, k], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cs,
                               dev(tok["dt_raw"][:, k], c.io), dev32(p["dt_bias"]), dev32(p["A"]),
                               dev32(p["D"]), dev(tok["z"][:, k], c.io), hs, yk, ngroups=c.ngroups)
        ys.append(host(yk))
    t.cuda.synchronize()
    return np.stack(ys, 1), host(cs), host(hs)


def check(cid, B, T, **kw):
    c, p, tok, cs0, h0 = inputs(cid, B, T, **kw)
    print(f"decode tokens: B{B} T{T} H{c.nheads} G{c.ngroups} {c.io}", flush=True)
    got = run_multi(c, p, tok, cs0, h0)
    ref = run_single(c, p, tok, cs0, h0)
    for name, g, r in zip(("y", "conv_state", "ssm_state"), got, ref):
        np.testing.assert_array_equal(g, r, err_msg=f"T={T} {name}")
    return c, p, tok, cs0, h0, got


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("T", [2, 3, 4, 5, 6])
def test_tokens_equal_one_token_calls(T, io):
    check(600 + T, 3, T, io=io)


def test_9b_batch64_four_tokens():
    check(610, 64, 4, H=128, G=8)


def test_one_group_twenty_heads():
    check(611, 2, 3, H=20, G=1)


@pytest.mark.parametrize("H, G", [(32, 8), (32, 4), (64, 4)])
def test_tokens_equal_staged_one_token_calls(H, G):
    """One-token calls at these small batches split each (sequence, group) over 4 workgroups
    whose 16 waves share 1, 2 or 4 heads and form y from LDS; the T-token call streams whole
    heads. Both must give the same bits."""
    check(620 + H // G, 2, 3, H=H, G=G)


def test_slots_three_tokens():
    """The slot form with 3 tokens equals gather -> 3-token call -> scatter."""
    t = torch()
    c, p, tok, _, _ = inputs(612, 4, 3)
    cpool, spool = si.draw_pools(c, 7)
    slots = np.array([5, -1, 0, 3], np.int32)
    cp, sp = dev(cpool, c.io), dev32(spool)
    y = empty((4, 3, c.d_inner), c.io)
    m2.mamba2_state_update_slots(dev(tok["xbc"], c.io), dev32(p["conv_w"]), dev32(p["conv_b"]), cp,
                                 dev(tok["dt_raw"], c.io), dev32(p["dt_bias"]), dev32(p["A"]), dev32(p["D"]),
                                 dev(tok["z"], c.io), sp, t.from_numpy(slots).cuda(), y, ngroups=c.ngroups)
    t.cuda.synchronize()
    own, ent = [0, 2, 3], [5, 0, 3]
    sub = {k: np.ascontiguousarray(v[own]) for k, v in tok.items()}
    yr, csr, hsr = run_multi(c, p, sub, cpool[ent], spool[ent])
    yg, cpg, spg = host(y), host(cp), host(sp)
    np.testing.assert_array_equal(yg[own], yr)
    assert np.all(yg[1] == 0)
    np.testing.assert_array_equal(cpg[ent], csr)
    np.testing.assert_array_equal(spg[ent], hsr)
    rest = [1, 2, 4, 6]
    np.testing.assert_array_equal(spg[rest], np.asarray(spool, np.float64)[rest])


def test_against_oracle():
    c, p, tok, cs0, h0, (y, cs, hs) = check(613, 2, 4)
    yr, csr, hr = oracle.state_update_tokens(tok["xbc"], p["conv_w"], p["conv_b"], cs0, tok["dt_raw"], p["dt_bias"],
                                             p["A"], p["D"], tok["z"], h0, nheads=c.nheads, ngroups=c.ngroups)
    assert_close(y, yr, c.io, "4-token y")
    assert_close(hs, hr, c.io, "4-token state", rounded=False)
    np.testing.assert_array_equal(cs, csr)
