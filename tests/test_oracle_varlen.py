"""Pins of the oracle's packed-batch prefill (oracle.conv_ssd_prefill_varlen), the serving
form of the layer core (an inference engine with an fp32 Mamba cache: neurohive,
section "Развертывание"). It is built from conv1d and ssd_scan, each pinned in
test_oracle_pins.py; these tests pin the packing and the cache handling against other
code paths:

- equal-length sequences packed with slots 0..S-1 equal the batch-dimension oracle call
  (conv1d / ssd_scan over [S][L]) started from the same states;
- a sequence split across two packed calls, handing its state and history through its
  pool entry, equals the whole sequence in one call;
- each sequence's outputs do not depend on the other sequences (bitwise);
- permuting the pool entries (and the pools with them) changes nothing;
- has_init = 0 equals zero pools; an entry out of range starts from zeros and leaves the
  pools untouched; an empty sequence keeps (or zeroes) its entry;
- io "bf16" stores the conv output as bf16 (round_bf16, pinned on exact tie cases) before
  the scan.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si

H, G, P, N = 4, 2, 64, 128


def cfg(cid=900):
    return si.Config(cid=cid, name=f"varlen{cid}", batch=1, seqlen=1, nheads=H, ngroups=G, chunk=64,
                     io="f32", h0_std=0.3)


def packed_inputs(c, total):
    """Seeded packed rows (one long stream cut into sequences) and parameters."""
    big = si.Config(cid=c.cid, name=c.name, batch=1, seqlen=max(total, 1), nheads=H, ngroups=G,
                    chunk=64, io="f32", h0_std=0.3)
    inp = si.draw_prefill(big)
    return {k: (v[0, :total] if k in ("xbc", "z", "dt_raw") else v) for k, v in inp.items()}


def run(inp, cu, slots, has_init, cpool, spool):
    return oracle.conv_ssd_prefill_varlen(inp["xbc"], cu, slots, has_init, cpool, spool, inp["conv_w"],
                                          inp["conv_b"], inp["dt_raw"], inp["dt_bias"], inp["A"], inp["D"],
                                          inp["z"], nheads=H, ngroups=G)


def test_equal_lengths_match_the_batched_oracle():
    c = cfg(901)
    S, L = 3, 37
    inp = packed_inputs(c, S * L)
    cpool, spool = si.draw_pools(c, S)
    cu = np.arange(S + 1) * L
    y, cp, sp = run(inp, cu, None, np.ones(S, np.int32), cpool, spool)
    xb = inp["xbc"].reshape(S, L, -1)
    xr, hist = oracle.conv1d(xb, inp["conv_w"], inp["conv_b"], cpool)
    x, Bm, Cm = oracle.split_xbc(xr, H, G)
    yr, hr = oracle.ssd_scan(x, Bm, Cm, inp["dt_raw"].reshape(S, L, H), inp["dt_bias"], inp["A"], inp["D"],
                             inp["z"].reshape(S, L, -1), spool, ngroups=G)
    np.testing.assert_allclose(y, yr.reshape(S * L, -1), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(cp, hist)
    np.testing.assert_allclose(sp, hr, rtol=1e-12, atol=1e-12)


def test_split_sequence_hands_off_through_the_pool():
    c = cfg(902)
    L1, L2 = 23, 41
    inp = packed_inputs(c, L1 + L2)
    cpool, spool = si.draw_pools(c, 2)
    slot = np.array([1], np.int32)
    whole = run(inp, [0, L1 + L2], slot, np.array([1], np.int32), cpool, spool)
    first = run({**inp, "xbc": inp["xbc"][:L1], "z": inp["z"][:L1], "dt_raw": inp["dt_raw"][:L1]},
                [0, L1], slot, np.array([1], np.int32), cpool, spool)
    second = run({**inp, "xbc": inp["xbc"][L1:], "z": inp["z"][L1:], "dt_raw": inp["dt_raw"][L1:]},
                 [0, L2], slot, np.array([1], np.int32), first[1], first[2])
    np.testing.assert_allclose(np.concatenate([first[0], second[0]]), whole[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(second[1], whole[1])
    np.testing.assert_allclose(second[2], whole[2], rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(whole[1][0], cpool[0])   # the other entry is untouched
    np.testing.assert_array_equal(whole[2][0], spool[0])


def test_sequences_are_independent():
    c = cfg(903)
    lens = [5, 17, 2, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    inp = packed_inputs(c, int(cu[-1]))
    cpool, spool = si.draw_pools(c, 6)
    slots = np.array([3, 0, 5, 1], np.int32)
    hi = np.array([1, 0, 1, 1], np.int32)
    y, cp, sp = run(inp, cu, slots, hi, cpool, spool)
    xb = inp["xbc"].copy()
    xb[cu[1]:cu[2]] += 1.0                              # perturb sequence 1 only
    y2, cp2, sp2 = run({**inp, "xbc": xb}, cu, slots, hi, cpool, spool)
    for i in (0, 2, 3):
        np.testing.assert_array_equal(y2[cu[i]:cu[i + 1]], y[cu[i]:cu[i + 1]])
        np.testing.assert_array_equal(sp2[slots[i]], sp[slots[i]])
        np.testing.assert_array_equal(cp2[slots[i]], cp[slots[i]])
    assert not np.array_equal(y2[cu[1]:cu[2]], y[cu[1]:cu[2]])


def test_slot_permutation_is_equivariant():
    c = cfg(904)
    lens = [9, 1, 14]
    cu = np.concatenate([[0], np.cumsum(lens)])
    inp = packed_inputs(c, int(cu[-1]))
    cpool, spool = si.draw_pools(c, 5)
    slots = np.array([4, 2, 0], np.int32)
    hi = np.array([1, 1, 0], np.int32)
    y, cp, sp = run(inp, cu, slots, hi, cpool, spool)
    perm = np.array([2, 4, 1, 0, 3])                    # entry e moves to perm[e]
    cpool2, spool2 = np.empty_like(cpool), np.empty_like(spool)
    cpool2[perm], spool2[perm] = cpool, spool
    y2, cp2, sp2 = run(inp, cu, perm[slots].astype(np.int32), hi, cpool2, spool2)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(cp2[perm], cp)
    np.testing.assert_array_equal(sp2[perm], sp)


def test_no_init_no_slot_and_empty_sequences():
    c = cfg(905)
    lens = [6, 0, 11]
    cu = np.concatenate([[0], np.cumsum(lens)])
    inp = packed_inputs(c, int(cu[-1]))
    cpool, spool = si.draw_pools(c, 3)
    zero_c, zero_s = np.zeros_like(cpool), np.zeros_like(spool)
    # has_init = 0 equals zero pools
    a = run(inp, cu, None, np.zeros(3, np.int32), cpool, spool)
    b = run(inp, cu, None, np.ones(3, np.int32), zero_c, zero_s)
    np.testing.assert_array_equal(a[0], b[0])
    # the empty sequence 1: with has_init it keeps its entry, without it the entry is zeroed
    keep = run(inp, cu, None, np.ones(3, np.int32), cpool, spool)
    np.testing.assert_array_equal(keep[1][1], cpool[1])
    np.testing.assert_array_equal(keep[2][1], spool[1])
    np.testing.assert_array_equal(a[1][1], zero_c[1])
    np.testing.assert_array_equal(a[2][1], zero_s[1])
    # an entry out of range: zeros in, nothing stored
    d = run(inp, cu, np.array([-1, 7, 2], np.int32), np.ones(3, np.int32), cpool, spool)
    np.testing.assert_array_equal(d[0][cu[0]:cu[1]], b[0][cu[0]:cu[1]])
    np.testing.assert_array_equal(d[1][:2], cpool[:2])
    np.testing.assert_array_equal(d[2][:2], spool[:2])


def test_round_bf16_ties_and_values():
    """Round-to-nearest-even at 8 significand bits: halfway cases go to the even neighbour,
    others to the nearest (1/3 = 1.0101010|1010...b x 2^-2 rounds up to 0.333984375)."""
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -2.5, 1 / 3, 0.0])
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -2.5, 0.333984375, 0.0])
    np.testing.assert_array_equal(oracle.round_bf16(v), want)


def test_bf16_io_rounds_the_conv_output():
    """io='bf16' equals the f32 oracle run on a hand-rounded conv output (one sequence)."""
    c = cfg(906)
    inp = packed_inputs(c, 20)
    y, _, _ = oracle.conv_ssd_prefill_varlen(inp["xbc"], [0, 20], None, None, None, None, inp["conv_w"],
                                             inp["conv_b"], inp["dt_raw"], inp["dt_bias"], inp["A"], inp["D"],
                                             inp["z"], nheads=H, ngroups=G, io="bf16")
    xr, _ = oracle.conv1d(inp["xbc"][None], inp["conv_w"], inp["conv_b"], None)
    x, Bm, Cm = oracle.split_xbc(oracle.round_bf16(xr), H, G)
    yr, _ = oracle.ssd_scan(x, Bm, Cm, inp["dt_raw"][None], inp["dt_bias"], inp["A"], inp["D"], inp["z"][None],
                            None, ngroups=G)
    np.testing.assert_array_equal(y, yr[0])


def test_lengths_recipe_sums_to_total():
    c = si.config(si.PREFILL_12B_8K)
    lens = si.draw_lengths(c, 16, 16, 2048, 8192)
    assert lens.sum() == 8192 and lens.min() >= 1
    s = si.draw_slots(c, 16, 40)
    assert len(set(s.tolist())) == 16 and s.min() >= 0 and s.max() < 40


if __name__ == "__main__":
    pytest.main([__file__, "-q"])
