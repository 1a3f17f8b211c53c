"""The seeded input generator: every slice of a workload is the same whichever way it is
drawn (whole, in token slabs, one decode step or many), so tests that draw in slabs or
batches see exactly the benchmark's inputs."""
import dataclasses

import numpy as np

import seeded_inputs as si


def small(**kw):
    return dataclasses.replace(si.GENERATE_9B_B8, batch=2, seqlen=700, **kw)


def test_token_slabs_equal_whole_draw():
    cfg = small()
    whole = si.draw_xbc(cfg)
    parts = [si.draw_xbc(cfg, a, b) for a, b in ((0, 1), (1, 300), (300, 513), (513, 700))]
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), whole)
    z = si.draw_z(cfg)
    np.testing.assert_array_equal(si.draw_z(cfg, 255, 257), z[:, 255:257])


def test_loguniform_dt_slabs_equal_whole_draw():
    cfg = small(dt_mode="loguniform")
    whole = si.draw_dt_raw(cfg)
    np.testing.assert_array_equal(si.draw_dt_raw(cfg, 100, 600), whole[:, 100:600])


def test_decode_steps_batched_equal_single():
    cfg = small()
    many = si.draw_decode_steps(cfg, 250, 262)
    for k in (250, 255, 256, 261):
        one = si.draw_decode_step(cfg, k)
        for name in ("xbc", "z", "dt_raw"):
            np.testing.assert_array_equal(many[name][k - 250], one[name][:, 0])


def test_decode_steps_differ_from_prefill_tokens():
    cfg = small()
    np.testing.assert_raises(AssertionError, np.testing.assert_array_equal,
                             si.draw_decode_step(cfg, 0)["xbc"], si.draw_xbc(cfg, 0, 1))


def test_bf16_inputs_are_exact_bf16():
    cfg = small()
    a = si.draw_xbc(cfg, 0, 64)
    np.testing.assert_array_equal(si.bf16_round(a), a)
