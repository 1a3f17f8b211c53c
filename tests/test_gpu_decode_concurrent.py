"""Small-batch decode calls in flight at the same time on two streams.

At the 9B shape with batch 8 (64 (sequence, group) pairs, fewer than the CU count / 2) the
one-token decode splits each pair's heads over 4 workgroups and shifts the shared B and C
conv-cache columns with a second kernel on the same stream. The call keeps no device state
of its own, so two such calls on different streams, on different caches, must give exactly
what they give one after the other. Each stream runs 24 steps on its own caches, launched
alternately; the results (every y, both caches) are compared bitwise with the same steps
run on one stream.
"""
import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import dev, dev32, host, torch

pytestmark = pytest.mark.gpu

m2 = pytest.importorskip("state_space_sequence_causal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")


STEPS = 24


def _set(cfg, seed_shift):
    c = si.config(cfg, cid=cfg.cid + seed_shift)
    p = si.draw_params(c)
    steps = si.draw_decode_steps(c, 0, STEPS)
    return dict(
        w=dev32(p["conv_w"]), b=dev32(p["conv_b"]), dtb=dev32(p["dt_bias"]), A=dev32(p["A"]), D=dev32(p["D"]),
        u=dev(steps["xbc"], "bf16"), z=dev(steps["z"], "bf16"), dt=dev(steps["dt_raw"], "bf16"),
        h0=si.draw_h0(si.config(c, h0_std=0.1)), cs0=si.draw_conv_state(c))


def _run(s, t, stream, state, cs, ys, k, G):
    with t.cuda.stream(stream):
        m2.mamba2_state_update(s["u"][k], s["w"], s["b"], cs, s["dt"][k], s["dtb"], s["A"], s["D"], s["z"][k],
                               state, ys[k], ngroups=G)


def test_two_small_batch_decodes_on_two_streams():
    t = torch()
    cfg = si.GENERATE_9B_B8
    B, H, G = cfg.batch, cfg.nheads, cfg.ngroups
    sets = [_set(cfg, 40), _set(cfg, 41)]

    def fresh(s):
        return dev32(s["h0"]), dev(s["cs0"], "bf16"), [t.empty((B, H * 64), dtype=t.bfloat16, device="cuda")
                                                      for _ in range(STEPS)]

    # serialized: all steps of set 0, then all of set 1, on the current stream
    ref = []
    main = t.cuda.current_stream()
    for s in sets:
        state, cs, ys = fresh(s)
        for k in range(STEPS):
            _run(s, t, main, state, cs, ys, k, G)
        t.cuda.synchronize()
        ref.append((host(state), host(cs), np.stack([host(v) for v in ys])))

    # concurrent: two streams at default priority, launches alternating
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    runs = [fresh(s) for s in sets]
    t.cuda.synchronize()
    print("two streams, 9B batch 8, 24 steps each", flush=True)
    for k in range(STEPS):
        for i in range(2):
            state, cs, ys = runs[i]
            _run(sets[i], t, streams[i], state, cs, ys, k, G)
    t.cuda.synchronize()
    for i in range(2):
        state, cs, ys = runs[i]
        np.testing.assert_array_equal(host(state), ref[i][0])
        np.testing.assert_array_equal(host(cs), ref[i][1])
        np.testing.assert_array_equal(np.stack([host(v) for v in ys]), ref[i][2])
