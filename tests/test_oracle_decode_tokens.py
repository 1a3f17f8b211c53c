"""Pin of the oracle's multi-token decode (oracle.state_update_tokens, the one-token step
of test_oracle_pins.py applied token after token): T tokens decoded from a conv history
and a state equal the prefill of the same T tokens (oracle conv1d over the tokens with
that history, then ssd_scan from that state): outputs, final state and new history. The
two paths share no code beyond the C conv and recurrence primitives, which are pinned on
their own."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si


@pytest.mark.parametrize("T", [1, 2, 5])
def test_tokens_equal_prefill_of_the_same_tokens(T):
    cfg = si.Config(cid=950 + T, name="dec-tokens", batch=2, seqlen=T, nheads=4, ngroups=2, chunk=64,
                    io="f32", h0_std=0.3)
    inp = si.draw_prefill(cfg)
    hist = si.draw_conv_state(cfg)
    y, cs, ss = oracle.state_update_tokens(inp["xbc"], inp["conv_w"], inp["conv_b"], hist, inp["dt_raw"],
                                           inp["dt_bias"], inp["A"], inp["D"], inp["z"], inp["h0"],
                                           nheads=4, ngroups=2)
    xr, hr = oracle.conv1d(inp["xbc"], inp["conv_w"], inp["conv_b"], hist)
    x, Bm, Cm = oracle.split_xbc(xr, 4, 2)
    yr, sr = oracle.ssd_scan(x, Bm, Cm, inp["dt_raw"], inp["dt_bias"], inp["A"], inp["D"], inp["z"], inp["h0"],
                             ngroups=2)
    np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ss, sr, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(cs, hr)
