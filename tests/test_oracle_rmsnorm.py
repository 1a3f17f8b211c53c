"""Pins of the oracle's group RMSNorm of the gated output (the block's RMSNorm, hyper.ai
summary of the Nemotron-Nano-2 report, section "方法", taken after the SiLU(z) gate):

    out[k] = g[k] / sqrt(mean over k's group of g^2 + eps) * weight[k],

each row cut into ngroups contiguous groups. Every pin below comes from outside the
oracle: hand-computed values, a closed form, numpy's vector norm, or an invariance of the
definition. Each test names the mistake it is there to catch.
"""
import numpy as np
import pytest

import oracle


def test_hand_example():
    """A wrong mean (sum instead of mean) or a missing square root changes these values."""
    g = np.array([[3.0, 4.0, 0.0, 1e-3]])
    out = oracle.group_rmsnorm(g, ngroups=2, eps=0.0)
    r0 = np.sqrt((9.0 + 16.0) / 2.0)      # group [3, 4]
    r1 = np.sqrt((1e-6) / 2.0)            # group [0, 1e-3]
    np.testing.assert_allclose(out, [[3.0 / r0, 4.0 / r0, 0.0, 1e-3 / r1]], rtol=1e-15)


def test_constant_group_closed_form():
    """A group of equal values c maps to c / sqrt(c^2 + eps) * w: catches eps misplaced
    (outside the square root, or added to the sum instead of the mean)."""
    c, eps, gs = -0.37, 1e-2, 16
    g = np.full((3, 2 * gs), c)
    w = np.linspace(0.5, 2.0, 2 * gs)
    out = oracle.group_rmsnorm(g, w, ngroups=2, eps=eps)
    np.testing.assert_allclose(out, np.broadcast_to(c / np.sqrt(c * c + eps) * w, g.shape), rtol=1e-14)


def test_one_group_is_scaled_unit_vector():
    """ngroups = 1, eps = 0: out = g * sqrt(width) / ||g||_2 * weight (numpy's norm)."""
    r = np.random.default_rng(7)
    g = r.standard_normal((5, 96))
    w = r.uniform(0.5, 1.5, 96)
    out = oracle.group_rmsnorm(g, w, ngroups=1, eps=0.0)
    ref = g * np.sqrt(96) / np.linalg.norm(g, axis=1, keepdims=True) * w
    np.testing.assert_allclose(out, ref, rtol=1e-13)


def test_groups_are_independent_and_contiguous():
    """Perturbing group 1 leaves groups 0 and 2 bitwise unchanged (catches strided groups
    or a norm over the whole row), and each group equals the one-group norm of its slice."""
    r = np.random.default_rng(8)
    g = r.standard_normal((4, 3 * 40))
    w = r.uniform(0.5, 1.5, 120)
    a = oracle.group_rmsnorm(g, w, ngroups=3)
    g2 = g.copy()
    g2[:, 40:80] *= 3.0
    g2[:, 50] += 1.0
    b = oracle.group_rmsnorm(g2, w, ngroups=3)
    np.testing.assert_array_equal(a[:, :40], b[:, :40])
    np.testing.assert_array_equal(a[:, 80:], b[:, 80:])
    for q in range(3):
        sl = slice(40 * q, 40 * (q + 1))
        np.testing.assert_allclose(a[:, sl], oracle.group_rmsnorm(g[:, sl], w[sl], ngroups=1), rtol=1e-15)


def test_scale_invariance_without_eps():
    """eps = 0: out(alpha g) = out(g) for alpha > 0 (catches a missing normalisation)."""
    r = np.random.default_rng(9)
    g = r.standard_normal((3, 64))
    np.testing.assert_allclose(oracle.group_rmsnorm(7.5 * g, ngroups=4, eps=0.0),
                               oracle.group_rmsnorm(g, ngroups=4, eps=0.0), rtol=1e-14)


def test_no_weight_means_ones():
    r = np.random.default_rng(10)
    g = r.standard_normal((2, 32))
    np.testing.assert_array_equal(oracle.group_rmsnorm(g, None, ngroups=2),
                                  oracle.group_rmsnorm(g, np.ones(32), ngroups=2))


def test_width_must_divide():
    with pytest.raises(ValueError):
        oracle.group_rmsnorm(np.ones((1, 10)), ngroups=3)
