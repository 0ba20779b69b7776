"""Pins of the oracle's KDA-layer steps around the operator (Kimi Linear summary,
section 4: unit-length queries and keys; per-head RMSNorm of the output, then a
sigmoid output gate) against closed forms."""
import numpy as np

import oracle


def test_l2_normalize_pythagorean_rows():
    x = np.zeros((2, 128))
    x[0, 3], x[0, 70] = 3.0, 4.0      # norm 5
    x[1, :4] = [1.0, 2.0, 2.0, 4.0]   # norm 5
    y = oracle.l2_normalize(x, eps=0.0)
    assert y[0, 3] == 0.6 and y[0, 70] == 0.8
    np.testing.assert_array_equal(y[1, :4], [0.2, 0.4, 0.4, 0.8])
    assert np.count_nonzero(y) == 6


def test_l2_normalize_eps_and_scale():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 3, 128))
    y = oracle.l2_normalize(x, eps=0.0)
    np.testing.assert_allclose(np.sum(y * y, axis=-1), 1.0, rtol=1e-15)
    np.testing.assert_allclose(oracle.l2_normalize(1000.0 * x, eps=0.0), y, rtol=1e-14)
    # eps bounds the result of a zero row (0 / sqrt(eps) = 0), no NaN
    assert not np.isnan(oracle.l2_normalize(np.zeros(128), eps=1e-6)).any()
    # a row of 1e-4: sum of squares 1.28e-6, so eps = 1e-6 gives 1e-4 / sqrt(2.28e-6)
    np.testing.assert_allclose(oracle.l2_normalize(np.full(128, 1e-4), eps=1e-6), 1e-4 / np.sqrt(2.28e-6),
                               rtol=1e-14)


def test_gated_rmsnorm_constant_vector_and_gate_limits():
    o = np.full((1, 128), -2.0)
    w = np.linspace(0.5, 1.5, 128)
    big = np.full((1, 128), np.inf)
    # RMS of a constant vector is its magnitude: o / rms = -1 (eps = 0); a gate of +inf passes all
    np.testing.assert_array_equal(oracle.gated_rmsnorm(o, big, w, eps=0.0), -w[None, :])
    # a gate of 0 halves it; -inf closes it
    np.testing.assert_array_equal(oracle.gated_rmsnorm(o, np.zeros((1, 128)), w, eps=0.0), -0.5 * w[None, :])
    assert np.all(oracle.gated_rmsnorm(o, -big, w, eps=0.0) == 0.0)
    # sigmoid(ln 3) = 3/4
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, np.full((1, 128), np.log(3.0)), np.ones(128), eps=0.0),
                               -0.75, rtol=1e-15)


def test_gated_rmsnorm_is_per_row_and_scale_free():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((5, 4, 128))
    g = rng.standard_normal((5, 4, 128))
    w = rng.uniform(0.5, 1.5, 128)
    y = oracle.gated_rmsnorm(o, g, w, eps=0.0)
    np.testing.assert_allclose(oracle.gated_rmsnorm(37.0 * o, g, w, eps=0.0), y, rtol=1e-14)
    # rows are independent: changing one row leaves the others
    o2 = o.copy()
    o2[2, 1] *= -3.0
    y2 = oracle.gated_rmsnorm(o2, g, w, eps=0.0)
    mask = np.ones((5, 4), bool)
    mask[2, 1] = False
    np.testing.assert_array_equal(y2[mask], y[mask])
    # with unit weight and an open gate the RMS of every output row is 1
    y3 = oracle.gated_rmsnorm(o, np.full_like(g, np.inf), np.ones(128), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y3 * y3, axis=-1)), 1.0, rtol=1e-14)
