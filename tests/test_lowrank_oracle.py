"""Pins of oracle.lowrank_z, the forget gate's pre-activation from its low-rank
projection (Kimi Linear summary, section 4), against cases whose result is known
without the contraction itself."""
import numpy as np

import oracle


def test_one_hot_rows_select_weight_columns():
    """u[t] = e_{j(t)} gives z[t, h, c] = W[h, c, j(t)] exactly: catches a contraction over the
    wrong axis of W and a transposed (c, j) layout."""
    rng = np.random.default_rng(7)
    H, r, T = 3, 32, 40
    W = rng.standard_normal((H, 128, r))
    js = rng.integers(0, r, size=T)
    u = np.zeros((T, r))
    u[np.arange(T), js] = 1.0
    z = oracle.lowrank_z(u, W)
    assert z.shape == (T, H, 128)
    for t in range(T):
        assert np.array_equal(z[t], W[:, :, js[t]])


def test_separable_inputs_closed_form():
    """u[t, j] = a_t b_j and W[h, c, j] = d_hc f_j give z = a_t d_hc (b . f)."""
    rng = np.random.default_rng(8)
    H, r, T = 2, 64, 17
    a, b, f = rng.standard_normal(T), rng.standard_normal(r), rng.standard_normal(r)
    d = rng.standard_normal((H, 128))
    z = oracle.lowrank_z(np.outer(a, b), d[:, :, None] * f[None, None, :])
    want = a[:, None, None] * d[None] * float(np.dot(b, f))
    np.testing.assert_allclose(z, want, rtol=1e-12, atol=1e-12)


def test_zero_rows_give_zero():
    rng = np.random.default_rng(9)
    u = rng.standard_normal((10, 32))
    u[3] = 0.0
    z = oracle.lowrank_z(u, rng.standard_normal((2, 128, 32)))
    assert not z[3].any() and z[2].any()
