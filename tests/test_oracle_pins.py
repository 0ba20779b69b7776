"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test names the passage it follows.  Pages:
  [K3]  "Kimi K3 architecture" (molayo1419.me), sequence-bottleneck section.
  [KL]  "Kimi Linear: An Expressive, Efficient Attention Architecture" summary
        (greeksharifa.github.io), sections 2.1, 2.2, 3, 3.1, 6.2, 6.3.

The expected values below never come from the oracle itself: they are closed
forms evaluated with numpy, exact algebraic identities, finite differences, or
values printed on the pages (tests/golden/).
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def _golden(name):
    rows = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        rows[parts[0]] = [float(x) for x in parts[1:]]
    return rows


def exact_unit_keys(rng, n, d=D):
    """n unit vectors with entries 0 or +-1/8 on 64 coordinates: exactly unit norm in float32."""
    out = np.zeros((n, d), np.float32)
    for i in range(n):
        idx = rng.permutation(d)[:64]
        out[i, idx] = rng.choice([-0.125, 0.125], size=64)
    return out


def exact_orthonormal_keys(rng, n, d=D):
    """n <= d exactly orthonormal float32 vectors: rows of two 64x64 Sylvester-Hadamard
    blocks scaled by 1/8, under a random signed permutation of the coordinates."""
    assert n <= d
    h = np.array([[1.0]])
    while h.shape[0] < 64:
        h = np.block([[h, h], [h, -h]])
    basis = np.zeros((d, d))
    basis[:64, :64] = h / 8.0
    basis[64:, 64:] = h / 8.0
    perm = rng.permutation(d)
    signs = rng.choice([-1.0, 1.0], size=d)
    basis = basis[:, perm] * signs
    rows = rng.permutation(d)[:n]
    return basis[rows].astype(np.float32)


def inputs(seed, T, H=2, dtype="f32", z_scale=1.0, s0_std=0.02, n_seqs=1):
    return synth.prefill_inputs(seed, T, H, dtype=dtype, z_scale=z_scale, s0_std=s0_std, n_seqs=n_seqs)


# ----------------------------------------------------------------- gate --

def test_gate_closed_values():
    """[K3] g = -5 Sigmoid(e^A z): logistic values at 0 and +-ln 3, and the limits."""
    ln3 = math.log(3.0)
    z = np.array([0.0, ln3, -ln3, np.inf, -np.inf, 1e4, -1e4], np.float32)
    g = oracle.gate(z, 0.0)
    # float32 ln 3 differs from ln 3 by < 3e-8; the logistic has slope <= 1/4.
    np.testing.assert_allclose(g[:3], [-2.5, -3.75, -1.25], rtol=0, atol=5 * 0.25 * 3e-8 + 1e-15)
    assert g[0] == -2.5
    assert g[3] == -5.0 and g[5] == -5.0
    assert g[4] == 0.0 and g[6] == 0.0
    # A enters as e^A: A = ln 2 halves the z that gives the same gate
    g2 = oracle.gate(np.array([ln3 / 2], np.float32), math.log(2.0))
    assert abs(g2[0] + 3.75) < 1e-6
    assert np.isnan(oracle.gate(np.array([np.nan], np.float32), 0.3)[0])


def test_gate_bounds_golden():
    """[K3] g in (g_min, 0) with g_min = -5, alpha > e^-5 ~ 6.7e-3, 16-token sums in (-80, 0)."""
    gold = _golden("gate_bounds.txt")
    gmin = gold["g_min"][0]
    rng = np.random.default_rng(0)
    z = (rng.standard_normal(200_000) * 4).astype(np.float32)
    for A in (-1.0, 0.0, 0.7, 1.0):
        g = oracle.gate(z, A)
        assert g.min() >= gmin and g.max() <= 0.0
        alpha = np.exp(g)
        # the printed bound, to its printed precision
        lb, tol = gold["alpha_lower_bound"]
        assert abs(math.exp(gmin) - lb) <= tol * lb
        assert alpha.min() >= math.exp(gmin) and alpha.max() <= 1.0
        tile = int(gold["tile_tokens"][0])
        sums = g[: (g.size // tile) * tile].reshape(-1, tile).sum(axis=1)
        assert sums.min() >= gold["tile_logdecay_lower"][0] and sums.max() <= 0.0
    # z = +inf hits the bound exactly: every factor of a tile then equals e^{-80}
    g = oracle.gate(np.full(16, np.inf, np.float32), 0.0)
    assert g.sum() == -80.0


# ------------------------------------------------------- closed forms --

def test_beta_zero_closed_form():
    """[KL 3] beta = 0: S_T = Diag(e^{sum g}) S0 and o_t = S0^T (e^{G_t} * q_t), G the running sum."""
    d = inputs(11, 150, H=2)
    beta = np.zeros_like(d["beta"])
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], beta, d["A"], d["S0"])
    for h in range(2):
        g = oracle.gate(d["z"][:, h], d["A"][h])
        G = np.cumsum(g, axis=0)
        S0 = d["S0"][0, h].astype(np.float64)
        exp_o = (np.exp(G) * d["q"][:, h]) @ S0
        # |G| reaches ~400 here: the float64 running sum carries ~1e-13 absolute error per
        # term, which exp turns into relative error; 1e-10 bounds that, not a model error.
        assert _rel(o[:, h], exp_o) < 1e-10
        assert _rel(S[0, h], np.exp(G[-1])[:, None] * S0) < 1e-10


def test_frozen_state_exact():
    """[KL 3] beta = 0 and alpha = 1 (z = -inf): the state is frozen, o_t = S0^T q_t."""
    d = inputs(12, 70, H=2)
    z = np.full_like(d["z"], -np.inf)
    beta = np.zeros_like(d["beta"])
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], z, beta, d["A"], d["S0"])
    assert np.array_equal(S, d["S0"].astype(np.float64))
    for h in range(2):
        exp_o = d["q"][:, h].astype(np.float64) @ d["S0"][0, h].astype(np.float64)
        assert _rel(o[:, h], exp_o) < 1e-13


@pytest.mark.parametrize("T", [5, 64, 100, 128])
def test_associative_recall_orthonormal_keys(T):
    """[KL 2.2, 3] alpha = 1, beta = 1, orthonormal keys: each write stores v_i exactly,
    S_T = (I - sum k_i k_i^T) S0 + sum k_i v_i^T and S_T^T k_i = v_i for every i."""
    rng = np.random.default_rng(T)
    K = exact_orthonormal_keys(rng, T)
    V = rng.standard_normal((T, D)).astype(np.float32)
    Q = exact_unit_keys(rng, T)
    S0 = (0.3 * rng.standard_normal((D, D))).astype(np.float32)
    z = np.full((T, 1, D), -np.inf, np.float32)
    beta = np.ones((T, 1), np.float32)
    args = (Q[:, None], K[:, None], V[:, None], z, beta, np.zeros(1, np.float32), S0[None, None])
    o, S = oracle.recurrent(*args)
    K64, V64, S064 = K.astype(np.float64), V.astype(np.float64), S0.astype(np.float64)
    expect = (np.eye(D) - K64.T @ K64) @ S064 + K64.T @ V64
    assert _rel(S[0, 0], expect) < 1e-12
    assert _rel(S[0, 0].T @ K64.T, V64.T) < 1e-12
    oc, Sc = oracle.chunk(*args, C=64)
    assert _rel(Sc[0, 0], expect) < 1e-12
    if T <= 8:
        ob, Sb = oracle.bruteforce(Q, K, V, z[:, 0], beta[:, 0], 0.0, S0)
        assert _rel(Sb, expect) < 1e-12


def test_delta_rule_is_gradient_step():
    """[KL 2.2] with alpha = 1, one step is S - beta * grad L(S), L(S) = 1/2 ||S^T k - v||^2
    (gradient by central finite differences, not by the formula)."""
    rng = np.random.default_rng(5)
    k = exact_unit_keys(rng, 1)[0]
    v = rng.standard_normal(D).astype(np.float32)
    q = exact_unit_keys(rng, 1)[0]
    S0 = rng.standard_normal((D, D)).astype(np.float32)
    for beta in (0.0, 0.3, 1.0, 1.7):
        o, S1 = oracle.recurrent(q[None, None], k[None, None], v[None, None],
                                 np.full((1, 1, D), -np.inf, np.float32),
                                 np.full((1, 1), beta, np.float32), np.zeros(1, np.float32),
                                 S0[None, None])
        S0d = S0.astype(np.float64)

        def loss(S):
            r = S.T @ k.astype(np.float64) - v
            return 0.5 * float(r @ r)

        eps = 1e-4
        for (i, j) in [(0, 0), (3, 7), (17, 100), (127, 127), (64, 1)]:
            Sp, Sm = S0d.copy(), S0d.copy()
            Sp[i, j] += eps
            Sm[i, j] -= eps
            grad = (loss(Sp) - loss(Sm)) / (2 * eps)
            step = S0d[i, j] - S1[0, 0][i, j]
            assert abs(step - beta * grad) < 1e-6 * max(1.0, abs(grad))


def test_erase_then_write_order():
    """[KL 3] decay first, then the delta correction: with beta = 1 and a unit key, right after
    step t the state returns v_t for k_t (any decay), and o_t = v_t when q_t = k_t
    (the read-out uses the updated state)."""
    rng = np.random.default_rng(9)
    T = 40
    K = exact_unit_keys(rng, T)
    V = rng.standard_normal((T, D)).astype(np.float32)
    z = rng.standard_normal((T, 1, D)).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((1, 1, D, D))).astype(np.float32)
    beta = np.ones((T, 1), np.float32)
    o, S = oracle.recurrent(K[:, None], K[:, None], V[:, None], z, beta, np.array([0.4], np.float32), S0)
    assert _rel(o[:, 0], V) < 1e-12
    for t in (1, 7, 40):
        _, St = oracle.recurrent(K[:t, None], K[:t, None], V[:t, None], z[:t], beta[:t],
                                 np.array([0.4], np.float32), S0)
        assert _rel(St[0, 0].T @ K[t - 1].astype(np.float64), V[t - 1]) < 1e-12


def test_scalar_gate_is_gated_deltanet():
    """[KL 2.2, 3] the same decay on every channel reduces KDA to Gated DeltaNet."""
    d = inputs(21, 90, H=1)
    zc = np.repeat(d["z"][:, :, :1], D, axis=2)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], zc, d["beta"], d["A"], d["S0"])
    alpha = np.exp(oracle.gate(zc[:, 0, 0], d["A"][0]))
    og, Sg = oracle.gdn(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], alpha, d["beta"][:, 0], d["S0"][0, 0])
    assert _rel(o[:, 0], og) < 1e-12
    assert _rel(S[0, 0], Sg) < 1e-12


def test_gdn_beta_zero_closed_form():
    """[KL 2.2] Gated DeltaNet with beta = 0 only decays: S_T = (prod alpha) S0."""
    rng = np.random.default_rng(3)
    T = 30
    q = rng.standard_normal((T, D)).astype(np.float32)
    alpha = rng.uniform(0.5, 1.0, T)
    S0 = rng.standard_normal((D, D))
    o, S = oracle.gdn(q, q, q, alpha, np.zeros(T, np.float32), S0)
    assert _rel(S, np.prod(alpha) * S0) < 1e-13
    assert _rel(o[-1], S.T @ q[-1].astype(np.float64)) < 1e-13


# ------------------------------------------- independent formulations --

@pytest.mark.parametrize("T", [1, 3, 8])
def test_bruteforce_matches_recurrence(T):
    """[KL 6.2] dense transition products Diag(a) - b k k^T Diag(a) give the same o and S."""
    d = inputs(30 + T, T, H=1, z_scale=1.5)
    for h in range(1):
        ob, Sb = oracle.bruteforce(d["q"][:, h], d["k"][:, h], d["v"][:, h], d["z"][:, h],
                                   d["beta"][:, h], d["A"][h], d["S0"][0, h])
        o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
        assert _rel(ob, o[:, h]) < 1e-12
        assert _rel(Sb, S[0, h]) < 1e-12


def test_bruteforce_beta_zero_closed_form():
    """The brute force on its own pin: beta = 0 gives o_t = S0^T (e^{G_t} * q_t)."""
    d = inputs(41, 6, H=1)
    ob, Sb = oracle.bruteforce(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["z"][:, 0],
                               np.zeros(6, np.float32), d["A"][0], d["S0"][0, 0])
    G = np.cumsum(oracle.gate(d["z"][:, 0], d["A"][0]), axis=0)
    assert _rel(ob, (np.exp(G) * d["q"][:, 0]) @ d["S0"][0, 0].astype(np.float64)) < 1e-12


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("shaped", [False, True])
def test_chunk_form_matches_recurrence(C, shaped):
    """[KL 3.1, App. B/C] the chunkwise WY/UT form with forward substitution reaches the
    recurrence's result, for full and partial chunks and packed sequences."""
    lens = [1, 9, 15, 16, 17, 63, 64, 65, 200]
    d = inputs(50 + C, sum(lens), H=2, z_scale=2.0, n_seqs=len(lens))
    cu = synth.cu_seqlens(lens)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu)
    oc, Sc = oracle.chunk(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu,
                          C=C, shaped=shaped)
    assert _rel(oc, o) < 1e-12
    assert _rel(Sc, S) < 1e-12


def test_chunk_form_at_the_gate_bound():
    """[K3] z = +inf on every channel: 16-token tiles reach e^{-80}; the sub-chunk factors stay
    finite and the shaped chunk form still equals the recurrence."""
    d = inputs(61, 130, H=1)
    z = np.full_like(d["z"], np.inf)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], z, d["beta"], d["A"], d["S0"])
    oc, Sc = oracle.chunk(d["q"], d["k"], d["v"], z, d["beta"], d["A"], d["S0"], C=64, shaped=True)
    assert np.isfinite(oc).all() and np.isfinite(Sc).all()
    assert _rel(oc, o) < 1e-12 and _rel(Sc, S) < 1e-12


def test_chunk_step_intermediates():
    """[KL 3.1] T is the inverse of (I + StrictTril Akk), Akk is strictly lower triangular,
    Delta = U - W S and the outgoing state agrees with the recurrence."""
    d = inputs(71, 64, H=1)
    S = d["S0"][0, 0].astype(np.float64)
    r = oracle.chunk_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["z"][:, 0], d["beta"][:, 0],
                          d["A"][0], S)
    n = 64
    assert np.all(np.triu(r["Akk"]) == 0)
    assert np.all(np.triu(r["Aqk"], 1) == 0)
    assert np.abs(r["T"] @ (np.eye(n) + r["Akk"]) - np.eye(n)).max() < 1e-12
    assert _rel(r["Delta"], r["U"] - r["W"] @ S) < 1e-12
    assert np.all(np.diff(r["G"], axis=0) <= 0) and r["G"].min() >= -5 * n
    o, Sf = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    assert _rel(r["o"], o[:, 0]) < 1e-12 and _rel(r["S"], Sf[0, 0]) < 1e-12


# ---------------------------------------------------------- structure --

def test_heads_are_independent():
    d = inputs(80, 77, H=3)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    d2 = {k: v.copy() for k, v in d.items()}
    d2["v"][:, 1] += 1.0
    d2["z"][:, 1] *= -1
    o2, S2 = oracle.recurrent(d2["q"], d2["k"], d2["v"], d2["z"], d2["beta"], d2["A"], d2["S0"])
    assert np.array_equal(o[:, 0], o2[:, 0]) and np.array_equal(o[:, 2], o2[:, 2])
    assert np.array_equal(S[:, 0], S2[:, 0]) and not np.array_equal(o[:, 1], o2[:, 1])


def test_varlen_pack_equals_separate_runs():
    """[KL 2.1] each packed sequence starts from its own initial state."""
    lens = [5, 64, 0, 70]
    d = inputs(81, sum(lens), H=2, n_seqs=len(lens))
    cu = synth.cu_seqlens(lens)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = {k: d[k][a:b] for k in ("q", "k", "v", "z", "beta")}
        on, Sn = oracle.recurrent(sl["q"], sl["k"], sl["v"], sl["z"], sl["beta"], d["A"], d["S0"][n:n + 1])
        assert np.array_equal(o[a:b], on) and np.array_equal(S[n], Sn[0])
    assert np.array_equal(S[2], d["S0"][2].astype(np.float64))  # empty sequence keeps S0


def test_value_permutation_equivariance():
    d = inputs(82, 50, H=1)
    perm = np.random.default_rng(0).permutation(D)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    op, Sp = oracle.recurrent(d["q"], d["k"], d["v"][:, :, perm], d["z"], d["beta"], d["A"],
                              d["S0"][..., perm])
    assert np.array_equal(op, o[..., perm]) and np.array_equal(Sp, S[..., perm])


def test_linear_in_state_and_values():
    d = inputs(83, 60, H=1)
    e = inputs(84, 60, H=1)
    a, b = 0.7, -1.3
    f = lambda v, s: oracle.recurrent(d["q"], d["k"], v, d["z"], d["beta"], d["A"], s)
    o1, S1 = f(d["v"], d["S0"])
    o2, S2 = f(e["v"], e["S0"])
    o3, S3 = f(a * d["v"].astype(np.float64) + b * e["v"], a * d["S0"].astype(np.float64) + b * e["S0"])
    # the mixed inputs are rounded to float32 on entry; compare to that precision
    assert _rel(o3, a * o1 + b * o2) < 1e-6 and _rel(S3, a * S1 + b * S2) < 1e-6


@pytest.mark.parametrize("split", [1, 37, 64, 128, 199])
def test_split_resume_equals_one_pass(split):
    """[KL 2.1] a chunk (or a later call) starts from the previous final state."""
    d = inputs(85, 200, H=2)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    part = lambda a, b: {k: d[k][a:b] for k in ("q", "k", "v", "z", "beta")}
    p1, p2 = part(0, split), part(split, 200)
    o1, S1 = oracle.recurrent(p1["q"], p1["k"], p1["v"], p1["z"], p1["beta"], d["A"], d["S0"])
    o2, S2 = oracle.recurrent(p2["q"], p2["k"], p2["v"], p2["z"], p2["beta"], d["A"], S1)
    assert np.array_equal(np.concatenate([o1, o2]), o) and np.array_equal(S2, S)
    oc1, Sc1 = oracle.chunk(p1["q"], p1["k"], p1["v"], p1["z"], p1["beta"], d["A"], d["S0"])
    oc2, Sc2 = oracle.chunk(p2["q"], p2["k"], p2["v"], p2["z"], p2["beta"], d["A"], Sc1)
    assert _rel(np.concatenate([oc1, oc2]), o) < 1e-12 and _rel(Sc2, S) < 1e-12


def test_decode_steps_equal_prefill():
    """[KL 6.3] generation applies the recurrent update one token at a time."""
    d = inputs(86, 12, H=2)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    St = d["S0"].astype(np.float64)
    for t in range(12):
        ot, St = oracle.decode_step(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1], d["z"][t:t + 1],
                                    d["beta"][t:t + 1], d["A"], St)
        assert np.array_equal(ot[0], o[t])
    assert np.array_equal(St, S)


def test_float32_twin_noise_floor():
    """The float32 recurrence stays within 1e-4 of float64 (the fp32 I/O bound)."""
    d = inputs(87, 640, H=2, z_scale=1.0)
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    o32, S32 = oracle.recurrent_f32(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    assert _rel(o32, o) < 1e-4 and _rel(S32, S) < 1e-4


def test_threads_do_not_change_results():
    d = inputs(88, 100, H=4)
    o1, S1 = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], threads=1)
    o4, S4, n = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], threads=4,
                                 return_threads=True)
    assert n == 4 and np.array_equal(o1, o4) and np.array_equal(S1, S4)
