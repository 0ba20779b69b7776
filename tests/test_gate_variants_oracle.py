"""Pins of the oracle's decay variants: the recurrence with given log-decays
(recurrent_g), Kimi Linear's unbounded negative-softplus decay (softplus_gate),
and the per-head scalar gate of Gated DeltaNet, against closed forms and the
pinned K3 recurrence."""
import math

import numpy as np

import oracle
import synth


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def test_softplus_closed_values():
    A = np.array([0.0, math.log(2.0)])
    z = np.zeros((1, 2, 128))
    z[0, :, 1], z[0, :, 2], z[0, :, 3], z[0, :, 4] = 50.0, -50.0, np.inf, -np.inf
    g = oracle.softplus_gate(z, A)
    assert g[0, 0, 0] == -math.log(2.0)                 # softplus(0) = ln 2, e^0 = 1
    assert g[0, 1, 0] == -2.0 * math.log(2.0)           # e^{ln 2} = 2
    np.testing.assert_allclose(g[0, 0, 1], -50.0, rtol=1e-15)          # softplus(z) -> z
    np.testing.assert_allclose(g[0, 0, 2], -math.exp(-50.0), rtol=1e-12)  # softplus(z) -> e^z
    assert g[0, 0, 3] == -np.inf and g[0, 0, 4] == 0.0  # unbounded below; z = -inf keeps the state


def test_softplus_identities():
    """Two properties softplus has whatever its formula: softplus(z) - softplus(-z) = z, and its
    derivative is the logistic function, here taken from the (separately pinned) K3 gate with
    e^A = 1, sigmoid(z) = -gate(z) / 5.  Checked by central differences of the oracle's decay."""
    rng = np.random.default_rng(3)
    A = rng.uniform(-1, 1, size=3)
    z = rng.uniform(-30, 30, size=(5, 3, 128))
    ea = np.exp(A)[None, :, None]
    sp = -oracle.softplus_gate(z, A) / ea
    sm = -oracle.softplus_gate(-z, A) / ea
    np.testing.assert_allclose(sp - sm, z, rtol=1e-12, atol=1e-12)
    h = 1e-5
    zc = rng.uniform(-8, 8, size=(4, 3, 128)).astype(np.float32).astype(np.float64)  # the gate reads fp32 z
    dsp = (oracle.softplus_gate(zc - h, A) - oracle.softplus_gate(zc + h, A)) / (2 * h) / ea
    sig = -np.stack([oracle.gate(zc[:, i], 0.0) for i in range(3)], axis=1) / 5.0
    np.testing.assert_allclose(dsp, sig, rtol=1e-7, atol=1e-9)
    g = oracle.softplus_gate(z, A)
    assert g.min() < -5.0 * math.e  # unbounded: well below the K3 bound g_min = -5


def test_given_log_decays_equal_the_k3_gate():
    d = synth.prefill_inputs(31, 200, 2, dtype="f32", s0_std=0.02)
    g = np.stack([oracle.gate(d["z"][:, h], d["A"][h]) for h in range(2)], axis=1)
    o1, S1 = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])
    o2, S2 = oracle.recurrent_g(d["q"], d["k"], d["v"], g, d["beta"], d["S0"])
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_given_log_decays_beta_zero_closed_form():
    """beta = 0 with any decay: S_T = Diag(e^{sum g}) S0 and o_t = S0^T (e^{G_t} * q_t)."""
    d = synth.prefill_inputs(32, 120, 2, dtype="f32", s0_std=0.02)
    g = oracle.softplus_gate(d["z"] - 4.0, d["A"])  # mild decay so nothing underflows
    o, S = oracle.recurrent_g(d["q"], d["k"], d["v"], g, np.zeros_like(d["beta"]), d["S0"])
    for h in range(2):
        G = np.cumsum(g[:, h], axis=0)
        S0 = d["S0"][0, h].astype(np.float64)
        assert _rel(S[0, h], np.exp(G[-1])[:, None] * S0) < 1e-12
        assert _rel(o[:, h], (np.exp(G) * d["q"][:, h]) @ S0) < 1e-12


def test_per_head_gate_is_gated_deltanet():
    """One gate value per (token, head) broadcast over the key channels is the scalar-gate rule,
    checked against the separately written Gated DeltaNet recurrence."""
    d = synth.prefill_inputs(33, 90, 1, dtype="f32", s0_std=0.02)
    zh = d["z"][:, :, :1]
    zb = np.broadcast_to(zh, d["z"].shape).astype(np.float32)
    o1, S1 = oracle.recurrent(d["q"], d["k"], d["v"], zb, d["beta"], d["A"], d["S0"])
    alpha = np.exp(oracle.gate(zh[:, 0, 0], d["A"][0]))
    o2, S2 = oracle.gdn(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], alpha, d["beta"][:, 0], d["S0"][0, 0])
    assert _rel(o1[:, 0], o2) < 1e-12 and _rel(S1[0, 0], S2) < 1e-12
