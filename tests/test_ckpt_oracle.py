"""Pins of oracle.states_at, the prefix-cache snapshots (Kimi K3 paper review,
Significance and Limitations paragraphs: the KDA state is checkpointed only at
sparse boundaries), against results that do not go through its own loop."""
import numpy as np

import oracle
import synth


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


LENS = [0, 100, 128, 300, 64, 257]
STRIDE = 64


def _pack(seed, H=2):
    cu = synth.cu_seqlens(LENS)
    d = synth.prefill_inputs(seed, int(cu[-1]), H, dtype="f32", s0_std=0.02, n_seqs=len(LENS))
    return d, cu


def test_slot_order_and_count():
    """One slot per whole stride of each sequence, sequence after sequence."""
    d, cu = _pack(21)
    S = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu, STRIDE)
    assert S.shape[0] == sum(n // STRIDE for n in LENS) == 0 + 1 + 2 + 4 + 1 + 4


def test_each_snapshot_is_a_prefix_run():
    """Snapshot m of sequence n equals S_final of one recurrent run over the sequence's first
    (m + 1) * stride tokens from S0 (a single call, no chaining)."""
    d, cu = _pack(22)
    S = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu, STRIDE)
    slot = 0
    for n, L in enumerate(LENS):
        a = int(cu[n])
        for m in range(L // STRIDE):
            b = a + (m + 1) * STRIDE
            _, Sf = oracle.recurrent(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["z"][a:b], d["beta"][a:b],
                                     d["A"], d["S0"][n:n + 1])
            assert _rel(S[slot], Sf[0]) < 1e-12, (n, m)
            slot += 1
    assert slot == S.shape[0]


def test_last_snapshot_is_the_final_state_on_a_stride_multiple():
    d, cu = _pack(23)
    S = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu, STRIDE)
    _, Sf = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu)
    # sequence 2 (128 tokens) owns slots 1, 2; sequence 4 (64 tokens) owns slot 7
    assert np.array_equal(S[2], Sf[2]) and np.array_equal(S[7], Sf[4])


def test_beta_zero_closed_form():
    """beta = 0: the state after t tokens is Diag(e^{sum of g over those tokens}) S0, with g the
    K3 gate written out here in numpy (-5 * sigmoid(e^A z)).  z is shifted down so that the
    decay over 300 tokens stays far from underflow; the check is elementwise relative."""
    d, cu = _pack(24)
    d["z"] = (d["z"] - 3.0).astype(np.float32)
    beta = np.zeros_like(d["beta"])
    S = oracle.states_at(d["q"], d["k"], d["v"], d["z"], beta, d["A"], d["S0"], cu, STRIDE)
    slot = 0
    for n, L in enumerate(LENS):
        a = int(cu[n])
        for m in range(L // STRIDE):
            b = a + (m + 1) * STRIDE
            for h in range(2):
                x = np.exp(np.float64(d["A"][h])) * d["z"][a:b, h].astype(np.float64)
                g = -5.0 / (1.0 + np.exp(-x))
                exp_S = np.exp(g.sum(axis=0))[:, None] * d["S0"][n, h].astype(np.float64)
                np.testing.assert_allclose(S[slot, h], exp_S, rtol=1e-11, atol=0)
            slot += 1


def test_stride_longer_than_every_sequence_gives_no_snapshot():
    d, cu = _pack(25)
    S = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu, 512)
    assert S.shape == (0, 2, 128, 128)
