"""GPU parity of the forget gate's low-rank projection fused into the operator
(Kimi Linear summary, section 4: the forget and output gates use low-rank
projections): z[t, h, c] = sum_j u[t, j] W[h, c, j] is formed inside the
kernels from bf16 factors instead of being read as [tokens, H, 128] fp32.
Compared with the oracle's recurrence on oracle.lowrank_z(u, W), for both decay
parameterisations, both I/O dtypes, packed ragged sequences, ranks 32 to 256,
and the decode step.

Bars as for the operator: max|Δ|/RMS <= 1e-2 (bf16 q/k/v), <= 1e-4 (fp32 q/k/v)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import err, say, to_dev

import gated_delta_rule_29_amd as kda

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}
LENS = [100, 0, 640, 17, 64, 383]


def log_decays(z, A, gate):
    """g [T, H, 128] float64 from the oracle's gates (the K3 gate takes z rounded to fp32)."""
    if gate == "softplus":
        return oracle.softplus_gate(z, A)
    z32 = np.asarray(z, np.float32)
    return np.stack([oracle.gate(z32[:, h], A[h]) for h in range(z32.shape[1])], axis=1)


def reference(d, cu, z, gate):
    return oracle.recurrent_g(d["q"], d["k"], d["v"], log_decays(z, d["A"], gate), d["beta"], d["S0"], cu)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["k3", "softplus"])
@pytest.mark.parametrize("rank", [32, 128, 256])
def test_prefill_lowrank_gate(io, gate, rank):
    cu = synth.cu_seqlens(LENS)
    T, H = int(cu[-1]), 3
    d = synth.prefill_inputs(5600 + rank, T, H, dtype=io, s0_std=0.02, n_seqs=len(LENS))
    u, W = synth.lowrank_gate(5600 + rank, T, H, rank)
    z = oracle.lowrank_z(u, W)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v = (to_dev(d[n], dt) for n in ("q", "k", "v"))
    beta, A, S0 = (to_dev(d[n], torch.float32) for n in ("beta", "A", "S0"))
    cu_t = to_dev(np.asarray(cu, np.int32), torch.int32)
    say(f"case lowrank prefill io={io} gate={gate} rank={rank}")
    o, Sf = kda.kda_chunk_fwd(q, k, v, None, beta, A, S0, cu_t, gate=gate, gate_u=to_dev(u, torch.bfloat16),
                              gate_w=to_dev(W, torch.bfloat16))
    torch.cuda.synchronize()
    o_ref, S_ref = reference(d, cu, z, gate)
    eo, es = err(o.cpu().numpy(), o_ref), err(Sf.cpu().numpy(), S_ref)
    say(f"  err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= TOL[io] and es <= TOL[io], (eo, es)


@pytest.mark.parametrize("io,bound", [("bf16", 3e-3), ("f32", 1e-5)])
def test_prefill_lowrank_equals_given_z_closely(io, bound):
    """The fused projection and the same z given in fp32 (rounded from float64) run the
    same recurrence.  Their z differ by the projection's fp32 summation order, about an
    ulp; with fp32 q/k/v that moves o by about that much.  With bf16 q/k/v such a nudge
    of a gate can flip the rounding of the fp16 chain operands (relative 2^-11), so
    there the bound is that noise level, still well inside the operator's bar."""
    T, H, rank = 1000, 4, 128
    d = synth.prefill_inputs(5650, T, H, dtype=io, s0_std=0.02)
    u, W = synth.lowrank_gate(5650, T, H, rank)
    z = oracle.lowrank_z(u, W).astype(np.float32)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v = (to_dev(d[n], dt) for n in ("q", "k", "v"))
    beta, A, S0 = (to_dev(d[n], torch.float32) for n in ("beta", "A", "S0"))
    say(f"case lowrank vs given z io={io}")
    o1, S1 = kda.kda_chunk_fwd(q, k, v, None, beta, A, S0, gate_u=to_dev(u, torch.bfloat16),
                               gate_w=to_dev(W, torch.bfloat16))
    o2, S2 = kda.kda_chunk_fwd(q, k, v, to_dev(z, torch.float32), beta, A, S0)
    torch.cuda.synchronize()
    eo, es = err(o1.cpu().numpy(), o2.cpu().numpy()), err(S1.cpu().numpy(), S2.cpu().numpy())
    say(f"  lowrank vs given z: {eo:.3e} {es:.3e}")
    assert eo <= bound and es <= bound


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["k3", "softplus"])
def test_decode_lowrank_gate(io, gate):
    N, H, rank = 7, 3, 64
    d = synth.decode_tokens(5700, 0, N, H, dtype=io)
    A = synth.head_params(5700, H)
    S = synth.initial_state(5700, N, H, 0.05)
    u, W = synth.lowrank_gate(5700, N, H, rank)
    z = oracle.lowrank_z(u, W)
    g = log_decays(z, A, gate)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v = (to_dev(d[n], dt) for n in ("q", "k", "v"))
    S_t = to_dev(S, torch.float32)
    say(f"case lowrank decode io={io} gate={gate}")
    o = kda.kda_decode_step(q, k, v, None, to_dev(d["beta"], torch.float32), to_dev(A, torch.float32), S_t,
                            gate=gate, gate_u=to_dev(u, torch.bfloat16), gate_w=to_dev(W, torch.bfloat16))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent_g(d["q"], d["k"], d["v"], g, d["beta"], S, np.arange(N + 1))
    eo, es = err(o.cpu().numpy(), o_ref), err(S_t.cpu().numpy(), S_ref)
    say(f"  err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= TOL[io] and es <= TOL[io], (eo, es)


def test_lowrank_gate_with_layer_steps_snapshots_and_softplus():
    """Every layer option at once on a ragged pack: q/k normalisation, the low-rank
    forget gate under softplus decay, snapshots, and the output step.  The operator part
    is held to the bar against the oracle; the output step to fp32 rounding against the
    step applied to the GPU's own operator output (as for the plain layer test)."""
    lens = [300, 64, 0, 257]
    cu = synth.cu_seqlens(lens)
    T, H, rank, eps, stride = int(cu[-1]), 2, 96, 1e-6, 128
    d = synth.prefill_inputs(5750, T, H, s0_std=0.02, n_seqs=len(lens))
    rng = np.random.Generator(np.random.PCG64(5751))
    for n in ("q", "k"):
        d[n] = synth.bf16_round(d[n] * rng.uniform(0.3, 3.0, size=(T, H, 1)).astype(np.float32))
    gate = (2.0 * rng.standard_normal((T, H, 128))).astype(np.float32)
    weight = rng.uniform(0.5, 1.5, size=128).astype(np.float32)
    u, W = synth.lowrank_gate(5750, T, H, rank)
    q, k, v = (to_dev(d[n], torch.bfloat16) for n in ("q", "k", "v"))
    beta, A, S0 = (to_dev(d[n], torch.float32) for n in ("beta", "A", "S0"))
    cu_t = to_dev(np.asarray(cu, np.int32), torch.int32)
    gu, gw = to_dev(u, torch.bfloat16), to_dev(W, torch.bfloat16)
    ck = torch.empty((kda.ckpt_count(lens, stride), H, 128, 128), dtype=torch.float32, device=q.device)
    say("case lowrank + softplus + layer steps + snapshots")
    kw = dict(gate="softplus", gate_u=gu, gate_w=gw, qk_l2norm=True, qk_eps=eps)
    y, S1 = kda.kda_chunk_fwd(q, k, v, None, beta, A, S0, cu_t, S_ckpt=ck, ckpt_stride=stride,
                              out_gate=to_dev(gate, torch.float32), norm_weight=to_dev(weight, torch.float32),
                              norm_eps=eps, **kw)
    o, S2 = kda.kda_chunk_fwd(q, k, v, None, beta, A, S0, cu_t, **kw)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    qn, kn = oracle.l2_normalize(d["q"], eps), oracle.l2_normalize(d["k"], eps)
    g = oracle.softplus_gate(oracle.lowrank_z(u, W), d["A"])
    o_ref, S_ref = oracle.recurrent_g(qn, kn, d["v"], g, d["beta"], d["S0"], cu)
    o_np = o.cpu().numpy()
    eo, es = err(o_np, o_ref), err(S1.cpu().numpy(), S_ref)
    ey = err(y.cpu().numpy(), oracle.gated_rmsnorm(o_np, gate, weight, eps))
    say(f"  err_o={eo:.3e} err_S={es:.3e} err_output_step={ey:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and ey <= 1e-5
    slot = 0
    for n, L in enumerate(lens):
        for m in range(L // stride):
            sl = slice(int(cu[n]), int(cu[n]) + (m + 1) * stride)
            _, S_m = oracle.recurrent_g(qn[sl], kn[sl], d["v"][sl], g[sl], d["beta"][sl], d["S0"][n:n + 1])
            assert err(ck[slot].cpu().numpy(), S_m[0]) <= TOL["bf16"], (n, m)
            slot += 1
    assert slot == ck.shape[0]
