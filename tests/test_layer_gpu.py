"""GPU parity of the KDA layer's steps fused into the prefill (kda_chunk_fwd_layer):
unit-length q and k computed inside, and the output's per-head RMSNorm followed by the
sigmoid output gate (Kimi Linear summary, section 4), against the oracle's
l2_normalize / recurrent / gated_rmsnorm.

Bars: max|Δ|/RMS <= 1e-2 (bf16 q/k/v) and <= 1e-4 (fp32 q/k/v), as for the operator."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, err, say, to_dev

import gated_delta_rule_29_amd as kda

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}
EPS = 1e-6
LENS = [0, 100, 640, 777, 64, 191]


def layer_inputs(seed, io, lens=LENS, H=3):
    """Operator inputs with q and k scaled off unit length per row, plus the output gate and weight."""
    cu = synth.cu_seqlens(lens)
    T = int(cu[-1])
    d = synth.prefill_inputs(seed, T, H, dtype=io, z_scale=1.5, s0_std=0.02, n_seqs=len(lens))
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    for n in ("q", "k"):
        x = d[n] * rng.uniform(0.3, 3.0, size=(T, H, 1)).astype(np.float32)
        if io == "bf16":
            x = synth.bf16_round(x)
        d[n] = x.astype(np.float32)
    d["gate"] = (2.0 * rng.standard_normal((T, H, 128))).astype(np.float32)
    d["weight"] = rng.uniform(0.5, 1.5, size=128).astype(np.float32)
    return d, cu


def upload(d, io, cu):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    t = {n: to_dev(d[n], dt) for n in ("q", "k", "v")}
    for n in ("z", "beta", "A", "S0", "gate", "weight"):
        t[n] = to_dev(d[n], torch.float32)
    t["cu"] = None if cu is None else to_dev(np.asarray(cu, np.int32), torch.int32)
    return t


def reference(d, cu, gate=True):
    qn, kn = oracle.l2_normalize(d["q"], EPS), oracle.l2_normalize(d["k"], EPS)
    o, S = oracle.recurrent(qn, kn, d["v"], d["z"], d["beta"], d["A"], d["S0"], cu)
    if gate:
        o = oracle.gated_rmsnorm(o, d["gate"], d["weight"], EPS)
    return o, S


def check_layer(t, d, cu, io, label):
    """Run the layer with both steps and with the normalisation alone.  The operator output
    (normalisation alone) is held to the operator's bar against the oracle.  The fused output
    is held to fp32 rounding against the output step applied to that operator output: the
    RMSNorm divides each row by its own RMS, so comparing the normalised rows with the
    oracle's would scale the operator's error by RMS(o) / RMS(row), which has no bound."""
    y, S1 = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"], qk_l2norm=True,
                              qk_eps=EPS, out_gate=t["gate"], norm_weight=t["weight"], norm_eps=EPS)
    o, S2 = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"], qk_l2norm=True,
                              qk_eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    o_ref, S_ref = reference(d, cu, gate=False)
    o_np = o.cpu().numpy()
    eo, es = err(o_np, o_ref), err(S1.cpu().numpy(), S_ref)
    ey = err(y.cpu().numpy(), oracle.gated_rmsnorm(o_np, d["gate"], d["weight"], EPS))
    say(f"  {label} err_o={eo:.3e} err_S={es:.3e} err_output_step={ey:.3e}")
    assert eo <= TOL[io] and es <= TOL[io], (eo, es)
    assert ey <= 1e-5, ey


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_layer_steps_match_oracle(io):
    d, cu = layer_inputs(5100, io)
    say(f"case layer steps io={io}")
    check_layer(upload(d, io, cu), d, cu, io, "layer")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_qk_normalisation_alone(io):
    d, cu = layer_inputs(5200, io)
    say(f"case qk normalisation io={io}")
    t = upload(d, io, cu)
    o, Sf = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"], qk_l2norm=True,
                              qk_eps=EPS)
    torch.cuda.synchronize()
    o_ref, S_ref = reference(d, cu, gate=False)
    eo, es = err(o.cpu().numpy(), o_ref), err(Sf.cpu().numpy(), S_ref)
    say(f"  err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= TOL[io] and es <= TOL[io], (eo, es)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_output_step_equals_separate_step(io):
    """With unit-length inputs, the fused output step equals the operator's plain output taken
    through gated_rmsnorm afterwards, to fp32 rounding (both sides use the same operator bits)."""
    d, cu = layer_inputs(5300, io)
    for n in ("q", "k"):
        x = oracle.l2_normalize(d[n]).astype(np.float32)
        d[n] = synth.bf16_round(x) if io == "bf16" else x
    say(f"case fused output step io={io}")
    t = upload(d, io, cu)
    o_plain, S1 = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"])
    o_fused, S2 = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"],
                                    out_gate=t["gate"], norm_weight=t["weight"], norm_eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    want = oracle.gated_rmsnorm(o_plain.cpu().numpy(), d["gate"], d["weight"], EPS)
    e = err(o_fused.cpu().numpy(), want)
    say(f"  err={e:.3e}")
    assert e <= 1e-5, e


def test_layer_steps_are_deterministic_and_keep_snapshots():
    d, cu = layer_inputs(5400, "bf16")
    say("case layer determinism + snapshots")
    t = upload(d, "bf16", cu)
    slots = kda.ckpt_count(LENS, 128)
    outs = []
    for _ in range(2):
        S_ck = torch.zeros((slots, 3, 128, 128), device=DEV)
        o, Sf = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"],
                                  qk_l2norm=True, qk_eps=EPS, out_gate=t["gate"], norm_weight=t["weight"],
                                  norm_eps=EPS, S_ckpt=S_ck, ckpt_stride=128)
        outs.append((o.clone(), Sf.clone(), S_ck))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))
    qn, kn = oracle.l2_normalize(d["q"], EPS), oracle.l2_normalize(d["k"], EPS)
    ref = oracle.states_at(qn, kn, d["v"], d["z"], d["beta"], d["A"], d["S0"], cu, 128)
    assert err(outs[0][2].cpu().numpy(), ref) <= TOL["bf16"]


@pytest.mark.timeout(300)
def test_layer_steps_64k():
    """The 64K x 16 workload with raw q, k and the output step fused in."""
    T, H = 65536, 16
    d, cu = layer_inputs(5500, "bf16", lens=[T], H=H)
    say("case layer steps 64K x 16")
    check_layer(upload(d, "bf16", None), d, cu, "bf16", "64K")
