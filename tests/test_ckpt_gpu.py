"""GPU parity of the prefix-cache state snapshots (kda_chunk_fwd_ckpt) against
oracle.states_at: the state after every `stride` tokens of each sequence
(Kimi K3 paper review, Significance and Limitations paragraphs: the KDA state
is kept at sparse checkpoint boundaries, up to 6,144 tokens apart).

Bars as for the prefill: max|S - S_ref| / RMS(S_ref) <= 1e-2 with bf16 q/k/v,
<= 1e-4 with fp32 q/k/v.  o and S_final must be the same bits as without
snapshots."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, err, say, to_dev

import gated_delta_rule_29_amd as kda

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}
LENS = [0, 100, 640, 777, 1280, 2000, 64, 191, 192]


def upload(d, io, cu):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v = (to_dev(d[n], dt) for n in ("q", "k", "v"))
    z, beta, A = (to_dev(d[n], torch.float32) for n in ("z", "beta", "A"))
    cu_t = None if cu is None else to_dev(np.asarray(cu, np.int32), torch.int32)
    S0 = to_dev(d["S0"], torch.float32)
    return q, k, v, z, beta, A, S0, cu_t


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("stride", [64, 192, 640])
def test_snapshots_match_oracle(io, stride):
    cu = synth.cu_seqlens(LENS)
    d = synth.prefill_inputs(4100 + stride, int(cu[-1]), 3, dtype=io, z_scale=1.5, s0_std=0.02, n_seqs=len(LENS))
    say(f"case snapshots io={io} stride={stride} lens={LENS}")
    q, k, v, z, beta, A, S0, cu_t = upload(d, io, cu)
    slots = kda.ckpt_count(LENS, stride)
    S_ck = torch.full((slots, 3, 128, 128), float("nan"), device=DEV)
    o1, Sf1 = kda.kda_chunk_fwd(q, k, v, z, beta, A, S0, cu_t, S_ckpt=S_ck, ckpt_stride=stride)
    o2, Sf2 = kda.kda_chunk_fwd(q, k, v, z, beta, A, S0, cu_t)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(Sf1, Sf2)
    ref = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu, stride)
    assert ref.shape[0] == slots
    got = S_ck.cpu().numpy()
    e = err(got, ref)
    say(f"  err_ckpt={e:.3e}")
    assert e <= TOL[io], e


def test_snapshot_on_a_stride_multiple_equals_the_final_state():
    cu = synth.cu_seqlens([640, 1280])
    d = synth.prefill_inputs(4200, int(cu[-1]), 2, s0_std=0.02, n_seqs=2)
    say("case snapshot == S_final")
    q, k, v, z, beta, A, S0, cu_t = upload(d, "bf16", cu)
    S_ck = torch.zeros((kda.ckpt_count([640, 1280], 320), 2, 128, 128), device=DEV)
    _, Sf = kda.kda_chunk_fwd(q, k, v, z, beta, A, S0, cu_t, S_ckpt=S_ck, ckpt_stride=320)
    torch.cuda.synchronize()
    assert S_ck.shape[0] == 6
    assert torch.equal(S_ck[1], Sf[0]) and torch.equal(S_ck[5], Sf[1])


def test_capacity_bounds_the_writes():
    cu = synth.cu_seqlens(LENS)
    d = synth.prefill_inputs(4300, int(cu[-1]), 2, s0_std=0.02, n_seqs=len(LENS))
    say("case capacity")
    q, k, v, z, beta, A, S0, cu_t = upload(d, "bf16", cu)
    slots = kda.ckpt_count(LENS, 64)
    cap = slots // 2
    S_big = torch.full((slots, 2, 128, 128), float("nan"), device=DEV)
    kda.kda_chunk_fwd(q, k, v, z, beta, A, S0, cu_t, S_ckpt=S_big[:cap], ckpt_stride=64)
    torch.cuda.synchronize()
    assert not torch.isnan(S_big[:cap]).any()
    assert torch.isnan(S_big[cap:]).all()


def test_batched_equal_lengths():
    B, T, H, stride = 3, 700, 2, 128
    d = synth.prefill_inputs(4400, B * T, H, s0_std=0.02, n_seqs=B)
    say("case batched snapshots")
    q, k, v, z, beta, A, S0, _ = upload(d, "bf16", None)
    shp = (B, T, H, 128)
    S_ck = torch.zeros((B * (T // stride), H, 128, 128), device=DEV)
    kda.kda_chunk_fwd(q.view(shp), k.view(shp), v.view(shp), z.view(shp), beta.view(B, T, H), A, S0,
                      S_ckpt=S_ck, ckpt_stride=stride)
    torch.cuda.synchronize()
    ref = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"],
                           synth.cu_seqlens([T] * B), stride)
    assert err(S_ck.cpu().numpy(), ref) <= TOL["bf16"]


@pytest.mark.timeout(300)
def test_prefill_64k_snapshots_every_6144_tokens():
    """The 64K x 16 workload with a snapshot every 6,144 tokens (the physical cache-block size the
    review names): 10 snapshots, all compared with the oracle."""
    w = synth.WORKLOADS["prefill_64k"]
    T, H = 65536, 16
    d = synth.prefill_inputs(w["seed"], T, H, z_scale=w.get("z_scale", 2.0), s0_std=w.get("s0_std", 0.02))
    say("case prefill_64k snapshots stride 6144")
    q, k, v, z, beta, A, S0, _ = upload(d, "bf16", None)
    S_ck = torch.zeros((T // 6144, H, 128, 128), device=DEV)
    kda.kda_chunk_fwd(q, k, v, z, beta, A, S0, S_ckpt=S_ck, ckpt_stride=6144)
    torch.cuda.synchronize()
    ref = oracle.states_at(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], None, 6144)
    e = err(S_ck.cpu().numpy(), ref)
    say(f"  err_ckpt={e:.3e}")
    assert e <= TOL["bf16"], e
