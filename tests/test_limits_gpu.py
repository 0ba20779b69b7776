"""GPU parity at the largest head count the prefill accepts (KDA_MAX_HEADS = 16,384 heads).

A chunk's rows of one input then span 64 x H x 512 B, the most the kernels address with 32-bit
buffer offsets.  T = 77 gives each head a full chunk and a ragged one.  Heads are independent, so
the fp64 oracle runs on a seeded sample of heads alone and is compared with those heads of the
GPU result.  Bar: max|d| / RMS(ref) <= 1e-2 (bf16 q/k/v) or 1e-4 (fp32 q/k/v)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import err, say, to_dev

import gated_delta_rule_29_amd as kda

pytestmark = pytest.mark.gpu

MAX_HEADS = 16384  # KDA_MAX_HEADS in include/kda.h
TOL = {"bf16": 1e-2, "f32": 1e-4}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prefill_at_the_head_limit(io):
    T, H = 77, MAX_HEADS
    say(f"case head limit io={io} T={T} H={H}: generating")
    d = synth.prefill_inputs(8100, T, H, dtype=io, z_scale=1.5, s0_std=0.02, slice_tokens=T)  # T rows drawn, not 4096
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v = (to_dev(d[n], dt) for n in ("q", "k", "v"))
    say(f"case head limit io={io}: GPU call")
    o, Sf = kda.kda_chunk_fwd(q, k, v, to_dev(d["z"], torch.float32), to_dev(d["beta"], torch.float32),
                              to_dev(d["A"], torch.float32), to_dev(d["S0"], torch.float32))
    torch.cuda.synchronize()
    heads = np.sort(np.concatenate([[0, 1, H // 2, H - 1], np.random.default_rng(8101).choice(H, 8, replace=False)]))
    hidx = torch.as_tensor(heads, device=o.device)
    o_h = o.index_select(1, hidx).cpu().numpy()
    S_h = Sf.index_select(1, hidx).cpu().numpy()
    del q, k, v, o, Sf
    sub = {n: np.ascontiguousarray(d[n][:, heads]) for n in ("q", "k", "v", "z", "beta", "S0")}
    o_ref, S_ref = oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["z"], sub["beta"], d["A"][heads], sub["S0"])
    eo, es = err(o_h, o_ref), err(S_h, S_ref)
    say(f"  heads {heads.tolist()}: err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= TOL[io] and es <= TOL[io]


def test_one_head_more_is_rejected():
    t = torch.empty((1, 64, MAX_HEADS + 1, 128), dtype=torch.bfloat16, device="cuda:0")
    z = torch.empty((1, 64, MAX_HEADS + 1, 128), device="cuda:0")
    beta, A = torch.empty((1, 64, MAX_HEADS + 1), device="cuda:0"), torch.zeros(MAX_HEADS + 1, device="cuda:0")
    say("case head limit + 1: rejected before any launch")
    with pytest.raises(kda.KDAError):
        kda.kda_chunk_fwd(t, t, t, z, beta, A)
