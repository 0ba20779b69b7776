"""Helpers shared by the GPU parity tests: upload seeded inputs, call the
library through its binding, compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import gated_delta_rule_29_amd as kda

DEV = "cuda:0"


def say(*a):
    """Name the case before each GPU step (flushed, so a fault still leaves a trace)."""
    print(*a, flush=True)
    sys.stdout.flush()


def err(a, ref):
    """max |a - ref| / RMS(ref) over the compared elements."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(a - ref)) / max(rms, 1e-300))


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=dtype)


def run_prefill(d, cu=None, S0=None, io="bf16", S_final_alias=False):
    """Run kda_chunk_fwd on host inputs d (q,k,v,z [T,H,128], beta [T,H], A [H]); returns numpy o, S_final."""
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    q, k, v = (to_dev(d[n], dt) for n in ("q", "k", "v"))
    z, beta, A = to_dev(d["z"], torch.float32), to_dev(d["beta"], torch.float32), to_dev(d["A"], torch.float32)
    cu_t = None if cu is None else to_dev(np.asarray(cu, np.int32), torch.int32)
    S0_t = None if S0 is None else to_dev(S0, torch.float32)
    if S_final_alias:
        o, Sf = kda.kda_chunk_fwd(q, k, v, z, beta, A, S0_t, cu_t, S_final=S0_t)
    else:
        o, Sf = kda.kda_chunk_fwd(q, k, v, z, beta, A, S0_t, cu_t)
    torch.cuda.synchronize()
    return o.cpu().numpy(), Sf.cpu().numpy()
