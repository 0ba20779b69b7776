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


def host_pool_size():
    """Worker threads for host-side generation and the oracle (the GPU host's CPU share, at most 16)."""
    import os
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def upload_prefill_streamed(seed, T_total, H, z_scale=1.0, dtype="bf16"):
    """Generate the packed prefill inputs of a workload slice by slice on a thread pool and copy them
    into device tensors (q, k, v in the I/O dtype; z, beta fp32), never holding the whole input on the host."""
    from concurrent.futures import ThreadPoolExecutor

    import synth

    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.empty(T_total, H, 128, dtype=dt, device=DEV)
    k, v = torch.empty_like(q), torch.empty_like(q)
    z = torch.empty(T_total, H, 128, dtype=torch.float32, device=DEV)
    beta = torch.empty(T_total, H, dtype=torch.float32, device=DEV)
    starts = list(range(0, T_total, synth.SLICE))

    def gen(t0):
        return t0, synth.prefill_tokens(seed, t0, min(t0 + synth.SLICE, T_total), H, dtype, z_scale)

    n = host_pool_size()
    with ThreadPoolExecutor(n) as ex:
        for b in range(0, len(starts), 2 * n):  # a bounded window of slices in flight
            for t0, d in ex.map(gen, starts[b:b + 2 * n]):
                t1 = t0 + d["q"].shape[0]
                for name, dst in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta)):
                    dst[t0:t1].copy_(torch.from_numpy(d[name]).to(DEV, dst.dtype))
    return q, k, v, z, beta
