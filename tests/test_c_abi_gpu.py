"""The C ABI driven with plain HIP device memory: buffers from hipMalloc, inputs and outputs moved
with hipMemcpy, the library's entry points called with raw pointers through ctypes.  No torch
tensor takes part, so this checks that libkda.so stands on its header alone (the binding's own
memory handling is tested elsewhere).  A packed prefill (bf16 q/k/v, ragged lengths) and one
decode step are compared with the fp64 oracle; bar max|d| / RMS <= 1e-2."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import err, say

import gated_delta_rule_29_amd as kda

pytestmark = pytest.mark.gpu

H2D, D2H = 1, 2  # hipMemcpyHostToDevice, hipMemcpyDeviceToHost


class Hip:
    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
        self.rt.hipFree.argtypes = [ctypes.c_void_p]
        self.rt.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        self.rt.hipDeviceSynchronize.argtypes = []
        self.bufs = []

    def ok(self, rc, what):
        assert rc == 0, f"{what} returned {rc}"

    def alloc(self, nbytes):
        p = ctypes.c_void_p()
        self.ok(self.rt.hipMalloc(ctypes.byref(p), max(int(nbytes), 1)), "hipMalloc")
        self.bufs.append(p)
        return p

    def put(self, a):
        a = np.ascontiguousarray(a)
        p = self.alloc(a.nbytes)
        self.ok(self.rt.hipMemcpy(p, a.ctypes.data_as(ctypes.c_void_p), a.nbytes, H2D), "hipMemcpy H2D")
        return p

    def get(self, p, shape, dtype):
        out = np.empty(shape, dtype)
        self.ok(self.rt.hipMemcpy(out.ctypes.data_as(ctypes.c_void_p), p, out.nbytes, D2H), "hipMemcpy D2H")
        return out

    def sync(self):
        self.ok(self.rt.hipDeviceSynchronize(), "hipDeviceSynchronize")

    def free(self):
        for p in self.bufs:
            self.rt.hipFree(p)
        self.bufs = []


def bf16_bits(x):
    """float32 values that are bf16-representable -> their bf16 bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    assert not np.any(u & 0xFFFF), "inputs must already be rounded to bf16"
    return (u >> 16).astype(np.uint16)


def test_prefill_and_decode_on_plain_hip_memory():
    lib = kda.load()
    hip = Hip()
    try:
        lens = [300, 64, 1, 190]
        cu = synth.cu_seqlens(lens)
        T, H, N = int(cu[-1]), 4, len(lens)
        d = synth.prefill_inputs(8300, T, H, dtype="bf16", z_scale=1.5, s0_std=0.02, n_seqs=N)
        say(f"case plain-HIP prefill lens={lens} H={H}")
        q, k, v = (hip.put(bf16_bits(d[n])) for n in ("q", "k", "v"))
        z, beta, A, S0 = (hip.put(d[n].astype(np.float32)) for n in ("z", "beta", "A", "S0"))
        cu_d = hip.put(np.asarray(cu, np.int32))
        o = hip.alloc(T * H * 128 * 4)
        Sf = hip.alloc(N * H * 128 * 128 * 4)
        wsb = lib.kda_chunk_fwd_workspace_bytes(T, N, H, 0)
        assert wsb > 0
        ws = hip.alloc(wsb)
        rc = lib.kda_chunk_fwd(q, k, v, 0, z, beta, A, S0, cu_d, 1, T, H, N, 128, 128, o, Sf, ws, wsb, None)
        assert rc == 0, lib.kda_status_str(rc)
        hip.sync()
        o_h = hip.get(o, (T, H, 128), np.float32)
        S_h = hip.get(Sf, (N, H, 128, 128), np.float32)
        o_ref, S_ref = oracle.recurrent(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"], cu)
        eo, es = err(o_h, o_ref), err(S_h, S_ref)
        say(f"  prefill err_o={eo:.3e} err_S={es:.3e}")
        assert eo <= 1e-2 and es <= 1e-2

        # one decode step from the prefill's final states, in place
        x = synth.decode_tokens(8301, 0, N, H)
        say(f"case plain-HIP decode N={N} H={H}")
        qd, kd, vd = (hip.put(bf16_bits(x[n])) for n in ("q", "k", "v"))
        zd, bd = hip.put(x["z"].astype(np.float32)), hip.put(x["beta"].astype(np.float32))
        od = hip.alloc(N * H * 128 * 4)
        rc = lib.kda_decode_step(qd, kd, vd, 0, zd, bd, A, Sf, N, H, 128, 128, od, None)
        assert rc == 0, lib.kda_status_str(rc)
        hip.sync()
        od_h = hip.get(od, (N, H, 128), np.float32)
        Sd_h = hip.get(Sf, (N, H, 128, 128), np.float32)
        od_ref, Sd_ref = oracle.decode_step(x["q"], x["k"], x["v"], x["z"], x["beta"], d["A"], S_h)
        e1, e2 = err(od_h, od_ref), err(Sd_h, Sd_ref)
        say(f"  decode err_o={e1:.3e} err_S={e2:.3e}")
        assert e1 <= 1e-2 and e2 <= 1e-2
    finally:
        hip.free()
