"""CPU oracle for the Kimi Delta Attention (KDA) operator -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it; it
shares no code with the HIP path.

It wraps ``kda_oracle.c`` (plain C, float64), which follows:

* "Kimi K3 architecture" (molayo1419.me), section on the sequence bottleneck:
  the gate g = -5 * Sigmoid(e^{A_h} z), alpha = exp(g), and the 16-token tiles;
* "Kimi Linear: An Expressive, Efficient Attention Architecture" summary
  (greeksharifa.github.io), sections 2.1-3.1 and 6.2: the recurrence, the
  chunkwise WY/UT form, the dense DPLR transition, and the Gated DeltaNet rule.

Functions and what pins them (tests/test_oracle_pins.py):

* ``gate``            closed values of the logistic function, bounds;
* ``recurrent``       the reference for all parity: closed forms (beta = 0,
                      frozen state), associative recall with orthonormal keys,
                      the gradient step of the delta rule, the Gated DeltaNet
                      special case, brute force and the chunk form;
* ``recurrent_f32``   float32 twin, checked against ``recurrent``;
* ``states_at``       prefix-cache snapshots: one full-prefix run per snapshot,
                      the beta = 0 closed form, the slot order;
* ``recurrent_g``     the recurrence with given log-decays: equals ``recurrent``
                      with the K3 gate, the beta = 0 closed form;
* ``softplus_gate``   the unbounded decay: softplus closed values and limits;
* ``lowrank_z``       the forget gate's pre-activation from its low-rank
                      projection: one-hot and separable inputs;
* ``l2_normalize``, ``gated_rmsnorm``  the KDA layer's steps around the operator:
                      Pythagorean triples, constant vectors, the logistic
                      function's closed values and limits;
* ``chunk``/``chunk_step``  the chunk form, checked against ``recurrent``;
* ``bruteforce``      dense transition products, checked against ``recurrent``
                      and against the closed forms;
* ``gdn``             scalar-gate rule, checked against the beta = 0 closed form.

Every function has at least one pin that does not go through this library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

# x86-64-v3 (AVX2 + FMA) runs on every host CPU these GPUs are paired with.
CFLAGS = ["-O3", "-march=x86-64-v3", "-std=c11", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libkda_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.kdao_gate.argtypes = [P, i64, ctypes.c_float, P]
        lib.kdao_gate.restype = None
        lib.kdao_recurrent.argtypes = [P] * 8 + [i32] * 4 + [P, P, i32]
        lib.kdao_recurrent.restype = i32
        lib.kdao_recurrent_g.argtypes = [P] * 7 + [i32] * 4 + [P, P, i32]
        lib.kdao_recurrent_g.restype = i32
        lib.kdao_recurrent_f32.argtypes = [P] * 8 + [i32] * 4 + [P, P, i32]
        lib.kdao_recurrent_f32.restype = i32
        lib.kdao_chunk.argtypes = [P] * 8 + [i32] * 7 + [P, P, i32]
        lib.kdao_chunk.restype = i32
        lib.kdao_chunk_step.argtypes = ([P] * 5 + [i64, i64, ctypes.c_float] + [i32] * 5
                                        + [P, P, i64] + [P] * 7)
        lib.kdao_chunk_step.restype = None
        lib.kdao_bruteforce.argtypes = [P] * 5 + [ctypes.c_float, P] + [i32] * 3 + [P, P]
        lib.kdao_bruteforce.restype = i32
        lib.kdao_gdn.argtypes = [P] * 6 + [i32] * 3 + [P, P]
        lib.kdao_gdn.restype = None
        _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    return np.ascontiguousarray(cu_seqlens, dtype=np.int64)


def gate(z, A: float) -> np.ndarray:
    """g = -5 * Sigmoid(e^A * z) in float64, elementwise over z."""
    z = _f32(z)
    g = np.empty(z.shape, dtype=np.float64)
    _load().kdao_gate(_ptr(z), z.size, float(A), _ptr(g))
    return g


def recurrent(q, k, v, z, beta, A, S0=None, cu_seqlens=None, threads: int = 0, return_threads=False):
    """Token-by-token KDA recurrence in float64.

    q, k, z: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; A: [H]; S0: [N, H, dk, dv] or None;
    cu_seqlens: [N+1] offsets (None: one sequence).  Returns (o [T,H,dv], S_final [N,H,dk,dv]).
    """
    q, k, v, z, beta, A = map(_f32, (q, k, v, z, beta, A))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = len(cu) - 1
    S0d = None if S0 is None else _f64(S0)
    o = np.zeros((T, H, dv), dtype=np.float64)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    n = _load().kdao_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A), _ptr(S0d),
                               _ptr(cu), N, H, dk, dv, _ptr(o), _ptr(Sf), int(threads))
    return (o, Sf, n) if return_threads else (o, Sf)


def recurrent_g(q, k, v, g, beta, S0=None, cu_seqlens=None, threads: int = 0):
    """The recurrence with the log-decays given directly: g [T, H, dk] float64, alpha = e^g
    (for decay parameterisations other than the K3 gate).  Same outputs as ``recurrent``."""
    q, k, v, beta = map(_f32, (q, k, v, beta))
    g = _f64(g)
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = len(cu) - 1
    S0d = None if S0 is None else _f64(S0)
    o = np.zeros((T, H, dv), dtype=np.float64)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    _load().kdao_recurrent_g(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0d), _ptr(cu), N, H, dk, dv,
                             _ptr(o), _ptr(Sf), int(threads))
    return o, Sf


def softplus_gate(z, A):
    """Kimi Linear's unbounded negative-softplus decay, the parameterisation K3 replaces (Kimi K3
    paper review, Method paragraph; the Kimi K3 architecture page, sequence-bottleneck section).
    Reading: g = -e^{A_h} * softplus(z), per (token, head, key channel), in float64; z: [T, H, dk],
    A: [H].  softplus is evaluated as max(z, 0) + log1p(e^{-|z|})."""
    z = np.asarray(z, dtype=np.float64)
    sp = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    return -np.exp(np.asarray(A, dtype=np.float64))[None, :, None] * sp


def recurrent_f32(q, k, v, z, beta, A, S0=None, cu_seqlens=None, threads: int = 0):
    """The same recurrence in float32 arithmetic (noise-floor reference)."""
    q, k, v, z, beta, A = map(_f32, (q, k, v, z, beta, A))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = len(cu) - 1
    S0f = None if S0 is None else _f32(S0)
    o = np.zeros((T, H, dv), dtype=np.float32)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float32)
    _load().kdao_recurrent_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A), _ptr(S0f),
                               _ptr(cu), N, H, dk, dv, _ptr(o), _ptr(Sf), int(threads))
    return o, Sf


def states_at(q, k, v, z, beta, A, S0=None, cu_seqlens=None, stride: int = 64, threads: int = 0):
    """State snapshots for a prefix cache (Kimi K3 paper review, Significance and
    Limitations paragraphs: the KDA state is checkpointed at sparse boundaries).

    Snapshot m of sequence n is the state after the sequence's first (m + 1) * stride
    tokens, for m < len_n // stride; the snapshots of all sequences follow one another
    in sequence order.  Returns an array [slots, H, dk, dv] in float64.  Each snapshot
    is the recurrence run over the next stride tokens from the previous snapshot (the
    state is all the recurrence carries from one token to the next).
    """
    q, k, v, z, beta, A = map(_f32, (q, k, v, z, beta, A))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = len(cu) - 1
    out = []
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        S = np.zeros((1, H, dk, dv)) if S0 is None else _f64(S0)[n:n + 1]
        for m in range((b - a) // stride):
            t0, t1 = a + m * stride, a + (m + 1) * stride
            _, S = recurrent(q[t0:t1], k[t0:t1], v[t0:t1], z[t0:t1], beta[t0:t1], A, S0=S, threads=threads)
            out.append(S[0])
    return np.array(out, dtype=np.float64).reshape(len(out), H, dk, dv)


def decode_step(q, k, v, z, beta, A, S, threads: int = 0):
    """One recurrent step for N sequences: q, k, v, z [N, H, d]; beta [N, H]; S [N, H, d, d].

    Returns (o [N, H, dv], S_new); the decode step is the recurrence applied to one token
    per sequence ([KL 6.3]: generation uses the recurrent update)."""
    N = q.shape[0]
    return recurrent(q, k, v, z, beta, A, S0=S, cu_seqlens=np.arange(N + 1), threads=threads)


def chunk(q, k, v, z, beta, A, S0=None, cu_seqlens=None, C: int = 64, sub: int = 16,
          shaped: bool = True, threads: int = 0):
    """Chunk form (WY/UT, forward substitution) in float64; same arguments as ``recurrent``."""
    q, k, v, z, beta, A = map(_f32, (q, k, v, z, beta, A))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = len(cu) - 1
    S0d = None if S0 is None else _f64(S0)
    o = np.zeros((T, H, dv), dtype=np.float64)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kdao_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A), _ptr(S0d),
                            _ptr(cu), N, H, dk, dv, int(C), int(sub), int(bool(shaped)),
                            _ptr(o), _ptr(Sf), int(threads))
    if rc < 0:
        raise ValueError("chunk form needs dk == dv, C >= 1, sub >= 1")
    return o, Sf


def chunk_step(q, k, v, z, beta, A: float, S, sub: int = 16, shaped: bool = True) -> dict:
    """One chunk of one head with every intermediate exposed.

    q, k, v, z: [n, d]; beta: [n]; S: [dk, dv] incoming state.  Returns a dict with
    G, Akk, T, W, U, Aqk, Delta, o and S (the outgoing state)."""
    q, k, v, z, beta = map(_f32, (q, k, v, z, beta))
    n, dk = q.shape
    dv = v.shape[1]
    if dk != dv:
        raise ValueError("dk == dv required")
    S = _f64(S).copy()
    out = {name: np.zeros(shape, dtype=np.float64) for name, shape in
           [("G", (n, dk)), ("Akk", (n, n)), ("T", (n, n)), ("W", (n, dk)), ("U", (n, dv)),
            ("Aqk", (n, n)), ("Delta", (n, dv)), ("o", (n, dv))]}
    _load().kdao_chunk_step(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), dk, 1, float(A), n, dk, dv,
                            int(sub), int(bool(shaped)), _ptr(S), _ptr(out["o"]), dv, _ptr(out["G"]),
                            _ptr(out["Akk"]), _ptr(out["T"]), _ptr(out["W"]), _ptr(out["U"]),
                            _ptr(out["Aqk"]), _ptr(out["Delta"]))
    out["S"] = S
    return out


def bruteforce(q, k, v, z, beta, A: float, S0=None):
    """Dense transition-product expansion, one head: q, k, z [T, dk]; v [T, dv]; beta [T]."""
    q, k, v, z, beta = map(_f32, (q, k, v, z, beta))
    T, dk = q.shape
    dv = v.shape[1]
    S0d = None if S0 is None else _f64(S0)
    o = np.zeros((T, dv), dtype=np.float64)
    Sf = np.zeros((dk, dv), dtype=np.float64)
    if _load().kdao_bruteforce(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), float(A), _ptr(S0d),
                               T, dk, dv, _ptr(o), _ptr(Sf)) != 0:
        raise ValueError("brute force supports T <= 64")
    return o, Sf


def gdn(q, k, v, alpha, beta, S0=None):
    """Gated DeltaNet with a scalar gate per token, one head: alpha, beta [T]."""
    q, k, v, beta = map(_f32, (q, k, v, beta))
    alpha = _f64(alpha)
    T, dk = q.shape
    dv = v.shape[1]
    S0d = None if S0 is None else _f64(S0)
    o = np.zeros((T, dv), dtype=np.float64)
    Sf = np.zeros((dk, dv), dtype=np.float64)
    _load().kdao_gdn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0d), T, dk, dv,
                     _ptr(o), _ptr(Sf))
    return o, Sf


def l2_normalize(x, eps: float = 1e-6):
    """The unit-length step the KDA layer applies to queries and keys before the operator
    (Kimi Linear summary, section 4): x / sqrt(sum_j x_j^2 + eps) over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gated_rmsnorm(o, gate, weight, eps: float = 1e-6):
    """The output steps of the KDA layer (Kimi Linear summary, section 4): a per-head RMSNorm
    over the value channels, then a data-dependent sigmoid gate.  o, gate: [..., dv];
    weight: [dv].  Returns o / sqrt(mean_j o_j^2 + eps) * weight * sigmoid(gate), in float64."""
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * np.asarray(weight, dtype=np.float64) * (1.0 / (1.0 + np.exp(-g)))


def lowrank_z(u, W):
    """The forget gate's pre-activation from its low-rank projection (Kimi Linear summary,
    section 4: the forget and output gates use low-rank projections).  Reading: the second
    factor of the projection maps a rank-r vector per token, shared by all heads, to every
    head's 128 key channels: z[t, h, c] = sum_j u[t, j] * W[h, c, j], in float64.
    u: [T, r]; W: [H, 128, r].  Returns z: [T, H, 128]."""
    u = np.asarray(u, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    H, dk, r = W.shape
    return (u @ W.reshape(H * dk, r).T).reshape(u.shape[0], H, dk)
