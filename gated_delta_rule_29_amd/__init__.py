"""MI355X-native Kimi Delta Attention (KDA) operator.

Thin ctypes binding over ``libkda.so`` (C ABI in ``include/kda.h``).  Every
step of the operator runs in the library's HIP kernels; this module only checks
tensor properties, allocates outputs / workspace through PyTorch and passes
raw device pointers and the current HIP stream.  There is no CPU fallback: if
the library is missing, every call raises.

    o, S_final = kda_chunk_fwd(q, k, v, g_raw, beta, A, S0=None, cu_seqlens=None)
    o = kda_decode_step(q, k, v, g_raw, beta, A, S)         # S updated in place

Operator (pages: "Kimi Linear: An Expressive, Efficient Attention Architecture"
summary, sections 3, 3.1 and 6.3; "Kimi K3 architecture", sequence-bottleneck
section): per head, S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
o_t = S_t^T q_t, a_t = exp(-5 * Sigmoid(exp(A_h) * z_t)).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_decode_step", "kda_chunk_fwd_workspace_bytes", "KDAError", "lib_path",
           "HEAD_DIM", "status_str", "load", "LayerOpts", "GATES"]

HEAD_DIM = 128
KDA_BF16, KDA_F32 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None


class KDAError(RuntimeError):
    pass


class LayerOpts(ctypes.Structure):
    """kda_layer_opts (include/kda.h): the KDA layer's steps fused into the prefill and decode, and
    the decay parameterisation."""
    _fields_ = [("qk_l2norm", ctypes.c_int32), ("qk_eps", ctypes.c_float), ("out_gate", ctypes.c_void_p),
                ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("gate_kind", ctypes.c_int32),
                ("gate_per_head", ctypes.c_int32), ("reverse_order", ctypes.c_int32), ("gate_u", ctypes.c_void_p),
                ("gate_w", ctypes.c_void_p), ("gate_rank", ctypes.c_int32)]


def _lowrank(gate_u, gate_w, rows, H, dev):
    """Check the low-rank forget gate factors: gate_u [rows, r] and gate_w [H, 128, r], bf16."""
    if gate_u is None and gate_w is None:
        return None, None, 0
    if gate_u is None or gate_w is None:
        raise ValueError("gate_u and gate_w go together")
    _need(gate_u, "gate_u", (torch.bfloat16,), dev)
    _need(gate_w, "gate_w", (torch.bfloat16,), dev)
    r = gate_u.shape[-1]
    if gate_u.numel() != rows * r or gate_w.shape != (H, HEAD_DIM, r):
        raise ValueError(f"gate_u must be [{rows}, r] and gate_w [{H}, {HEAD_DIM}, r]")
    return gate_u.data_ptr(), gate_w.data_ptr(), int(r)


GATES = {"k3": 0, "softplus": 1}  # kda_layer_opts::gate_kind


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise KDAError(f"{_LIB_PATH} is missing: build it with `python -m gated_delta_rule_29_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i64, i32, i32, ctypes.c_int]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, P, P,
                                  sz, P]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_timed.argtypes = lib.kda_chunk_fwd.argtypes + [P]
    lib.kda_chunk_fwd_noalloc.argtypes = lib.kda_chunk_fwd.argtypes[:17] + [P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_ckpt.argtypes = lib.kda_chunk_fwd.argtypes[:17] + [P, i64, i64] + lib.kda_chunk_fwd.argtypes[17:]
    lib.kda_chunk_fwd_ckpt.restype = ctypes.c_int
    lib.kda_chunk_fwd_layer.argtypes = (lib.kda_chunk_fwd.argtypes[:15] + [ctypes.POINTER(LayerOpts), P, P, P, i64, i64]
                                        + lib.kda_chunk_fwd.argtypes[17:])
    lib.kda_chunk_fwd_layer.restype = ctypes.c_int
    lib.kda_chunk_fwd_timed.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [P, P, P, ctypes.c_int, P, P, P, P, i32, i32, i32, i32, P, P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step_layer.argtypes = (lib.kda_decode_step.argtypes[:12] + [ctypes.POINTER(LayerOpts)]
                                          + lib.kda_decode_step.argtypes[12:])
    lib.kda_decode_step_layer.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().kda_status_str(int(status)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise KDAError(f"{what}: {status_str(rc)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_gpu(t, name="q"):
    """The kernels take device pointers: a host tensor would hand them host addresses."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")


def _keep_for(stream, *tensors):
    """Tensors this binding allocated were allocated for the current stream; when the library runs on
    another one, tell the caching allocator, so their memory is not reused before that work ends."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _out(t, name, shape, device):
    """A caller-supplied output: fp32, contiguous, on the inputs' device and exactly `shape` (the kernels
    write that many values into it)."""
    _need(t, name, (torch.float32,), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _need(t, name, dtypes, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kda_chunk_fwd_workspace_bytes(T_total: int, n_seqs: int, H: int, dtype=torch.bfloat16) -> int:
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load().kda_chunk_fwd_workspace_bytes(int(T_total), int(n_seqs), int(H), code))


def ckpt_count(lengths, stride: int) -> int:
    """Snapshot slots kda_chunk_fwd needs for sequences of these lengths: sum of len // stride."""
    return int(sum(int(n) // int(stride) for n in lengths))


def kda_chunk_fwd(q, k, v, g_raw, beta, A, S0=None, cu_seqlens=None, *, o=None, S_final=None,
                  workspace=None, stream=None, return_final_state=True, stage_events=None,
                  S_ckpt=None, ckpt_stride=0, qk_l2norm=False, qk_eps=1e-6, out_gate=None, norm_weight=None,
                  norm_eps=1e-6, gate="k3", gate_u=None, gate_w=None):
    """Chunkwise KDA prefill.

    q, k, v: [B, T, H, 128] (or [T, H, 128]) bf16 or fp32; g_raw: same shape fp32 (the gate's z);
    beta: [B, T, H] fp32; A: [H] fp32; S0: [N, H, 128, 128] fp32 or None (zeros);
    cu_seqlens: int32 device tensor [N+1] packing N sequences along T (then B must be 1).
    Returns (o [.., H, 128] fp32, S_final [N, H, 128, 128] fp32 or None).
    stage_events: optional ctypes array of six hipEvent_t recorded at the library's stage boundaries.
    S_ckpt, ckpt_stride: optional state snapshots (kda_chunk_fwd_ckpt): S_ckpt is an fp32 tensor
    [slots, H, 128, 128] (see ckpt_count), filled with the state after every ckpt_stride tokens of each
    sequence, sequence after sequence.
    qk_l2norm, out_gate, norm_weight (kda_chunk_fwd_layer): the KDA layer's steps fused in -- q and k
    given raw and normalised to unit length inside; o returned as RMSNorm(o) * norm_weight *
    sigmoid(out_gate) (out_gate: fp32, shaped like o; norm_weight: fp32 [128]).
    gate: "k3" (g = -5 Sigmoid(e^A z)) or "softplus" (g = -e^A softplus(z), unbounded); g_raw shaped
    [B, T, H] (or [T, H]) gives one gate value per (token, head) for all 128 channels.
    gate_u, gate_w: the forget gate's low-rank projection fused in, z[t, h, c] = sum_j gate_u[t, j]
    gate_w[h, c, j] (bf16, [tokens, r] and [H, 128, r], r a multiple of 32 up to 256); g_raw is then
    ignored and may be None.
    """
    lib = load()
    _on_gpu(q)
    squeeze = q.dim() == 3
    if g_raw is None and gate_u is None:
        raise ValueError("g_raw is required without gate_u / gate_w")
    if squeeze:
        q, k, v, beta = (x.unsqueeze(0) for x in (q, k, v, beta))
        g_raw = None if g_raw is None else g_raw.unsqueeze(0)
        if o is not None:
            _out(o, "o", (q.shape[1], q.shape[2], v.shape[-1]), q.device)
            o = o.unsqueeze(0)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128] or [T, H, 128]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    io = (torch.bfloat16, torch.float32)
    _need(q, "q", io, dev)
    _need(k, "k", (q.dtype,), dev)
    _need(v, "v", (q.dtype,), dev)
    lr_u, lr_w, lr_r = _lowrank(gate_u, gate_w, B * T, H, dev)
    if lr_u is not None:
        g_raw, per_head = None, False
    else:
        _need(g_raw, "g_raw", (torch.float32,), dev)
        per_head = g_raw.shape == q.shape[:3]
    _need(beta, "beta", (torch.float32,), dev)
    _need(A, "A", (torch.float32,), dev)
    if k.shape != q.shape or (g_raw is not None and g_raw.shape != q.shape and not per_head) \
            or v.shape[:3] != q.shape[:3] or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}")
    if A.shape != (H,):
        raise ValueError("A must be [H]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
        if B != 1:
            raise ValueError("cu_seqlens needs B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if S0 is not None:
        _need(S0, "S0", (torch.float32,), dev)
        if S0.shape != (N, H, dk, dv):
            raise ValueError(f"S0 must be [{N}, {H}, {dk}, {dv}]")
    mine = []  # tensors allocated here
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
        mine.append(o)
    else:
        _out(o, "o", (B, T, H, dv), dev)
    if S_final is not None:
        _out(S_final, "S_final", (N, H, dk, dv), dev)
    elif return_final_state:
        S_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        mine.append(S_final)
    dtype = KDA_BF16 if q.dtype == torch.bfloat16 else KDA_F32
    need = int(lib.kda_chunk_fwd_workspace_bytes(B * T, N, H, dtype))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        mine.append(workspace)
    else:
        _need(workspace, "workspace", (torch.uint8,), dev)
    args = (_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(g_raw), _ptr(beta), _ptr(A), _ptr(S0),
            _ptr(cu_seqlens), B, T, H, N, dk, dv, _ptr(o), _ptr(S_final), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    layer = qk_l2norm or out_gate is not None or gate != "k3" or per_head or lr_u is not None
    if S_ckpt is not None:
        _need(S_ckpt, "S_ckpt", (torch.float32,), dev)
        if S_ckpt.dim() != 4 or S_ckpt.shape[1:] != (H, dk, dv):
            raise ValueError(f"S_ckpt must be [slots, {H}, {dk}, {dv}]")
    if layer:
        if stage_events is not None:
            raise ValueError("stage_events and the fused layer steps cannot be combined")
        if out_gate is not None:
            _need(out_gate, "out_gate", (torch.float32,), dev)
            if norm_weight is None:
                raise ValueError("out_gate needs norm_weight")
            _need(norm_weight, "norm_weight", (torch.float32,), dev)
            if out_gate.numel() != B * T * H * dv or norm_weight.shape != (dv,):
                raise ValueError("out_gate must be shaped like o and norm_weight must be [128]")
        opts = LayerOpts(int(bool(qk_l2norm)), float(qk_eps), None if out_gate is None else out_gate.data_ptr(),
                         None if norm_weight is None else norm_weight.data_ptr(), float(norm_eps), GATES[gate],
                         int(per_head), 0, lr_u, lr_w, lr_r)
        ck = (_ptr(S_ckpt), int(ckpt_stride), S_ckpt.shape[0]) if S_ckpt is not None else (None, 0, 0)
        rc = lib.kda_chunk_fwd_layer(*args[:15], ctypes.byref(opts), args[15], args[16], *ck, *args[17:])
        _check(rc, "kda_chunk_fwd_layer")
    elif S_ckpt is not None:
        if stage_events is not None:
            raise ValueError("stage_events and S_ckpt cannot be combined")
        rc = lib.kda_chunk_fwd_ckpt(*args[:17], _ptr(S_ckpt), int(ckpt_stride), S_ckpt.shape[0], *args[17:])
        _check(rc, "kda_chunk_fwd_ckpt")
    elif stage_events is None:
        rc = lib.kda_chunk_fwd(*args)
        _check(rc, "kda_chunk_fwd")
    else:
        rc = lib.kda_chunk_fwd_timed(*args, ctypes.cast(stage_events, ctypes.c_void_p))
        _check(rc, "kda_chunk_fwd")
    _keep_for(stream, *mine)
    if squeeze:
        o = o.squeeze(0)
    return o, S_final


def kda_chunk_fwd_noalloc(q, k, v, g_raw, beta, A, o, S0=None, cu_seqlens=None, S_final=None, stream=None):
    """kda_chunk_fwd on the library's own device-resident workspace (kda_chunk_fwd_noalloc): nothing is
    allocated, so the caller passes o ([.., H, 128] fp32, shaped like v) and, if wanted, S_final
    ([N, H, 128, 128] fp32).  Problems larger than the workspace raise KDAError (KDA_ERR_WORKSPACE);
    calls that overlap on one GPU race.  Arguments are otherwise as kda_chunk_fwd."""
    lib = load()
    _on_gpu(q)
    if q.dim() == 3:
        q, k, v, beta, g_raw = (x.unsqueeze(0) for x in (q, k, v, beta, g_raw))
        o = o.unsqueeze(0)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128] or [T, H, 128]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (torch.bfloat16, torch.float32), dev)
    for t, name in ((k, "k"), (v, "v")):
        _need(t, name, (q.dtype,), dev)
    for t, name in ((g_raw, "g_raw"), (beta, "beta"), (A, "A"), (o, "o")):
        _need(t, name, (torch.float32,), dev)
    if k.shape != q.shape or g_raw.shape != q.shape or v.shape[:3] != q.shape[:3] or beta.shape != (B, T, H) \
            or A.shape != (H,) or o.shape != (B, T, H, dv):
        raise ValueError("inconsistent shapes")
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (torch.int32,), dev)
        N = cu_seqlens.numel() - 1
    for t, name in ((S0, "S0"), (S_final, "S_final")):
        if t is not None:
            _need(t, name, (torch.float32,), dev)
            if t.shape != (N, H, dk, dv):
                raise ValueError(f"{name} must be [{N}, {H}, {dk}, {dv}]")
    dtype = KDA_BF16 if q.dtype == torch.bfloat16 else KDA_F32
    rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(g_raw), _ptr(beta), _ptr(A), _ptr(S0),
                                   _ptr(cu_seqlens), B, T, H, N, dk, dv, _ptr(o), _ptr(S_final), _stream(stream))
    _check(rc, "kda_chunk_fwd_noalloc")


def kda_decode_step(q, k, v, g_raw, beta, A, S, *, o=None, stream=None, qk_l2norm=False, qk_eps=1e-6,
                    out_gate=None, norm_weight=None, norm_eps=1e-6, gate="k3", reverse_order=False, gate_u=None,
                    gate_w=None):
    """One recurrent step for N sequences: q, k, v [N, H, 128]; g_raw [N, H, 128] (or [N, H]: one
    value per head); beta [N, H]; A [H]; S [N, H, 128, 128] fp32 updated in place.  Returns o
    [N, H, 128] fp32.  qk_l2norm, out_gate, norm_weight, norm_eps, gate: as kda_chunk_fwd
    (kda_decode_step_layer).  reverse_order: visit the (sequence, head) states last to first (same
    results, same speed).
    gate_u [N, r], gate_w [H, 128, r]: the low-rank forget gate, as kda_chunk_fwd (g_raw may be None)."""
    lib = load()
    _on_gpu(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (torch.bfloat16, torch.float32), dev)
    _need(k, "k", (q.dtype,), dev)
    _need(v, "v", (q.dtype,), dev)
    lr_u, lr_w, lr_r = _lowrank(gate_u, gate_w, N, H, dev)
    if lr_u is not None:
        g_raw, per_head = None, False
    else:
        if g_raw is None:
            raise ValueError("g_raw is required without gate_u / gate_w")
        _need(g_raw, "g_raw", (torch.float32,), dev)
        per_head = g_raw.shape == (N, H)
    _need(beta, "beta", (torch.float32,), dev)
    _need(A, "A", (torch.float32,), dev)
    _need(S, "S", (torch.float32,), dev)
    if k.shape != q.shape or (g_raw is not None and g_raw.shape != q.shape and not per_head) \
            or beta.shape != (N, H) or S.shape != (N, H, dk, dv):
        raise ValueError("inconsistent shapes")
    if gate not in GATES:
        raise ValueError(f"gate must be one of {sorted(GATES)}")
    mine = None
    if o is None:
        o = mine = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    else:
        _out(o, "o", (N, H, dv), dev)
    dtype = KDA_BF16 if q.dtype == torch.bfloat16 else KDA_F32
    args = (_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(g_raw), _ptr(beta), _ptr(A), _ptr(S), N, H, dk, dv)
    if qk_l2norm or out_gate is not None or gate != "k3" or per_head or reverse_order or lr_u is not None:
        if out_gate is not None:
            _need(out_gate, "out_gate", (torch.float32,), dev)
            if norm_weight is None:
                raise ValueError("out_gate needs norm_weight")
            _need(norm_weight, "norm_weight", (torch.float32,), dev)
            if out_gate.numel() != N * H * dv or norm_weight.shape != (dv,):
                raise ValueError("out_gate must be shaped like o and norm_weight must be [128]")
        opts = LayerOpts(int(bool(qk_l2norm)), float(qk_eps), None if out_gate is None else out_gate.data_ptr(),
                         None if norm_weight is None else norm_weight.data_ptr(), float(norm_eps), GATES[gate],
                         int(per_head), int(bool(reverse_order)), lr_u, lr_w, lr_r)
        rc = lib.kda_decode_step_layer(*args, ctypes.byref(opts), _ptr(o), _stream(stream))
        _check(rc, "kda_decode_step_layer")
    else:
        rc = lib.kda_decode_step(*args, _ptr(o), _stream(stream))
        _check(rc, "kda_decode_step")
    _keep_for(stream, mine)
    return o
