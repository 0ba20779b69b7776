"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/kda.h declares, and rejects bad arguments with the documented
status codes before any HIP call."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_29_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, DTYPE, SEQLENS, ALIGN, WORKSPACE, HIP, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_bytes", "kda_status_str",
              "kda_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kda.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = kda.load()
    for code in (OK, NULL, SHAPE, DTYPE, SEQLENS, ALIGN, WORKSPACE, HIP, ALIAS):
        s = lib.kda_status_str(code).decode()
        assert s.startswith("KDA_")
    assert "UNKNOWN" in lib.kda_status_str(12345).decode()
    assert lib.kda_version() >= 100


def test_workspace_size():
    lib = kda.load()
    for dt in (0, 1):
        assert lib.kda_chunk_fwd_workspace_bytes(0, 0, 16, dt) == 0
        assert lib.kda_chunk_fwd_workspace_bytes(-1, 1, 16, dt) == 0
        a = lib.kda_chunk_fwd_workspace_bytes(65536, 1, 16, dt)
        b = lib.kda_chunk_fwd_workspace_bytes(4 * 65536, 1, 16, dt)
        assert a > 0 and b >= a
        assert lib.kda_chunk_fwd_workspace_bytes(64, 1, 2, dt) > lib.kda_chunk_fwd_workspace_bytes(64, 1, 1, dt)
    assert lib.kda_chunk_fwd_workspace_bytes(64, 1, 1, 9) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(64, 1, 16384, 0) > 0  # KDA_MAX_HEADS
    assert lib.kda_chunk_fwd_workspace_bytes(64, 1, 16385, 0) == 0
    # both paths keep one block of chain operands per (chunk, head): the size grows with ceil(T/64) + N
    for dt in (0, 1):
        assert lib.kda_chunk_fwd_workspace_bytes(65, 1, 1, dt) > lib.kda_chunk_fwd_workspace_bytes(64, 1, 1, dt)
        per_chunk_head = lib.kda_chunk_fwd_workspace_bytes(64 * 4096, 1, 16, dt) / (4097 * 16)
        assert 64 * 1024 < per_chunk_head < 192 * 1024


# Fake, 256-aligned, non-overlapping "device" addresses: validation must fail
# before any of them is dereferenced or handed to HIP.
BASE = 1 << 40


def fake(i, off=0):
    return ctypes.c_void_p(BASE + (i << 32) + off)


def prefill_args(**kw):
    a = dict(q=fake(1), k=fake(2), v=fake(3), dtype=0, z=fake(4), beta=fake(5), A=fake(6), S0=fake(7),
             cu=None, B=1, T=128, H=2, N=1, dk=128, dv=128, o=fake(8), Sf=fake(9), ws=fake(10),
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return a


def call_prefill(a):
    lib = kda.load()
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["beta"], a["A"], a["S0"], a["cu"],
                             a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"], a["o"], a["Sf"], a["ws"],
                             a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dk=64), SHAPE), (dict(dv=256), SHAPE), (dict(T=-1), SHAPE), (dict(H=-2), SHAPE),
    (dict(H=16385), SHAPE), (dict(dtype=7), DTYPE),
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(z=None), NULL),
    (dict(beta=None), NULL), (dict(A=None), NULL), (dict(o=None), NULL),
    (dict(N=2), SEQLENS), (dict(cu=fake(11), B=2, N=2), SEQLENS), (dict(cu=fake(11), N=0), SEQLENS),
    (dict(q=fake(1, 8)), ALIGN), (dict(Sf=fake(9, 4)), ALIGN), (dict(ws=fake(10, 2)), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1000), WORKSPACE),
    (dict(o=fake(1, 64)), ALIAS), (dict(o=fake(7)), ALIAS), (dict(o=fake(10, 4096)), ALIAS),
])
def test_prefill_rejects(kw, code):
    assert call_prefill(prefill_args(**kw)) == code


def test_prefill_empty_problem_is_ok_without_gpu():
    assert call_prefill(prefill_args(B=0, N=0, T=0)) == OK
    assert call_prefill(prefill_args(H=0)) == OK


def call_prefill_ckpt(a, S_ckpt=fake(12), stride=128, cap=4):
    lib = kda.load()
    return lib.kda_chunk_fwd_ckpt(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["beta"], a["A"], a["S0"], a["cu"],
                                  a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"], a["o"], a["Sf"], S_ckpt,
                                  stride, cap, a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("ck,code", [
    (dict(S_ckpt=None), NULL), (dict(stride=0), SHAPE), (dict(stride=100), SHAPE), (dict(stride=-64), SHAPE),
    (dict(cap=-1), SHAPE), (dict(S_ckpt=fake(12, 8)), ALIGN),
    (dict(S_ckpt=fake(8)), ALIAS), (dict(S_ckpt=fake(7, 65536)), ALIAS), (dict(S_ckpt=fake(10, 256)), ALIAS),
    (dict(S_ckpt=fake(1, 1024)), ALIAS),
])
def test_prefill_ckpt_rejects(ck, code):
    assert call_prefill_ckpt(prefill_args(), **ck) == code


def test_prefill_ckpt_checks_the_plain_arguments_too():
    assert call_prefill_ckpt(prefill_args(dk=64)) == SHAPE
    assert call_prefill_ckpt(prefill_args(ws=None)) == WORKSPACE
    assert call_prefill_ckpt(prefill_args(B=0, N=0, T=0)) == OK


Opts = kda.LayerOpts


def call_prefill_layer(a, opts, S_ckpt=None, stride=0, cap=0):
    lib = kda.load()
    return lib.kda_chunk_fwd_layer(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["beta"], a["A"], a["S0"],
                                   a["cu"], a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"],
                                   None if opts is None else ctypes.byref(opts), a["o"], a["Sf"], S_ckpt, stride,
                                   cap, a["ws"], a["ws_bytes"], a["stream"])


def test_prefill_layer_rejects():
    gate, w = fake(13).value, fake(14).value
    assert call_prefill_layer(prefill_args(), None) == NULL
    assert call_prefill_layer(prefill_args(), Opts(1, 1e-6, gate, None, 1e-6)) == NULL
    assert call_prefill_layer(prefill_args(), Opts(1, -1.0, None, None, 0.0)) == SHAPE
    assert call_prefill_layer(prefill_args(), Opts(0, 0.0, gate, w, float("nan"))) == SHAPE
    assert call_prefill_layer(prefill_args(), Opts(0, 0.0, gate + 4, w, 0.0)) == ALIGN
    assert call_prefill_layer(prefill_args(o=fake(13, 256)), Opts(0, 0.0, gate, w, 0.0)) == ALIAS
    assert call_prefill_layer(prefill_args(), Opts(0, 0.0, gate, w, 0.0), S_ckpt=fake(12), stride=100,
                              cap=1) == SHAPE
    assert call_prefill_layer(prefill_args(B=0, N=0, T=0), Opts(1, 1e-6, gate, w, 1e-6)) == OK


def test_prefill_gate_options_are_checked():
    gate, w = fake(13).value, fake(14).value
    for kind in (-1, 2, 7):
        assert call_prefill_layer(prefill_args(), Opts(0, 0.0, None, None, 0.0, kind, 0)) == SHAPE
    # g_raw spans [tokens, H, 128] floats, or [tokens, H] with the per-head gate (256 tokens x heads here)
    assert call_prefill_layer(prefill_args(o=fake(4, 2048)), Opts(0, 0.0, None, None, 0.0, 1, 0)) == ALIAS
    assert call_prefill_layer(prefill_args(o=fake(4, 512)), Opts(0, 0.0, None, None, 0.0, 1, 1)) == ALIAS
    assert call_prefill_layer(prefill_args(B=0, N=0, T=0), Opts(0, 0.0, gate, w, 0.0, 1, 1)) == OK
    # reverse_order is a decode option
    assert call_prefill_layer(prefill_args(B=0, N=0, T=0), Opts(0, 0.0, None, None, 0.0, 0, 0, 1)) == SHAPE


def test_prefill_lowrank_gate_options_are_checked():
    u, w = fake(15).value, fake(16).value
    # rank: a multiple of 32 in [32, 256]; not with the per-head gate
    for r in (0, 16, 48, 288):
        assert call_prefill_layer(prefill_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, w, r)) == SHAPE
    assert call_prefill_layer(prefill_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 1, 0, u, w, 64)) == SHAPE
    assert call_prefill_layer(prefill_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, None, 64)) == NULL
    assert call_prefill_layer(prefill_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u + 2, w, 64)) == ALIGN
    assert call_prefill_layer(prefill_args(o=fake(15, 256)), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, w, 64)) == ALIAS
    assert call_prefill_layer(prefill_args(o=fake(16, 256)), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, w, 64)) == ALIAS
    # without the factors g_raw is required
    assert call_prefill_layer(prefill_args(z=None), Opts(0, 0.0, None, None, 0.0)) == NULL
    assert call_prefill_layer(prefill_args(z=None, B=0, N=0, T=0),
                              Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, w, 128)) == OK


def test_ckpt_count():
    assert kda.ckpt_count([0, 63, 64, 6143, 6144, 20000], 6144) == 0 + 0 + 0 + 0 + 1 + 3
    assert kda.ckpt_count([128, 129, 255, 256], 128) == 1 + 1 + 1 + 2


def decode_args(**kw):
    a = dict(q=fake(1), k=fake(2), v=fake(3), dtype=0, z=fake(4), beta=fake(5), A=fake(6), S=fake(7), N=4, H=2,
             dk=128, dv=128, o=fake(8), stream=None)
    a.update(kw)
    return a


def call_decode(a):
    lib = kda.load()
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["beta"], a["A"], a["S"], a["N"],
                               a["H"], a["dk"], a["dv"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dk=127), SHAPE), (dict(N=-1), SHAPE), (dict(dtype=-1), DTYPE),
    (dict(S=None), NULL), (dict(o=None), NULL), (dict(A=None), NULL),
    (dict(S=fake(7, 4)), ALIGN), (dict(o=fake(7, 256)), ALIAS), (dict(o=fake(3)), ALIAS),
])
def test_decode_rejects(kw, code):
    assert call_decode(decode_args(**kw)) == code


def test_decode_empty_is_ok_without_gpu():
    assert call_decode(decode_args(N=0)) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(kda.KDAError):
        kda.load()


def call_decode_layer(a, opts):
    lib = kda.load()
    return lib.kda_decode_step_layer(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["beta"], a["A"], a["S"],
                                     a["N"], a["H"], a["dk"], a["dv"], None if opts is None else ctypes.byref(opts),
                                     a["o"], a["stream"])


def test_decode_layer_rejects():
    gate, w = fake(13).value, fake(14).value
    assert call_decode_layer(decode_args(), None) == NULL
    assert call_decode_layer(decode_args(), Opts(0, 0.0, gate, None, 0.0)) == NULL
    assert call_decode_layer(decode_args(), Opts(0, -1.0, None, None, 0.0)) == SHAPE
    assert call_decode_layer(decode_args(), Opts(0, 0.0, None, None, 0.0, 5, 0)) == SHAPE
    assert call_decode_layer(decode_args(), Opts(0, 0.0, gate + 8, w, 0.0)) == ALIGN
    assert call_decode_layer(decode_args(o=fake(13, 256)), Opts(0, 0.0, gate, w, 0.0)) == ALIAS
    # g_raw is [N, H] floats with the per-head gate (8 values here), [N, H, 128] otherwise
    assert call_decode_layer(decode_args(o=fake(4, 1024)), Opts(0, 0.0, None, None, 0.0, 0, 0)) == ALIAS
    assert call_decode_layer(decode_args(o=fake(4, 16)), Opts(0, 0.0, None, None, 0.0, 0, 1)) == ALIAS
    assert call_decode_layer(decode_args(N=0), Opts(1, 1e-6, gate, w, 1e-6, 1, 1)) == OK
    u, wl = fake(15).value, fake(16).value
    assert call_decode_layer(decode_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, wl, 40)) == SHAPE
    assert call_decode_layer(decode_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, None, wl, 64)) == NULL
    assert call_decode_layer(decode_args(z=None), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, None, 64)) == NULL
    assert call_decode_layer(decode_args(o=fake(15, 64)), Opts(0, 0.0, None, None, 0.0, 0, 0, 0, u, wl, 64)) == ALIAS


def call_prefill_noalloc(a):
    lib = kda.load()
    return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["beta"], a["A"], a["S0"],
                                     a["cu"], a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"], a["o"], a["Sf"],
                                     a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dk=64), SHAPE), (dict(dtype=7), DTYPE), (dict(q=None), NULL), (dict(N=2), SEQLENS),
    (dict(q=fake(1, 8)), ALIGN), (dict(o=fake(1, 64)), ALIAS),
    # more than the library's own workspace holds: rejected before any HIP call
    (dict(T=8192, H=16), WORKSPACE), (dict(T=4096, H=16, dtype=1), WORKSPACE),
])
def test_prefill_noalloc_rejects(kw, code):
    assert call_prefill_noalloc(prefill_args(**kw)) == code


def test_prefill_noalloc_limit_matches_the_header():
    text = open(HEADER).read()
    limit = int(re.search(r"#define KDA_NOALLOC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", text).group(1)) << 20
    lib = kda.load()
    assert lib.kda_chunk_fwd_workspace_bytes(4544, 1, 16, 0) <= limit < lib.kda_chunk_fwd_workspace_bytes(4608, 1, 16, 0)
    assert call_prefill_noalloc(prefill_args(B=0, N=0, T=0)) == OK


def test_binding_refuses_host_tensors():
    """Host tensors would hand host addresses to the kernels: the binding refuses them first."""
    import torch
    q = torch.zeros(64, 2, 128, dtype=torch.bfloat16)
    z, beta, A = torch.zeros(64, 2, 128), torch.zeros(64, 2), torch.zeros(2)
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_chunk_fwd(q, q, q, z, beta, A)
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_chunk_fwd_noalloc(q, q, q, z, beta, A, torch.zeros(64, 2, 128))
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_decode_step(q[:4], q[:4], q[:4], z[:4], beta[:4], A, torch.zeros(4, 2, 128, 128))


@pytest.mark.parametrize("bad", ["dtype", "shape", "contiguous", "device"])
def test_binding_checks_caller_outputs(bad):
    """A caller-supplied output must be exactly what the kernels write: fp32, contiguous, the given shape."""
    import torch
    cpu = torch.device("cpu")
    shape = (3, 2, 128)
    t = {"dtype": torch.zeros(shape, dtype=torch.bfloat16), "shape": torch.zeros(3, 2, 64),
         "contiguous": torch.zeros(2, 3, 128).transpose(0, 1), "device": torch.zeros(shape, device="meta")}[bad]
    with pytest.raises((TypeError, ValueError)):
        kda._out(t, "o", shape, cpu)
    kda._out(torch.zeros(shape), "o", shape, cpu)  # the right one passes
