"""kda_chunk_fwd_noalloc (the prefill on the library's own device-resident workspace, for callers
that cannot allocate) against kda_chunk_fwd on the same inputs: two calls in a row, the second on
a smaller problem, for both q/k/v dtypes; the same bits are expected, and the bar of the operator
(max|d| / RMS <= 1e-2 with bf16 q/k/v, 1e-4 with fp32) is asserted too.  Calls go through the
C ABI (the binding marshals arguments only)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import DEV, err, say, to_dev

import gated_delta_rule_29_amd as kda

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-4}


def upload(d, io, cu):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    t = {n: to_dev(d[n], dt) for n in ("q", "k", "v")}
    for n in ("z", "beta", "A", "S0"):
        t[n] = to_dev(d[n], torch.float32)
    t["cu"] = None if cu is None else to_dev(np.asarray(cu, np.int32), torch.int32)
    return t


def compare(t, io, label):
    o_ref, S_ref = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], t["S0"], t["cu"])
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    kda.kda_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"], o, t["S0"], t["cu"], S_final=S)
    torch.cuda.synchronize()
    eo = err(o.cpu().numpy(), o_ref.cpu().numpy())
    es = err(S.cpu().numpy(), S_ref.cpu().numpy())
    say(f"  {label}: err_o={eo:.3e} err_S={es:.3e} same bits={torch.equal(o, o_ref) and torch.equal(S, S_ref)}")
    assert eo <= TOL[io] and es <= TOL[io], (eo, es)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_entry_point(io):
    # first call: 2,048 tokens x 16 heads (bf16) or 1,024 x 8 (fp32)
    T, H = (2048, 16) if io == "bf16" else (1024, 8)
    d = synth.prefill_inputs(7100, T, H, dtype=io, s0_std=0.02)
    say(f"case noalloc io={io} T={T} H={H}")
    compare(upload(d, io, None), io, "first call")
    # second call, smaller: a ragged pack over 4 heads; the workspace keeps the first call's contents
    lens = [300, 77, 0, 129, 1]
    cu = synth.cu_seqlens(lens)
    d = synth.prefill_inputs(7200, int(cu[-1]), 4, dtype=io, z_scale=1.5, s0_std=0.02, n_seqs=len(lens))
    say(f"case noalloc io={io} lens={lens} H=4")
    compare(upload(d, io, cu), io, "second call")


def test_noalloc_rejects_what_does_not_fit():
    T, H = 8192, 16
    t = {n: torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV) for n in ("q", "k", "v")}
    z = torch.empty((T, H, 128), device=DEV)
    beta, A = torch.empty((T, H), device=DEV), torch.zeros(H, device=DEV)
    o = torch.empty((T, H, 128), device=DEV)
    say("case noalloc too large")
    with pytest.raises(kda.KDAError, match="WORKSPACE"):
        kda.kda_chunk_fwd_noalloc(t["q"], t["k"], t["v"], z, beta, A, o)


@pytest.mark.parametrize("io,lens", [("bf16", None), ("bf16", [700, 0, 64, 333]), ("f32", [500, 129])])
def test_noalloc_under_graph_capture(io, lens):
    """The entry point for callers that cannot allocate, captured into a graph and replayed: every
    replay, with eager work on the same buffers between replays, gives the bits of the eager call.
    The library records no memset; the NaN fills below are eager, outside the graph."""
    H = 8
    if lens is None:
        T, cu = 1024, None
        d = synth.prefill_inputs(7300, T, H, dtype=io, s0_std=0.02)
    else:
        cu = synth.cu_seqlens(lens)
        d = synth.prefill_inputs(7400, int(cu[-1]), H, dtype=io, z_scale=1.5, s0_std=0.02, n_seqs=len(lens))
    say(f"case noalloc graph io={io} lens={lens} H={H}")
    t = upload(d, io, cu)
    args = (t["q"], t["k"], t["v"], t["z"], t["beta"], t["A"])
    o_ref, S_ref = kda.kda_chunk_fwd(*args, t["S0"], t["cu"])
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    kda.kda_chunk_fwd_noalloc(*args, o, t["S0"], t["cu"], S_final=S)  # eager first call: set-up runs here
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.kda_chunk_fwd_noalloc(*args, o, t["S0"], t["cu"], S_final=S)
    for rep in range(3):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, o_ref) and torch.equal(S, S_ref)
        say(f"  replay {rep}: same bits={same}")
        assert same
    eo = err(o.cpu().numpy(), o_ref.cpu().numpy())
    assert eo == 0.0
