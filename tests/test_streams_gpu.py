"""Products on several streams with their default workspaces, and a HIP graph replayed after the default
workspace of its stream was outgrown.  The split reduction's arrival counters and partial sums live in
the workspace, so each stream has its own, and a buffer that is outgrown stays alive for the graphs that
name it."""
import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def _case(seed):
    w = synth.small(1024, 4096, 64, 0.75, 0.55, 16, seed=seed)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, w.t_s, w.v_s, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    return w, pk, oh.masked_weight(bits_of(w.w_bf16), inter["mask"])


def test_two_streams_default_workspaces():
    w, pk, wh = _case(41)
    assert hinm.spmm_workspace_bytes(pk.plan, 16) > 0          # the split decode: counters and partials
    g = torch.Generator().manual_seed(41)
    xs = [torch.randn(w.cin, 16, generator=g).to(torch.bfloat16) for _ in range(2)]
    xd = [x.to(DEV) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty(w.cout, 16, dtype=torch.bfloat16, device=DEV) for _ in range(24)] for _ in range(2)]
    torch.cuda.synchronize()
    print("[streams] 2 x 24 products interleaved on two streams", flush=True)
    for i in range(24):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                hinm.spmm(pk, xd[k], out=outs[k][i])
    torch.cuda.synchronize()
    for k in range(2):
        xf = synth.as_f64(xs[k])
        check_y(outs[k][0], oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"stream {k}")
        for i in range(1, 24):
            assert torch.equal(outs[k][i].view(torch.int16), outs[k][0].view(torch.int16)), (k, i)


def test_graph_replay_after_the_workspace_grew():
    w, pk, wh = _case(42)
    g = torch.Generator().manual_seed(42)
    x16 = torch.randn(w.cin, 16, generator=g).to(torch.bfloat16)
    x64 = torch.randn(w.cin, 64, generator=g).to(torch.bfloat16)
    assert hinm.spmm_workspace_bytes(pk.plan, 64) > hinm.spmm_workspace_bytes(pk.plan, 16)
    s = torch.cuda.Stream()
    x16d, x64d = x16.to(DEV), x64.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y_eager = hinm.spmm(pk, x16d)                   # makes the stream's default workspace
    torch.cuda.synchronize()
    out = torch.empty_like(y_eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        hinm.spmm(pk, x16d, out=out)
    with torch.cuda.stream(s):
        y64 = hinm.spmm(pk, x64d)                       # outgrows that workspace
    torch.cuda.synchronize()
    print("[streams] graph replays after the workspace grew", flush=True)
    for r in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), y_eager.view(torch.int16)), f"replay {r}"
        with torch.cuda.stream(s):
            y64b = hinm.spmm(pk, x64d)
        torch.cuda.synchronize()
        assert torch.equal(y64b.view(torch.int16), y64.view(torch.int16))
    xf = synth.as_f64(x16)
    check_y(out, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "graph replay")
    xf = synth.as_f64(x64)
    check_y(y64, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "batch 64")
