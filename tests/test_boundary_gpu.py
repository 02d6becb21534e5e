"""Boundary search for v_s on the GPU (hinm_boundary_search) against the CPU oracle.

Bar: the chosen v_s and the number of grid points visited equal the oracle's (an index-like decision);
each visited point's retained importance R_total agrees to 1e-12 relative (both float64, summed in
different orders).  Where two consecutive R_total of the oracle lie within that tolerance of each other the
stop decision is a tie and either choice is accepted, checked against the GPU's own trace.  The down_proj
sweep compares with the stored oracle results (tests/golden/down_proj_boundary.json, written by
tests/golden/make_boundary.py, which calls only the oracle).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL = 1e-12


def stop_index(trace):
    """Index of the point the rule returns: the last before the first strict decrease."""
    for k in range(1, len(trace)):
        if trace[k][1] < trace[k - 1][1]:
            return k - 1
    return len(trace) - 1


def check_search(v_gpu, tr_gpu, v_ref, tr_ref, cin, what):
    assert len(tr_gpu) >= 1
    for (va, ra), (vb, rb) in zip(tr_gpu, tr_ref):
        assert va == vb, f"{what}: grid point {va} vs {vb}"
        assert abs(ra - rb) <= RTOL * abs(rb), f"{what}: R_total at v={va}: {ra!r} vs {rb!r}"
    if v_gpu == v_ref:
        assert len(tr_gpu) == len(tr_ref), f"{what}: visited {len(tr_gpu)} vs {len(tr_ref)} points"
        return
    # a different stop is only acceptable at a tie of the oracle's own values
    k = stop_index(tr_gpu)
    kk = min(k + 1, len(tr_ref) - 1)
    gap = abs(tr_ref[kk][1] - tr_ref[kk - 1][1])
    assert gap <= 2 * RTOL * abs(tr_ref[kk][1]), f"{what}: v_s {v_gpu} vs {v_ref} without a tie (gap {gap})"


def run_gpu(w, t_s, perm=True, step=0.01):
    print(f"[boundary] {w.name} {w.cout}x{w.cin} R={w.tile_rows} t_s={t_s}", flush=True)
    return hinm.boundary_search(w.importance.to(DEV), w.perm.to(DEV) if perm else None, w.tile_rows, t_s, step)


@pytest.mark.parametrize("t_s", [0.6, 0.7, 0.8])
def test_boundary_search_down_proj_sweep(t_s):
    with open(os.path.join(GOLDEN, "down_proj_boundary.json")) as f:
        gold = {r["t_s"]: r for r in json.load(f)["results"]}[t_s]
    w = synth.down_proj_sweep(t_s)
    v, trace = run_gpu(w, t_s)
    check_search(v, trace, gold["v_s"], [tuple(x) for x in gold["trace"]], w.cin, f"down_proj t_s={t_s}")
    p = hinm.plan(w.cout, w.cin, 64, t_s, v)
    assert (p.n_dense, p.n_24, p.n_pruned) == (gold["n_dense"], gold["n_24"], gold["n_pruned"])


SMALL = [
    (dict(cout=256, cin=512, tile_rows=64, seed=61), 0.75, True),
    (dict(cout=256, cin=512, tile_rows=64, seed=62), 0.5, True),      # grid down to v_s = 0
    (dict(cout=128, cin=1024, tile_rows=32, seed=63), 0.8, False),    # identity perm
    (dict(cout=192, cin=256, tile_rows=48, seed=64), 0.6, True),
    (dict(cout=64, cin=128, tile_rows=16, seed=65), 0.55, True),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_boundary_search_small_vs_oracle(case):
    kw, t_s, use_perm = SMALL[case]
    w = synth.draw(f"bsmall{case}", kw["cout"], kw["cin"], kw["tile_rows"], t_s, None, 1, kw["seed"],
                   n_outliers=kw["cin"] // 20, importance="sq")
    v, trace = run_gpu(w, t_s, perm=use_perm)
    perm = w.perm.numpy() if use_perm else np.tile(np.arange(w.cin), (w.cout // w.tile_rows, 1))
    v_ref, tr_ref = oh.boundary_search(w.importance.numpy(), perm, w.cout, w.cin, w.tile_rows, t_s)
    check_search(v, trace, v_ref, tr_ref, w.cin, f"case {case}")
    # the full grid agrees point by point too (the early stop relies on it)
    grid = oh.boundary_grid(w.importance.numpy(), perm, w.cout, w.cin, w.tile_rows, t_s)
    for (va, ra), (vb, rb) in zip(trace, grid):
        assert va == vb and abs(ra - rb) <= RTOL * abs(rb)


def test_boundary_search_is_deterministic():
    w = synth.draw("bdet", 256, 1024, 64, 0.7, None, 1, 66, n_outliers=50, importance="sq")
    a = run_gpu(w, 0.7)
    b = run_gpu(w, 0.7)
    assert a == b


def test_boundary_search_rejects_bad_inputs():
    w = synth.draw("bbad", 128, 256, 64, 0.7, None, 1, 67, importance="sq")
    perm = w.perm.clone()
    perm[0, 3] = perm[0, 4]
    with pytest.raises(hinm.HinmError) as e:
        hinm.boundary_search(w.importance.to(DEV), perm.to(DEV), 64, 0.7)
    assert e.value.name == "HINM_EPERM"
    imp = w.importance.clone()
    imp[5, 7] = -1.0
    with pytest.raises(hinm.HinmError) as e:
        hinm.boundary_search(imp.to(DEV), w.perm.to(DEV), 64, 0.7)
    assert e.value.name == "HINM_EIMPORTANCE"
