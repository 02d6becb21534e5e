"""bench.py on the host: the arithmetic behind every roofline fraction, and the one-GPU contract.

The algorithmic bytes of a product are the packed values (cout x kept x 2), the 2-bit 2:4 metadata (cout x n_24
/ 8), the int32 index lists (n_tiles x (n_dense + n_24) x 4), X (cin x batch x 2) and Y (cout x batch x 2); the
useful flops are 2 x cout x kept x batch.  Counts come from the oracle's plan; the products are written out
here, not taken from bench.py, and the totals are also checked against the figures quoted for the headline and
the q_proj decode workloads (26.55 MB and 87.93 MB for 4096x11008 at batch 16 and 2048, 18.87 MB for q_proj at
batch 16).
"""
import os
import subprocess
import sys

import pytest

import oracle.hinm as oh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
hinm = pytest.importorskip("structured_sparse_gemm_amd")
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _expected(cout, cin, tile_rows, t_s, v_s, batch):
    p = oh.plan(cout, cin, tile_rows, t_s, v_s)
    kept = cin - (p.n_pruned + p.n_24 // 2)          # every row keeps its dense entries and half its 2:4 vectors
    assert kept == p.n_dense + p.n_24 // 2
    tiles = cout // tile_rows
    nbytes = cout * kept * 2 + cout * p.n_24 // 8 + tiles * (p.n_dense + p.n_24) * 4 + cin * batch * 2 + cout * batch * 2
    return nbytes, 2 * cout * kept * batch


@pytest.mark.parametrize("shape,batch,quoted", [
    ((4096, 11008, 64, 0.75, 0.55), 16, 26_550_784),
    ((4096, 11008, 64, 0.75, 0.55), 2048, 87_933_440),
    ((4096, 4096, 64, 0.5, 0.25), 16, 18_874_368),
    ((11008, 4096, 64, 0.75, 0.55), 2048, None),
    ((128, 256, 32, 0.75, 0.5), 8, None),
])
def test_algorithmic_bytes_and_flops(shape, batch, quoted):
    cout, cin, R, t, v = shape
    want_bytes, want_flops = _expected(cout, cin, R, t, v, batch)
    if quoted is not None:
        assert want_bytes == quoted
    got = bench.algorithmic(hinm.plan(cout, cin, R, t, v), batch)
    assert got["bytes"] == want_bytes
    assert got["useful_flops"] == want_flops
    assert got["dense_equiv_flops"] == 2 * cout * cin * batch


def test_headline_flops_match_the_quoted_figure():
    # 46.17 GFLOP of useful work per batch-2048 product of the 4096x11008 weight
    _, flops = _expected(4096, 11008, 64, 0.75, 0.55, 2048)
    assert flops == 46_170_898_432


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
