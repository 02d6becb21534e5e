"""Seeded random sweeps of hinm_spmm_group and of the per-tile layout (hinm_pack_tiles / hinm_spmm_tiles).

Groups: 2 to 6 weights sharing cin and tile_rows, each with its own row count, t_s and v_s, over batches 1 to
3000; every weight's Y against the float64 oracle, and bit for bit against its own hinm_spmm whenever the group
runs one launch per weight (tile_rows not a multiple of 64), or neither launch splits K and both take the same
token block (batch <= 64, or >= 1024).
Per-tile: 2 to 12 tiles of 64 or 128 rows with random per-tile v_s; the packed buffers and tile table bit-exact
against the oracle's per-tile pack, the products within the bar, over batches 1 to 3000."""
import math

import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")

N_GROUP = 32
N_TILES = 32


def _batch(rng, macs, cap=1.5e9):
    b = int(round(math.exp(rng.uniform(0.0, math.log(3000)))))
    return max(1, min(b, int(cap // macs)))


@pytest.mark.parametrize("i", range(N_GROUP))
def test_random_group_vs_oracle(i):
    rng = np.random.default_rng(9500 + i)
    R = int(rng.choice([32, 64, 64, 64, 128]))
    n = int(rng.integers(2, 7))
    cin = 4 * int(rng.integers(16, 700))
    ws = []
    for g in range(n):
        t = float(rng.uniform(0.2, 0.9))
        v = float(rng.uniform(max(0.0, 2 * t - 1), t))
        ws.append(synth.small(R * int(rng.integers(1, 9)), cin, R, t, v, 1, seed=int(rng.integers(1, 1 << 30))))
    rows = sum(w.cout for w in ws)
    b = _batch(rng, rows * cin)
    print(f"[random group] case {i}: {n} weights, rows {[w.cout for w in ws]}, cin {cin}, R {R}, batch {b}", flush=True)
    pks = [hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), R, w.t_s, w.v_s, w.perm.to(DEV)) for w in ws]
    grp = hinm.Group(pks)
    x = torch.randn(cin, b, generator=torch.Generator().manual_seed(i)).to(torch.bfloat16)
    xd = x.to(DEV)
    ys = hinm.spmm_group(grp, xd)
    singles = [hinm.spmm(pk, xd) for pk in pks]
    torch.cuda.synchronize()
    xf = synth.as_f64(x)
    unsplit = all(hinm.spmm_workspace_bytes(pk.plan, b) == 0 for pk in pks) and grp.workspace_bytes(b) == 0
    for g, (w, y, y1) in enumerate(zip(ws, ys, singles)):
        _, _, inter = oracle_pack(w)
        wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"group case {i} weight {g}")
        if R % 64 or (unsplit and (b <= 64 or b >= 1024)):
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"group case {i} weight {g} vs hinm_spmm"


@pytest.mark.parametrize("i", range(N_TILES))
def test_random_tiles_vs_oracle(i):
    rng = np.random.default_rng(9800 + i)
    R = int(rng.choice([64, 64, 128]))
    T = int(rng.integers(2, 13))
    cin = 4 * int(rng.integers(16, 700))
    t = float(rng.uniform(0.2, 0.9))
    lo = max(0.0, 2 * t - 1)
    v = [float(x) for x in rng.uniform(lo, t, T)]
    w = synth.small(T * R, cin, R, t, v[0], 1, seed=int(rng.integers(1, 1 << 30)))
    b = _batch(rng, T * R * cin)
    print(f"[random tiles] case {i}: {T * R}x{cin} R={R} t_s={t:.3f} v_s {min(v):.3f}..{max(v):.3f} batch {b}",
          flush=True)
    pk = hinm.pack_tiles(w.w_bf16.to(DEV), w.importance.to(DEV), R, t, v, w.perm.to(DEV))
    plans = oh.plan_tiles(w.cout, cin, R, t, v)
    ref, inter = oh.pack_tiles(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), plans,
                               with_intermediates=True)
    torch.cuda.synchronize()
    assert np.array_equal(pk.tiles.cpu().numpy(), ref["tiles"])
    for k, dt in (("val_dense", np.uint16), ("idx_dense", None), ("val_24", np.uint16), ("meta_24", np.uint64),
                  ("idx_24", None)):
        got = getattr(pk, k).cpu().numpy()
        got = got.view(dt) if dt is not None else got
        assert np.array_equal(got, ref[k]), k
    x = torch.randn(cin, b, generator=torch.Generator().manual_seed(i)).to(torch.bfloat16)
    y = hinm.spmm(pk, x.to(DEV))
    y2 = hinm.spmm(pk, x.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"tiles case {i}")
