"""The two X paths of the batch > 64 product kernel against each other and against the oracle.

X rows go straight from the buffer loads into LDS when they are 16-byte aligned; HINM_PREFILL_PATH=staged
selects the register-staged gather for the same launch.  Both add the same products in the same order
(dense K-blocks, then 2:4 K-blocks, one MFMA chain per accumulator), so their outputs must be
bit-identical; each must also meet the product bar against the float64 oracle
(|Y - Y_o| <= 1e-2 (|W_hat| |X|), relative Frobenius <= 5e-3).  Shapes cover fewer than seven K-blocks
in a region (the short pipeline), ragged last token blocks, two 64-row blocks per tile, the output-row
map, the per-tile layout and X with a row stride larger than the batch.
"""
import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def both_paths(fn):
    with hinm.options(prefill_path=0):
        a = fn()
    with hinm.options(prefill_path=1):
        b = fn()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "LDS-direct and register-staged X paths differ"
    return a


@pytest.mark.parametrize("shape", [
    (128, 256, 64, 0.75, 0.5),      # 2 dense blocks, 1 2:4 block: short pipelines only
    (192, 1024, 64, 0.6, 0.35),     # both regions between 3 and 12 blocks
    (256, 2048, 128, 0.75, 0.55),   # two 64-row blocks per tile
    (128, 512, 64, 0.5, 0.0),       # no dense region
    (128, 700, 64, 0.75, 0.75),     # no 2:4 region
])
@pytest.mark.parametrize("batch", [65, 300, 1024, 1300])
def test_prefill_paths_vs_oracle(shape, batch):
    cout, cin, R, t, v = shape
    w = synth.small(cout, cin, R, t, v, 1, seed=cout + cin + batch)
    print(f"[prefill] {cout}x{cin} R={R} t_s={t} v_s={v} batch={batch}", flush=True)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), R, t, v, w.perm.to(DEV))
    x = torch.randn(cin, batch, generator=torch.Generator().manual_seed(batch)).to(torch.bfloat16)
    xd = x.to(DEV)
    y = both_paths(lambda: hinm.spmm(pk, xd))
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"prefill {shape} batch {batch}")


def test_prefill_paths_row_map_and_stride():
    w = synth.small(256, 1536, 64, 0.75, 0.55, 1, seed=41)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.75, 0.55, w.perm.to(DEV))
    big = torch.randn(1536, 1400, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    x = big[:, :1288]                                          # ldx 1400 > batch 1288, 16-byte rows
    xd = big.to(DEV)[:, :1288]
    rows = torch.from_numpy(np.random.default_rng(3).permutation(256).astype(np.int32)).to(DEV)
    print("[prefill] row map, ldx 1400, batch 1288", flush=True)
    y = both_paths(lambda: hinm.spmm(pk, xd, out_rows=rows))
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    ref = oh.scatter_rows(oh.spmm(wh, xf), rows.cpu().numpy())
    check_y(y, ref, oh.scatter_rows(np.abs(wh) @ np.abs(xf), rows.cpu().numpy()), "row map")


def test_prefill_paths_per_tile():
    w = synth.small(640, 2048, 64, 0.75, 0.55, 1, seed=43)
    rng = np.random.default_rng(43)
    v = [float(u) for u in rng.uniform(0.5, 0.75, w.cout // 64)]
    pk = hinm.pack_tiles(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.75, v, w.perm.to(DEV))
    x = torch.randn(2048, 1100, generator=torch.Generator().manual_seed(43)).to(torch.bfloat16)
    xd = x.to(DEV)
    print("[prefill] per-tile layout, batch 1100", flush=True)
    y = both_paths(lambda: hinm.spmm(pk, xd))
    plans = oh.plan_tiles(w.cout, w.cin, 64, 0.75, v)
    _, inter = oh.pack_tiles(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), plans, with_intermediates=True)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "per-tile")


def test_prefill_nonfinite_pruned_rows_do_not_reach_y():
    """X rows of columns pruned in every tile (their weights are zero) hold NaN and Inf; the product
    gathers only kept columns and reads pads as zeros, so Y stays finite and equal to the oracle's."""
    w = synth.small(128, 1024, 64, 0.75, 0.55, 1, seed=44)
    dead = np.arange(0, 1024, 4)[:200]                      # 200 <= n_pruned columns, zero in every row
    wb = w.w_bf16.clone()
    wb[:, torch.as_tensor(dead)] = 0
    imp = wb.float().abs()
    pk = hinm.pack(wb.to(DEV), imp.to(DEV), 64, 0.75, 0.55, w.perm.to(DEV))
    x = torch.randn(1024, 1024, generator=torch.Generator().manual_seed(44)).to(torch.bfloat16)
    x[torch.as_tensor(dead[::2])] = float("nan")
    x[torch.as_tensor(dead[1::2])] = float("inf")
    xd = x.to(DEV)
    print("[prefill] non-finite pruned rows", flush=True)
    y = both_paths(lambda: hinm.spmm(pk, xd))
    p = oh.plan(128, 1024, 64, 0.75, 0.55)
    _, inter = oh.pack(bits_of(wb), imp.numpy(), w.perm.numpy(), p, with_intermediates=True)
    assert not inter["mask"][:, dead].any(), "the zero columns must be pruned in every tile"
    wh = oh.masked_weight(bits_of(wb), inter["mask"])
    xf = synth.as_f64(x)
    xf[dead] = 0.0                                           # pruned everywhere: never multiplied
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "non-finite pruned rows")


@pytest.mark.parametrize("layout", ["aligned", "contiguous", "offset"])
def test_prefill_last_x_row_ragged_tails(layout):
    """The last input channel kept in every tile, at batches whose last token block ends inside a
    16-byte chunk (odd and even remainders), with X rows 16-byte aligned (row stride a multiple of 8
    tokens), contiguous (stride = batch) or starting 2 bytes past a 16-byte boundary.  The gathers of
    the last X row end at the buffer's end, where the range check works per dword; both X paths must
    bring every token of it back."""
    w = synth.small(128, 264, 64, 0.6, 0.35, 1, seed=23)
    w.importance[:, -1] = w.importance.max() * 4.0
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.6, 0.35, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    assert (wh[:, -1] != 0).all()
    for b in (65, 97, 129, 300, 1025, 1027, 1030, 1031, 1279, 2047):
        x = torch.randn(264, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16)
        x[-1] = torch.linspace(1.0, 2.0, b).to(torch.bfloat16)          # never zero: a lost token shows
        if layout == "aligned":
            buf = torch.zeros(264, (b + 7) // 8 * 8, dtype=torch.bfloat16, device=DEV)
            buf[:, :b].copy_(x.to(DEV))
            xd = buf[:, :b]
        elif layout == "contiguous":
            xd = x.to(DEV)
        else:
            buf = torch.empty(264 * b + 1, dtype=torch.bfloat16, device=DEV)
            buf[1:].copy_(x.reshape(-1).to(DEV))
            xd = buf[1:].view(264, b)
        print(f"[prefill] last row, batch={b} layout={layout}", flush=True)
        y = both_paths(lambda: hinm.spmm(pk, xd))
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"last row batch {b} {layout}")


@pytest.mark.parametrize("splits", [2, 4])
def test_prefill_split_k(splits):
    """Each work item's K range split over 2 or 4 workgroups (partial sums through the workspace, added
    in split order): within the bar of the oracle, identical on both X paths, bit-identical from one
    call to the next (the counters are back at zero), and ragged tails included."""
    w = synth.small(256, 2048, 64, 0.6, 0.35, 1, seed=61)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.6, 0.35, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    for b in (65, 200, 1031, 1100):
        x = torch.randn(2048, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16)
        xd = x.to(DEV)
        with hinm.options(prefill_splits=splits):
            ws = torch.zeros(hinm.spmm_workspace_bytes(pk.plan, b), dtype=torch.uint8, device=DEV)
            assert ws.numel() > 0
            print(f"[prefill] split K {splits} ways, batch={b}", flush=True)
            y = both_paths(lambda: hinm.spmm(pk, xd, workspace=ws))
            y2 = hinm.spmm(pk, xd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        assert not ws[:4 * 16384].any(), "arrival counters not back at zero"
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"split K {splits}, batch {b}")


def test_prefill_split_k_default_full_size():
    """q_proj 4096x4096 at batch 128: 64 work items, so the default splits each one 4 ways."""
    w = synth.q_proj(batch=16)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, w.t_s, w.v_s, w.perm.to(DEV))
    assert hinm.spmm_workspace_bytes(pk.plan, 128) > 0
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    x = torch.randn(4096, 128, generator=torch.Generator().manual_seed(128)).to(torch.bfloat16)
    print("[prefill] q_proj batch 128, default K split", flush=True)
    y = hinm.spmm(pk, x.to(DEV))
    torch.cuda.synchronize()
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "q_proj batch 128")


def test_prefill_nearly_one_item_per_unit_k_halves():
    """down_proj 4096x11008 at batches 800, 1000 and 1023: 4 token blocks of 256 (the last one ragged) x 64
    tiles = 256 items on a long K range, so each item's K range is split in two (the workspace holds the
    arrival counters and the halves' partial sums).  Every output row against the oracle, and the unsplit
    schedule of the same product within the same bar."""
    w = synth.down_proj(batch=16)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), w.tile_rows, w.t_s, w.v_s, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    for batch in (800, 1000, 1023):
        assert hinm.spmm_workspace_bytes(pk.plan, batch) > 0, "the K split is not in effect"
        x = torch.randn(w.cin, batch, generator=torch.Generator().manual_seed(7 + batch)).to(torch.bfloat16)
        xd = x.to(DEV)
        print(f"[prefill] down_proj batch={batch} (K halves)", flush=True)
        y = hinm.spmm(pk, xd)
        with hinm.options(prefill_splits=1):
            y1 = hinm.spmm(pk, xd)
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        ref, scale = oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf)
        check_y(y, ref, scale, f"down_proj batch {batch}, K halves")
        check_y(y1, ref, scale, f"down_proj batch {batch}, unsplit")
