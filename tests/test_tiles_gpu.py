"""Per-tile v_s on the GPU: hinm_pack_tiles, hinm_spmm_tiles and hinm_boundary_search_tiles against the oracle.

Bars: packed buffers and tile table bit-exact against oracle.pack_tiles; products within the product
tolerance of the oracle (|Y - Y_o| <= 1e-2 (|W_hat| |X|), relative Frobenius <= 5e-3), and bit-identical
to the uniform product when every tile has the same v_s; per-tile v_s of the search equal to the oracle's
(a tile may differ only where the oracle's own consecutive values tie within 1e-12).
"""
import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def random_v(n_tiles, t_s, seed):
    rng = np.random.default_rng(seed)
    lo = max(0.0, 2 * t_s - 1)
    return [float(x) for x in rng.uniform(lo, t_s, n_tiles)]


def pack_both(w, v):
    print(f"[tiles] {w.name} {w.cout}x{w.cin} R={w.tile_rows} t_s={w.t_s}", flush=True)
    pk = hinm.pack_tiles(w.w_bf16.to(DEV), w.importance.to(DEV), w.tile_rows, w.t_s, v, w.perm.to(DEV))
    plans = oh.plan_tiles(w.cout, w.cin, w.tile_rows, w.t_s, v)
    ref, inter = oh.pack_tiles(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), plans,
                               with_intermediates=True)
    return pk, plans, ref, inter


def assert_tiles_packed_equal(pk, ref):
    assert np.array_equal(pk.tiles.cpu().numpy(), ref["tiles"])
    assert np.array_equal(pk.val_dense.cpu().numpy().view(np.uint16), ref["val_dense"])
    assert np.array_equal(pk.idx_dense.cpu().numpy(), ref["idx_dense"])
    assert np.array_equal(pk.val_24.cpu().numpy().view(np.uint16), ref["val_24"])
    assert np.array_equal(pk.meta_24.cpu().numpy().view(np.uint64), ref["meta_24"])
    assert np.array_equal(pk.idx_24.cpu().numpy(), ref["idx_24"])


PACK_CASES = [
    (lambda: synth.small(256, 1024, 64, 0.75, 0.55, 1, seed=81), 81),
    (lambda: synth.small(192, 512, 32, 0.6, 0.3, 1, seed=82), 82),
    (lambda: synth.small(128, 256, 16, 0.5, 0.25, 1, seed=83), 83),
    (lambda: synth.small(640, 4096, 64, 0.75, 0.55, 1, seed=84), 84),
]


@pytest.mark.parametrize("case", range(len(PACK_CASES)))
def test_pack_tiles_bit_exact(case):
    mk, seed = PACK_CASES[case]
    w = mk()
    v = random_v(w.cout // w.tile_rows, w.t_s, seed)
    pk, plans, ref, _ = pack_both(w, v)
    assert_tiles_packed_equal(pk, ref)


def test_pack_tiles_equal_v_matches_uniform_pack():
    w = synth.small(512, 2048, 64, 0.75, 0.55, 1, seed=85)
    pk_u = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.75, 0.55, w.perm.to(DEV))
    pk_t = hinm.pack_tiles(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.75, [0.55] * 8, w.perm.to(DEV))
    assert torch.equal(pk_t.val_dense, pk_u.val_dense.reshape(pk_t.val_dense.shape))
    assert torch.equal(pk_t.idx_dense, pk_u.idx_dense.reshape(-1))
    assert torch.equal(pk_t.val_24, pk_u.val_24.reshape(pk_t.val_24.shape))
    assert torch.equal(pk_t.meta_24, pk_u.meta_24.reshape(pk_t.meta_24.shape))
    assert torch.equal(pk_t.idx_24, pk_u.idx_24.reshape(-1))
    for batch in (16, 300, 2048):
        x = torch.randn(w.cin, batch, generator=torch.Generator().manual_seed(batch)).to(torch.bfloat16).to(DEV)
        a = hinm.spmm(pk_u, x)
        b = hinm.spmm(pk_t, x)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"batch {batch}"


@pytest.mark.parametrize("batch", [1, 16, 40, 64, 100, 300, 1100])
def test_spmm_tiles_vs_oracle(batch):
    w = synth.small(640, 4096, 64, 0.75, 0.55, 1, seed=86)
    v = random_v(w.cout // 64, 0.75, 86)
    pk, plans, ref, inter = pack_both(w, v)
    print(f"[tiles]   spmm batch={batch}", flush=True)
    x = torch.randn(w.cin, batch, generator=torch.Generator().manual_seed(batch + 7)).to(torch.bfloat16)
    y = hinm.spmm(pk, x.to(DEV))
    torch.cuda.synchronize()
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    assert np.array_equal(wh, oh.unpack_tiles(ref, plans))
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"spmm_tiles batch {batch}")


@pytest.mark.parametrize("per_xcd", ["1", "3"])
def test_spmm_tiles_cost_ordered_schedule(per_xcd):
    """Few persistent workgroups, so each takes several (token block, tile) items in cost order: same bits
    as the launch with one item per workgroup, and within the bar of the oracle."""
    w = synth.small(640, 2048, 64, 0.75, 0.55, 1, seed=88)
    v = random_v(w.cout // 64, 0.75, 88)
    pk, plans, ref, inter = pack_both(w, v)
    x = torch.randn(w.cin, 1100, generator=torch.Generator().manual_seed(88)).to(torch.bfloat16)
    y_one = hinm.spmm(pk, x.to(DEV))
    print(f"[tiles]   cost-ordered schedule, {per_xcd} workgroups per XCD", flush=True)
    with hinm.options(prefill_per_xcd=int(per_xcd)):
        y_few = hinm.spmm(pk, x.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y_one.view(torch.int16), y_few.view(torch.int16))
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    check_y(y_few, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"cost-ordered, {per_xcd} per XCD")


def test_spmm_tiles_needs_64_row_tiles():
    w = synth.small(96, 256, 32, 0.75, 0.55, 1, seed=87)
    pk = hinm.pack_tiles(w.w_bf16.to(DEV), w.importance.to(DEV), 32, 0.75, random_v(3, 0.75, 87), w.perm.to(DEV))
    with pytest.raises(hinm.HinmError) as e:
        hinm.spmm(pk, torch.zeros(256, 16, dtype=torch.bfloat16, device=DEV))
    assert e.value.name == "HINM_ESHAPE"


def stop_index(trace):
    for k in range(1, len(trace)):
        if trace[k][1] < trace[k - 1][1]:
            return k - 1
    return len(trace) - 1


@pytest.mark.parametrize("case", range(3))
def test_boundary_search_tiles_vs_oracle(case):
    shapes = [(512, 1024, 64, 0.75), (256, 512, 32, 0.6), (192, 256, 64, 0.5)]
    cout, cin, R, t_s = shapes[case]
    w = synth.draw(f"bts{case}", cout, cin, R, t_s, None, 1, 90 + case, n_outliers=cin // 20, importance="sq")
    print(f"[tiles] boundary {cout}x{cin} R={R} t_s={t_s}", flush=True)
    v_gpu, pts = hinm.boundary_search_tiles(w.importance.to(DEV), w.perm.to(DEV), R, t_s)
    v_ref, traces = oh.boundary_search_tiles(w.importance.numpy(), w.perm.numpy(), cout, cin, R, t_s)
    for t in range(cout // R):
        if v_gpu[t] == v_ref[t]:
            assert pts[t] == len(traces[t]), f"tile {t}: {pts[t]} vs {len(traces[t])} points"
            continue
        tr = traces[t]
        k = min(stop_index(tr) + 1, len(tr) - 1)
        assert abs(tr[k][1] - tr[k - 1][1]) <= 2e-12 * abs(tr[k][1]), f"tile {t}: {v_gpu[t]} vs {v_ref[t]}"


def test_per_tile_search_pack_product_end_to_end():
    """Per-tile v_s from the device search, packed per tile, multiplied: equal to the oracle chain."""
    w = synth.draw("bte2e", 512, 2048, 64, 0.7, None, 1, 95, n_outliers=100, importance="sq")
    v, _ = hinm.boundary_search_tiles(w.importance.to(DEV), w.perm.to(DEV), 64, 0.7)
    assert len(set(v)) > 1
    pk, plans, ref, inter = pack_both(w, v)
    assert_tiles_packed_equal(pk, ref)
    x = torch.randn(w.cin, 64, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    y = hinm.spmm(pk, x.to(DEV))
    torch.cuda.synchronize()
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "per-tile end to end")
