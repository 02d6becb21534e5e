"""Output-channel permutation at write-out (hinm_spmm_rows) and cross-layer index translation
(hinm_translate_indices) on the GPU, against the oracle's definitions and against the plain product.

Bar: bit-exact.  A scattered product writes the same bf16 values as the plain product, only to other
rows; a translated index list equals the oracle's translation; a product over permuted storage with
translated indices gathers the same values in the same order as the product over channel order.
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


def packed_on_gpu(w):
    print(f"[next] pack {w.name} {w.cout}x{w.cin} R={w.tile_rows}", flush=True)
    return hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), w.tile_rows, w.t_s, w.v_s, w.perm.to(DEV))


def as_bits(t):
    return t.view(torch.int16)


# (workload, batch, path it takes)
ROWS_CASES = [
    (lambda: synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=51), 16, "split decode"),
    (lambda: synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=51), 300, "prefill"),
    (lambda: synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=51), 2048, "prefill NT 256"),
    (lambda: synth.small(96, 1024, 48, 0.5, 0.25, 1, seed=52), 100, "generic, split reduce"),
    (lambda: synth.small(96, 1024, 48, 0.5, 0.25, 1, seed=52), 16, "16-row decode"),
    (lambda: synth.tiny(), 8, "tiny"),
]


@pytest.mark.parametrize("case", range(len(ROWS_CASES)))
def test_spmm_rows_scatter(case):
    mk, batch, what = ROWS_CASES[case]
    w = mk()
    pk = packed_on_gpu(w)
    print(f"[next]   spmm_rows batch={batch} ({what})", flush=True)
    g = torch.Generator().manual_seed(100 + case)
    x = torch.randn(w.cin, batch, generator=g).to(torch.bfloat16)
    out_rows = torch.from_numpy(np.random.default_rng(case).permutation(w.cout).astype(np.int32))
    y = hinm.spmm(pk, x.to(DEV))
    ys = hinm.spmm(pk, x.to(DEV), out_rows=out_rows.to(DEV))
    torch.cuda.synchronize()
    # same bf16 values, rows moved: ys[out_rows[r]] == y[r]
    assert torch.equal(as_bits(ys)[out_rows.to(DEV).long()], as_bits(y))
    # and against the oracle at every size: scatter of the float64 product
    p, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    ref = oh.scatter_rows(oh.spmm(wh, xf), out_rows.numpy())
    scale = oh.scatter_rows(np.abs(wh) @ np.abs(xf), out_rows.numpy())
    check_y(ys, ref, scale, f"spmm_rows {what}")


def test_spmm_rows_into_strided_output():
    w = synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=53)
    pk = packed_on_gpu(w)
    x = torch.randn(w.cin, 40, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    big = torch.full((w.cout, 48), 7, dtype=torch.int16, device=DEV)
    out = big.view(torch.bfloat16)[:, :40]
    out_rows = torch.from_numpy(np.random.default_rng(9).permutation(w.cout).astype(np.int32)).to(DEV)
    hinm.spmm(pk, x, out=out, out_rows=out_rows)
    y = hinm.spmm(pk, x)
    torch.cuda.synchronize()
    assert torch.equal(as_bits(out)[out_rows.long()], as_bits(y))
    assert torch.all(big[:, 40:] == 7)                     # nothing past the batch is written


def test_translate_indices_matches_oracle_and_permuted_storage():
    wb = synth.small(128, 1024, 64, 0.75, 0.55, 1, seed=54)
    pk = packed_on_gpu(wb)
    ref_d, ref_s = pk.idx_dense.cpu().numpy(), pk.idx_24.cpu().numpy()
    sigma = np.random.default_rng(11).permutation(wb.cin).astype(np.int32)
    for batch in (16, 300):
        x = torch.randn(wb.cin, batch, generator=torch.Generator().manual_seed(batch)).to(torch.bfloat16)
        y_ref = hinm.spmm(pk, x.to(DEV)).clone()
        stored = torch.empty_like(x)
        stored[torch.from_numpy(sigma).long()] = x                 # row sigma[c] holds channel c
        pk_t = hinm.HinmPacked(pk.plan, pk.val_dense, pk.idx_dense.clone(), pk.val_24, pk.meta_24, pk.idx_24.clone())
        hinm.translate_indices(pk_t, torch.from_numpy(sigma).to(DEV))
        assert np.array_equal(pk_t.idx_dense.cpu().numpy(), oh.translate_indices(ref_d, sigma))
        assert np.array_equal(pk_t.idx_24.cpu().numpy(), oh.translate_indices(ref_s, sigma))
        y_t = hinm.spmm(pk_t, stored.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(as_bits(y_t), as_bits(y_ref)), f"batch {batch}"


def test_two_layer_chain_through_permuted_activations():
    """Layer A writes through out_rows = sigma; layer B with indices translated by sigma reads that
    output directly and gives exactly the product over A's output in channel order."""
    wa = synth.small(1024, 512, 64, 0.75, 0.55, 1, seed=55)
    wb = synth.small(256, 1024, 64, 0.75, 0.55, 1, seed=56)
    pa, pb = packed_on_gpu(wa), packed_on_gpu(wb)
    sigma = torch.from_numpy(np.random.default_rng(12).permutation(wa.cout).astype(np.int32)).to(DEV)
    pb_t = hinm.HinmPacked(pb.plan, pb.val_dense, pb.idx_dense.clone(), pb.val_24, pb.meta_24, pb.idx_24.clone())
    hinm.translate_indices(pb_t, sigma)
    for batch in (16, 256):
        x = torch.randn(wa.cin, batch, generator=torch.Generator().manual_seed(batch)).to(torch.bfloat16).to(DEV)
        ya = hinm.spmm(pa, x)
        ya_stored = hinm.spmm(pa, x, out_rows=sigma)
        yb = hinm.spmm(pb, ya)
        yb_t = hinm.spmm(pb_t, ya_stored)
        torch.cuda.synchronize()
        assert torch.equal(as_bits(yb_t), as_bits(yb)), f"batch {batch}"


def test_translate_rejects_a_non_permutation():
    w = synth.small(128, 1024, 64, 0.75, 0.55, 1, seed=57)
    pk = packed_on_gpu(w)
    before = (pk.idx_dense.clone(), pk.idx_24.clone())
    bad = np.random.default_rng(13).permutation(w.cin).astype(np.int32)
    bad[5] = bad[6]
    with pytest.raises(hinm.HinmError) as e:
        hinm.translate_indices(pk, torch.from_numpy(bad).to(DEV))
    assert e.value.name == "HINM_EPERM"
    assert torch.equal(pk.idx_dense, before[0]) and torch.equal(pk.idx_24, before[1])
    bad[5] = w.cin                                             # out of range
    with pytest.raises(hinm.HinmError):
        hinm.translate_indices(pk, torch.from_numpy(bad).to(DEV))
