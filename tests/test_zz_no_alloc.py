"""hinm_spmm_noalloc (no workspace, no device allocation; scratch in the library's static device array)
against hinm_spmm with a caller workspace, through the C ABI: the same kernels and split counts, so the
same bits, and within the bar of the oracle.  Two calls in a row per shape, the second with a smaller
batch (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def _packed(cout, cin, seed):
    w = synth.small(cout, cin, 64, 0.75, 0.55, 1, seed=seed)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, w.t_s, w.v_s, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    return w, pk, oh.masked_weight(bits_of(w.w_bf16), inter["mask"])


@pytest.mark.parametrize("shape,batches", [
    ((1024, 4096), (64, 16)),        # split decode: 16 row blocks, K split 16 ways
    ((4096, 4096), (128, 100)),      # batch > 64 with the K split (64 items, 4 ways: 32 MiB of partials)
    ((512, 2048), (300, 65)),        # 8 tiles: K split at 128-token blocks, ragged tails
    ((19200, 2048), (40, 16)),       # split decode with two split counts (300 row blocks)
    ((9600, 2048), (200, 129)),      # batch > 64 with two split counts (300 items of 128 tokens)
])
def test_noalloc_matches_spmm(shape, batches):
    cout, cin = shape
    w, pk, wh = _packed(cout, cin, seed=cout + cin)
    for i, b in enumerate(batches):
        need = hinm.spmm_workspace_bytes(pk.plan, b)
        assert 0 < need <= hinm.HINM_NOALLOC_SCRATCH_BYTES
        x = torch.randn(cin, b, generator=torch.Generator().manual_seed(17 * b + i)).to(torch.bfloat16)
        xd = x.to(DEV)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        y_ref = hinm.spmm(pk, xd, workspace=ws)
        y = torch.full((cout, b), 3.0, dtype=torch.bfloat16, device=DEV)
        print(f"[noalloc] {cout}x{cin} batch {b} (call {i + 1}), workspace need {need} bytes", flush=True)
        hinm.spmm_noalloc(pk, xd, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"batch {b}: differs from hinm_spmm"
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"noalloc {cout}x{cin} batch {b}")


def test_noalloc_without_split_and_repeat():
    """A product that needs no scratch (one K range per workgroup), then one that does, twice."""
    w, pk, wh = _packed(11008 // 4, 1024, seed=5)
    for b in (2048, 16, 16):
        x = torch.randn(1024, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16)
        y = torch.empty(pk.plan.cout, b, dtype=torch.bfloat16, device=DEV)
        print(f"[noalloc] {pk.plan.cout}x1024 batch {b}", flush=True)
        hinm.spmm_noalloc(pk, x.to(DEV), y)
        y_ref = hinm.spmm(pk, x.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
