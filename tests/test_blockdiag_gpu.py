"""Block-diagonal input permutations (PermLLM summary, block-wise permutation: P = diag(P_1 .. P_NB), here
blocks of 64 channels).  hinm_pack records that the perm kept every column inside its block of 64
(HINM_PACKED_WINDOWED); the product then pairs token blocks per tile in its batch > 64 schedule.  The
products match the oracle within the bar, the schedule does not change a bit, and the staggered K order
(default) and the plain one both meet the bar."""
import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def block_perm(n_tiles, cin, seed, block=64):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(n_tiles):
        r = np.arange(cin)
        for b0 in range(0, cin, block):
            b1 = min(cin, b0 + block)
            r[b0:b1] = b0 + rng.permutation(b1 - b0)
        rows.append(r)
    return torch.from_numpy(np.stack(rows).astype(np.int32))


def _case(cout, cin, seed, t_s=0.75, v_s=0.55):
    w = synth.small(cout, cin, 64, t_s, v_s, 1, seed=seed)
    w.perm = block_perm(cout // 64, cin, seed)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, t_s, v_s, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    return w, pk, oh.masked_weight(bits_of(w.w_bf16), inter["mask"])


def test_flag_set_for_block_diagonal_and_identity_perms_only():
    w = synth.small(256, 1024, 64, 0.75, 0.55, 1, seed=3)
    args = (w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.75, 0.55)
    assert hinm.pack(*args, perm=w.perm.to(DEV)).flags & hinm.HINM_PACKED_WINDOWED == 0       # random perm
    assert hinm.pack(*args, perm=None).flags & hinm.HINM_PACKED_WINDOWED                       # identity
    assert hinm.pack(*args, perm=block_perm(4, 1024, 3).to(DEV)).flags & hinm.HINM_PACKED_WINDOWED
    bp = block_perm(4, 1024, 4)
    bp[2, [63, 64]] = bp[2, [64, 63]]                                                            # one swap across blocks
    assert hinm.pack(*args, perm=bp.to(DEV)).flags & hinm.HINM_PACKED_WINDOWED == 0


@pytest.mark.parametrize("shape", [(1024, 4096), (4096, 11008)])
def test_block_diagonal_products_vs_oracle(shape):
    cout, cin = shape
    w, pk, wh = _case(cout, cin, seed=cout % 97)
    assert pk.flags & hinm.HINM_PACKED_WINDOWED
    for b in (1, 16, 300, 1031, 2048):
        x = torch.randn(cin, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16)
        print(f"[blockdiag] {cout}x{cin} batch {b}", flush=True)
        y = hinm.spmm(pk, x.to(DEV))
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"block-diagonal {cout}x{cin} batch {b}")
        if b > 64:
            # the paired-token-block schedule changes no bit; the plain K order meets the bar too
            with hinm.options(prefill_tb_group=1):
                y1 = hinm.spmm(pk, x.to(DEV))
            with hinm.options(prefill_stagger=1):
                y2 = hinm.spmm(pk, x.to(DEV))
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
            check_y(y2, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"plain K order, batch {b}")


def test_translate_keeps_the_flag_only_for_block_diagonal_maps():
    w, pk, wh = _case(256, 1024, seed=8)
    assert pk.flags & hinm.HINM_PACKED_WINDOWED
    hinm.translate_indices(pk, block_perm(1, 1024, 9)[0].to(DEV))
    assert pk.flags & hinm.HINM_PACKED_WINDOWED
    hinm.translate_indices(pk, torch.from_numpy(np.random.default_rng(1).permutation(1024).astype(np.int32)).to(DEV))
    assert pk.flags & hinm.HINM_PACKED_WINDOWED == 0
