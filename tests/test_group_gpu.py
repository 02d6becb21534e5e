"""hinm_spmm_group: several packed weights that read the same X, in one launch, against the float64
oracle per weight (the same bar as hinm_spmm), and bit for bit against hinm_spmm where both launches
split the reduction the same way."""
import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def _packed(w):
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), w.tile_rows, w.t_s, w.v_s, w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    return pk, oh.masked_weight(bits_of(w.w_bf16), inter["mask"])


def _check_group(ws, batches, label):
    pks, whs = zip(*[_packed(w) for w in ws])
    grp = hinm.Group(pks)
    cin = ws[0].cin
    for b in batches:
        x = torch.randn(cin, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16)
        print(f"[group] {label}: {len(ws)} weights, batch {b}", flush=True)
        ys = hinm.spmm_group(grp, x.to(DEV))
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        for g, (y, wh) in enumerate(zip(ys, whs)):
            check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"{label} weight {g} batch {b}")
    return pks, grp


def test_group_qkv_shapes():
    """Three 4096 x 4096 weights (the q, k, v of a 7B-shaped layer) at decode and prefill batches."""
    ws = [synth.stack_layer(3, proj, batch=1) for proj in (0, 1, 2)]
    pks, grp = _check_group(ws, (1, 16, 64, 2048), "qkv")
    # at batch 2048 both the group and each single product run unsplit: same bits
    x = torch.randn(4096, 2048, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    ys = hinm.spmm_group(grp, x)
    for pk, y in zip(pks, ys):
        assert torch.equal(y.view(torch.int16), hinm.spmm(pk, x).view(torch.int16))


def test_group_gate_up_shapes():
    ws = [synth.stack_layer(7, proj, batch=1) for proj in (4, 5)]
    _check_group(ws, (1, 16, 32, 64, 300), "gate/up")


def test_group_mixed_regions_and_ragged_batches():
    """Weights with different t_s / v_s (so different K-block counts) and rows, ragged batches, a
    strided X."""
    ws = [synth.small(512, 2048, 64, 0.75, 0.55, 1, seed=21), synth.small(256, 2048, 64, 0.5, 0.25, 1, seed=22),
          synth.small(768, 2048, 64, 0.6, 0.6, 1, seed=23)]
    pks, grp = _check_group(ws, (1, 7, 17, 33, 63, 65, 129, 1000, 1031), "mixed")
    big = torch.randn(2048, 40, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    outs = [torch.full((pk.plan.cout, 48), 7.0, dtype=torch.bfloat16, device=DEV) for pk in pks]
    hinm.spmm_group(grp, big.to(DEV)[:, :24], outs=[o[:, :24] for o in outs])
    torch.cuda.synchronize()
    xf = synth.as_f64(big[:, :24])
    for o, w in zip(outs, ws):
        _, _, inter = oracle_pack(w)
        wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
        check_y(o[:, :24], oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "strided")
        assert (o[:, 24:] == 7.0).all()


def test_group_32_row_tiles_run_one_launch_each():
    ws = [synth.small(128, 512, 32, 0.75, 0.5, 1, seed=31), synth.small(96, 512, 32, 0.5, 0.25, 1, seed=32)]
    pks, grp = _check_group(ws, (1, 16, 100), "32-row tiles")
    x = torch.randn(512, 100, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    ys = hinm.spmm_group(grp, x)
    for pk, y in zip(pks, ys):
        assert torch.equal(y.view(torch.int16), hinm.spmm(pk, x).view(torch.int16))


def test_group_of_eight_weights():
    """The largest group (8 weights, so every weight boundary of the split decode is a real one), rows
    and regions differing per weight, at split-decode and prefill batches."""
    shapes = [(64, 0.75, 0.55), (128, 0.5, 0.25), (192, 0.6, 0.6), (64, 0.8, 0.7), (256, 0.75, 0.5),
              (128, 0.5, 0.5), (320, 0.7, 0.45), (64, 0.55, 0.3)]
    ws = [synth.small(rows, 1024, 64, t, v, 1, seed=40 + i) for i, (rows, t, v) in enumerate(shapes)]
    _check_group(ws, (1, 5, 16, 40, 64, 200), "eight")


def test_split_decode_two_split_counts():
    """300 row blocks at batch <= 64: two workgroups share a compute unit (at 17-32 tokens with the
    smaller rounds), so 512 run at once; the first 88 row blocks run whole and the last 212 split in two
    (88 + 424 = 512 workgroups); at 33-64 tokens the same split over one workgroup per unit.  Alone
    and as a group with a second weight (300 + 16 row blocks)."""
    w = synth.small(19200, 2048, 64, 0.75, 0.55, 1, seed=50)
    pk, wh = _packed(w)
    need = hinm.spmm_workspace_bytes(pk.plan, 16)
    assert need >= 2 * 19200 * 16 * 4          # partial planes for two splits
    for b in (1, 7, 16, 17, 25, 32, 33, 64):
        x = torch.randn(2048, b, generator=torch.Generator().manual_seed(60 + b)).to(torch.bfloat16)
        print(f"[two split counts] batch {b}", flush=True)
        y = hinm.spmm(pk, x.to(DEV))
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"two split counts batch {b}")
    w2 = synth.small(1024, 2048, 64, 0.5, 0.25, 1, seed=51)
    _check_group([w, w2], (1, 16, 20, 32, 48), "two split counts")


def test_prefill_two_split_counts():
    """150 row blocks in two 128-token blocks (batch 129-255): 300 items for the 512-workgroup grid, so
    on each XCD the first items run whole and the rest in two K halves.  Alone, and as the q/k/v group
    at batch 200 (384 items)."""
    w = synth.small(9600, 2048, 64, 0.75, 0.55, 1, seed=52)
    pk, wh = _packed(w)
    assert hinm.spmm_workspace_bytes(pk.plan, 200) > 0          # the split's partial sums
    for b in (129, 200, 255):
        x = torch.randn(2048, b, generator=torch.Generator().manual_seed(70 + b)).to(torch.bfloat16)
        print(f"[prefill two split counts] batch {b}", flush=True)
        y = hinm.spmm(pk, x.to(DEV))
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"prefill two split counts batch {b}")
    ws = [synth.stack_layer(4, proj, batch=1) for proj in (0, 1, 2)]
    _check_group(ws, (200,), "qkv prefill two split counts")
