"""hinm_gyro_permute on the GPU against the oracle (oracle/gyro.py).

Bars: the new perm bit-exact and the cost trace equal to the last bit (both sides add the same float64
terms in the same order, without fused multiply-adds), on the same seeded draws; the product through the
permuted pack within the product bar of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle.gyro as og
import oracle.hinm as oh
import synth
from helpers import bits_of, check_y

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")


def case(cout, cin, R, t, v, seed, power=3):
    rng = np.random.default_rng(seed)
    d = (rng.random((cout, cin)) ** power).astype(np.float32)
    p = oh.plan(cout, cin, R, t, v)
    perm = np.stack([rng.permutation(cin) for _ in range(p.n_tiles)]).astype(np.int32)
    return d, p, perm


def run_both(d, p, perm, rounds, s, iters, seed):
    n = og.n_clusters(p.groups, s)
    sample, init = synth.gyro_draws(seed, rounds, p.n_tiles, p.groups, n)
    print(f"[gyro] {p.cout}x{p.cin} R={p.tile_rows} G={p.groups} N={n} rounds={rounds} iters={iters}", flush=True)
    got, tr = hinm.gyro_permute(torch.from_numpy(d).to(DEV), torch.from_numpy(perm).to(DEV), p.tile_rows, p.t_s,
                                p.v_s, rounds, s, iters, sample, init)
    torch.cuda.synchronize()
    want, tr_ref = og.gyro_permutation(d, perm, p, rounds, s, iters, sample, init)
    return got.cpu().numpy(), tr, want, tr_ref


@pytest.mark.parametrize("args", [
    ((128, 96, 32, 0.75, 0.5), 3, 3, 2),
    ((256, 512, 64, 0.75, 0.55), 2, 8, 3),
    ((192, 256, 64, 0.6, 0.35), 2, 5, 1),
    ((128, 200, 64, 0.5, 0.0), 2, 100, 2),      # one cluster holds every group
    ((64, 1024, 64, 0.75, 0.55), 1, 32, 4),
])
def test_gyro_matches_oracle(args):
    shape, rounds, s, iters = args
    d, p, perm = case(*shape, seed=sum(shape[:2]))
    got, tr, want, tr_ref = run_both(d, p, perm, rounds, s, iters, seed=shape[1])
    assert np.array_equal(got, want)
    assert np.array_equal(tr, tr_ref), (tr, tr_ref)
    assert np.all(np.diff(tr, axis=0) <= 0) and np.all(tr[-1] <= tr[0])


def test_gyro_zero_rounds_and_no_24_region():
    d, p, perm = case(128, 96, 32, 0.75, 0.5, seed=5)
    got, tr, want, tr_ref = run_both(d, p, perm, 0, 4, 2, seed=5)
    assert np.array_equal(got, perm) and np.array_equal(tr, tr_ref)
    d, p, perm = case(128, 96, 32, 0.75, 0.75, seed=6)             # v_s = t_s: no 2:4 region
    got, tr, want, tr_ref = run_both(d, p, perm, 2, 4, 2, seed=6)
    assert np.array_equal(got, perm) and not tr.any()


def test_gyro_then_pack_and_product():
    """The permuted pack multiplies like the oracle's, and keeps more importance than the original perm."""
    w = synth.small(256, 512, 64, 0.75, 0.55, 1, seed=9)
    d = w.importance.numpy()
    p = oh.plan(256, 512, 64, 0.75, 0.55)
    perm = w.perm.numpy().astype(np.int32)
    got, tr, want, _ = run_both(d, p, perm, 3, 8, 3, seed=9)
    assert np.array_equal(got, want)
    assert oh.retained_importance(d, got, p) > oh.retained_importance(d, perm, p)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.75, 0.55, torch.from_numpy(got).to(DEV))
    x = torch.randn(512, 300, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    y = hinm.spmm(pk, x.to(DEV))
    torch.cuda.synchronize()
    _, inter = oh.pack(bits_of(w.w_bf16), d, got, p, with_intermediates=True)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), "gyro-permuted product")


def test_gyro_rejects_a_bad_perm():
    d, p, perm = case(128, 96, 32, 0.75, 0.5, seed=7)
    perm[1, 3] = perm[1, 4]
    n = og.n_clusters(p.groups, 4)
    sample, init = synth.gyro_draws(7, 1, p.n_tiles, p.groups, n)
    with pytest.raises(hinm.HinmError) as e:
        hinm.gyro_permute(torch.from_numpy(d).to(DEV), torch.from_numpy(perm).to(DEV), 32, 0.75, 0.5, 1, 4, 2,
                          sample, init)
    assert e.value.name == "HINM_EPERM"


def test_gyro_full_width_tiles_match_oracle():
    """Two tiles of the down_proj width (cin 11008, 1101 groups per tile, clusters of 32): bit-exact."""
    d, p, perm = case(128, 11008, 64, 0.75, 0.55, seed=12, power=1)
    got, tr, want, tr_ref = run_both(d, p, perm, 1, 32, 3, seed=12)
    assert p.groups == 1101
    assert np.array_equal(got, want)
    assert np.array_equal(tr, tr_ref)
    assert np.all(tr[1] < tr[0])
