"""Seeded random sweep of hinm_pack against the oracle: every packed buffer bit-exact.

Each case draws a weight shape (tile_rows 16 to 192, 1 to 10 tiles, cin 16 to 2396), t_s and v_s anywhere in
their legal range, an importance that is |W|, W*W, |W| rounded to a few levels (so most scores tie and the
(-score, column) order decides) or |W| with whole columns zeroed (+0.0 and ties at zero), and a perm that is
random, the identity, block-diagonal in blocks of 64, or reversed."""
import numpy as np
import pytest
import torch

import synth
from helpers import assert_packed_equal, device_packed_numpy, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
DEV = torch.device("cuda:0")

N_CASES = 64


def draw_case(i):
    rng = np.random.default_rng(9100 + i)
    R = int(rng.choice([16, 32, 48, 64, 64, 128, 192]))
    T = int(rng.integers(1, 11))
    cin = 4 * int(rng.integers(4, 600))
    t = float(rng.uniform(0.0, 0.95))
    v = float(rng.uniform(max(0.0, 2 * t - 1), t))
    imp = str(rng.choice(["abs", "sq", "levels", "zero_columns"]))
    perm = str(rng.choice(["random", "identity", "block64", "reversed"]))
    return dict(R=R, T=T, cin=cin, t=t, v=v, imp=imp, perm=perm, seed=int(rng.integers(1, 1 << 30)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_pack_vs_oracle(i):
    c = draw_case(i)
    cout, cin = c["T"] * c["R"], c["cin"]
    print(f"[random pack] case {i}: {cout}x{cin} R={c['R']} t_s={c['t']:.3f} v_s={c['v']:.3f} "
          f"importance {c['imp']} perm {c['perm']}", flush=True)
    w = synth.small(cout, cin, c["R"], c["t"], c["v"], 1, seed=c["seed"],
                    importance="sq" if c["imp"] == "sq" else "abs")
    rng = np.random.default_rng(c["seed"])
    if c["imp"] == "levels":
        w.importance = torch.round(w.importance / w.importance.max() * 3.0)
    elif c["imp"] == "zero_columns":
        imp = w.importance.clone()
        imp[:, torch.from_numpy(rng.random(cin) < 0.2)] = 0.0
        w.importance = imp
    if c["perm"] == "identity":
        w.perm = torch.arange(cin, dtype=torch.int32).repeat(c["T"], 1)
    elif c["perm"] == "reversed":
        w.perm = torch.arange(cin - 1, -1, -1, dtype=torch.int32).repeat(c["T"], 1)
    elif c["perm"] == "block64":
        rows = []
        for _ in range(c["T"]):
            r = np.arange(cin)
            for b0 in range(0, cin, 64):
                b1 = min(cin, b0 + 64)
                r[b0:b1] = b0 + rng.permutation(b1 - b0)
            rows.append(r)
        w.perm = torch.from_numpy(np.stack(rows).astype(np.int32))
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.contiguous().to(DEV), c["R"], c["t"], c["v"],
                   w.perm.contiguous().to(DEV))
    torch.cuda.synchronize()
    p, want, _ = oracle_pack(w)
    assert (pk.plan.n_dense, pk.plan.n_24, pk.plan.n_pruned) == (p.n_dense, p.n_24, p.n_pruned)
    assert_packed_equal(device_packed_numpy(pk), want)
    windowed = bool(pk.flags & hinm.HINM_PACKED_WINDOWED)
    assert windowed == (c["perm"] in ("identity", "block64") or cin <= 64), "block-of-64 flag"
