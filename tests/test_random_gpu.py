"""Seeded random sweep over the launch space of hinm_spmm / hinm_spmm_rows.

Each case draws a weight shape (tile_rows 16 to 192: multiples of 64 run the split decode and prefill kernels,
the others the 16-row decode and generic kernels; 1 to 12 tiles; cin 16 to 3596), t_s and v_s anywhere in their
legal range (so any mix of dense, 2:4 and pruned regions, empty regions included), a batch from 1 to 3000
(log-uniform), an X that is contiguous, row-padded or 2 bytes off 16-byte alignment, a row-padded Y, and in some
cases an output-row map.  Every case is checked against the float64 oracle with the same bar as every other
product test, and a second call must give the same bits."""
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

N_CASES = 160
MAX_MACS = 1.5e9          # cout x cin x batch, so the float64 oracle product stays well under a second


def draw_case(i):
    rng = np.random.default_rng(7000 + i)
    R = int(rng.choice([16, 32, 48, 64, 64, 64, 128, 192]))
    T = int(rng.integers(1, 13))
    cin = 4 * int(rng.integers(4, 900))
    t = float(rng.uniform(0.0, 0.95))
    v = float(rng.uniform(max(0.0, 2 * t - 1), t))
    batch = int(round(math.exp(rng.uniform(0.0, math.log(3000)))))
    batch = max(1, min(batch, int(MAX_MACS // (T * R * cin))))
    layout = str(rng.choice(["contiguous", "padded", "offset"]))
    x_pad = int(rng.integers(1, 41))
    y_pad = int(rng.choice([0, 0, 3, 8]))
    rows = bool(rng.random() < 0.3)
    return dict(R=R, T=T, cin=cin, t=t, v=v, batch=batch, layout=layout, x_pad=x_pad, y_pad=y_pad, rows=rows,
                seed=int(rng.integers(1, 1 << 30)))


def make_x(x: torch.Tensor, layout: str, pad: int) -> torch.Tensor:
    cin, b = x.shape
    if layout == "contiguous":
        return x.to(DEV)
    if layout == "padded":
        big = torch.zeros(cin, b + pad, dtype=torch.bfloat16, device=DEV)
        big[:, :b] = x.to(DEV)
        return big[:, :b]
    flat = torch.zeros(cin * b + 1, dtype=torch.bfloat16, device=DEV)      # one element off alignment
    xd = flat[1:].view(cin, b)
    xd.copy_(x.to(DEV))
    return xd


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_vs_oracle(i):
    c = draw_case(i)
    cout = c["T"] * c["R"]
    print(f"[random] case {i}: {cout}x{c['cin']} R={c['R']} t_s={c['t']:.3f} v_s={c['v']:.3f} batch={c['batch']} "
          f"X {c['layout']} Y pad {c['y_pad']} rows={c['rows']}", flush=True)
    w = synth.small(cout, c["cin"], c["R"], c["t"], c["v"], 1, seed=c["seed"])
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), c["R"], c["t"], c["v"], w.perm.to(DEV))
    _, _, inter = oracle_pack(w)
    wh = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])
    b = c["batch"]
    x = torch.randn(c["cin"], b, generator=torch.Generator().manual_seed(c["seed"])).to(torch.bfloat16)
    xd = make_x(x, c["layout"], c["x_pad"])
    out_rows = None
    if c["rows"]:
        out_rows = torch.from_numpy(np.random.default_rng(c["seed"]).permutation(cout).astype(np.int32)).to(DEV)
    ys = []
    for _ in range(2):
        big = torch.full((cout, b + c["y_pad"]), 5.0, dtype=torch.bfloat16, device=DEV)
        hinm.spmm(pk, xd, out=big[:, :b], out_rows=out_rows)
        ys.append(big)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16)), "second call differs"
    if c["y_pad"]:
        assert (ys[0][:, b:] == 5.0).all(), "wrote past the batch in a padded Y"
    y = ys[0][:, :b]
    if out_rows is not None:
        y = y[out_rows.long()]                     # Y row out_rows[r] holds product row r
    xf = synth.as_f64(x)
    check_y(y, oh.spmm(wh, xf), np.abs(wh) @ np.abs(xf), f"random case {i}")
