"""Seeded synthetic inputs for the HiNM sparse-weight x dense-activation product.

This module only draws random numbers and builds input tensors with the
shapes, value distributions and structure of the workloads the FlexHiNM-GP
page discusses (LLaMA-7B-shaped linear layers; random per-tile input
permutations).  It holds none of the method's arithmetic: no region counts,
no ranking, no masks, no products.  Both the CPU oracle and the HIP path
receive exactly what this module returns.

Draw order (numpy ``default_rng(seed)``), fixed so both sides see the same
bits:
  1. column scales  ``exp(N(0,1))``            shape [cin]
  2. weight         ``sigma * N(0,1) * scale``  shape [cout, cin]
  3. outlier columns (optional): ``rng.choice(cin, n_out, replace=False)``,
     those columns multiplied by ``outlier_scale``
  4. permutations   ``rng.permutation(cin)`` for every output tile
  5. activations    ``N(0,1)``                  shape [cin, batch]

Weights and activations are rounded to bf16 (round-to-nearest-even, done by
torch's dtype conversion) before either side sees them.  Importance is an
input of the method; the workloads fix it as |W| or W*W of the weights.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    """Everything one run of the path consumes, already materialised."""

    name: str
    cout: int
    cin: int
    tile_rows: int
    t_s: float
    v_s: Optional[float]          # None: the caller chooses it (boundary search)
    batch: int
    w_bf16: torch.Tensor          # [cout, cin] bf16 (CPU)
    importance: torch.Tensor      # [cout, cin] fp32 (CPU)
    perm: torch.Tensor            # [cout // tile_rows, cin] int32 (CPU)
    x_bf16: torch.Tensor          # [cin, batch] bf16 (CPU)
    w_f32: Optional[torch.Tensor] = None  # the unrounded weight when drawn in fp32
    x_f32: Optional[torch.Tensor] = None  # the unrounded activations when drawn in fp32

    @property
    def n_tiles(self) -> int:
        return self.cout // self.tile_rows


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 tensor (every bf16 value is an fp64 value)."""
    return t.to(torch.float64).numpy()


def draw(name: str, cout: int, cin: int, tile_rows: int, t_s: float, v_s: Optional[float],
         batch: int, seed: int, sigma: float = 0.02, colscale: bool = True,
         n_outliers: int = 0, outlier_scale: float = 10.0, importance: str = "abs",
         importance_from_f32: bool = False, identity_perm: bool = False) -> Workload:
    """Draw one workload.  ``importance`` is "abs" (|W|) or "sq" (W*W)."""
    if cout % tile_rows:
        raise ValueError("cout must be a multiple of tile_rows")
    rng = np.random.default_rng(seed)
    scale = np.exp(rng.standard_normal(cin)) if colscale else np.ones(cin)
    w = sigma * rng.standard_normal((cout, cin)) * scale[None, :]
    if n_outliers:
        cols = rng.choice(cin, size=n_outliers, replace=False)
        w[:, cols] *= outlier_scale
    n_tiles = cout // tile_rows
    if identity_perm:
        perm = np.tile(np.arange(cin, dtype=np.int32), (n_tiles, 1))
    else:
        perm = np.stack([rng.permutation(cin) for _ in range(n_tiles)]).astype(np.int32)
    x = rng.standard_normal((cin, batch))
    w32 = torch.from_numpy(w.astype(np.float32))
    wb = w32.to(torch.bfloat16)
    src = w32 if importance_from_f32 else wb.to(torch.float32)
    if importance == "abs":
        imp = src.abs()
    elif importance == "sq":
        imp = src * src
    else:
        raise ValueError(importance)
    x32 = torch.from_numpy(x.astype(np.float32))
    xb = x32.to(torch.bfloat16)
    return Workload(name, cout, cin, tile_rows, t_s, v_s, batch, wb.contiguous(),
                    imp.contiguous(), torch.from_numpy(perm).contiguous(), xb.contiguous(),
                    w32 if importance_from_f32 else None, x32 if importance_from_f32 else None)


# The five workload families.  Sizes follow LLaMA-7B's linear layers
# (q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008).

def tiny(seed: int = 0, batch: int = 8) -> Workload:
    """W 128x256 drawn in fp32 with sigma 1, tile_rows 32, t_s 0.75, v_s 0.5, X 256x8."""
    return draw("tiny_128x256", 128, 256, 32, 0.75, 0.5, batch, seed, sigma=1.0,
                importance="abs", importance_from_f32=True)


def q_proj(seed: int = 0, batch: int = 16) -> Workload:
    """LLaMA-7B q_proj 4096x4096, tile_rows 64, t_s 0.5, v_s 0.25, decode batch 16."""
    return draw("q_proj_4096x4096", 4096, 4096, 64, 0.5, 0.25, batch, seed)


def up_proj(seed: int = 0, batch: int = 2048) -> Workload:
    """LLaMA-7B up_proj 11008x4096, tile_rows 64, t_s 0.75, v_s 0.55, prefill batch 2048."""
    return draw("up_proj_11008x4096", 11008, 4096, 64, 0.75, 0.55, batch, seed)


def down_proj_sweep(t_s: float, seed: int = 0, batch: int = 1) -> Workload:
    """LLaMA-7B down_proj 4096x11008 with 5% outlier columns x10, importance W*W.

    v_s is left open: the sweep picks it by the boundary search at each t_s.
    """
    return draw(f"down_proj_4096x11008_ts{t_s}", 4096, 11008, 64, t_s, None, batch, seed,
                n_outliers=int(round(0.05 * 11008)), importance="sq")


def down_proj(seed: int = 0, batch: int = 16, t_s: float = 0.75, v_s: float = 0.55) -> Workload:
    """LLaMA-7B down_proj 4096x11008 (cout x cin), tile_rows 64, t_s 0.75, v_s 0.55."""
    return draw("down_proj_4096x11008", 4096, 11008, 64, t_s, v_s, batch, seed)


# Layer-stack shapes: (name, cout, cin), seeds 1000 + 7*layer + proj.
STACK_PROJS = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
               ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))


def stack_layer(layer: int, proj: int, batch: int, t_s: float = 0.75, v_s: float = 0.55) -> Workload:
    """One linear layer of the 32-layer 7B-shaped stack, iid N(0, 0.02) weights."""
    name, cout, cin = STACK_PROJS[proj]
    return draw(f"stack_L{layer}_{name}", cout, cin, 64, t_s, v_s, batch, 1000 + 7 * layer + proj,
                colscale=False)


def small(cout: int, cin: int, tile_rows: int, t_s: float, v_s: float, batch: int, seed: int,
          **kw) -> Workload:
    """A small workload of the same distribution, for tests."""
    return draw(f"small_{cout}x{cin}", cout, cin, tile_rows, t_s, v_s, batch, seed, **kw)


def gyro_draws(seed: int, rounds: int, n_tiles: int, groups: int, n_clusters: int):
    """Random draws of the gyro permutation, made by the caller and given to both sides:
    sample uint8 [rounds][n_tiles][groups] (the position taken out of each 2:4 group) and
    init int32 [rounds][n_tiles][n_clusters] (distinct groups whose drawn vectors start the centroids)."""
    rng = np.random.default_rng(seed)
    sample = rng.integers(0, 4, size=(rounds, n_tiles, groups), dtype=np.uint8)
    init = np.zeros((rounds, n_tiles, n_clusters), dtype=np.int32)
    for r in range(rounds):
        for t in range(n_tiles):
            if n_clusters:
                init[r, t] = rng.choice(groups, n_clusters, replace=False)
    return sample, init
