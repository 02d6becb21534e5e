"""Shared test helpers: oracle runs, packed-buffer comparison, the Y tolerance."""
from __future__ import annotations

import numpy as np
import torch

import oracle.hinm as oh
import synth


def bits_of(w_bf16: torch.Tensor) -> np.ndarray:
    return w_bf16.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_pack(w: synth.Workload, v_s=None, perm="given"):
    p = oh.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s if v_s is None else v_s)
    pr = None if perm is None else w.perm.numpy()
    packed, inter = oh.pack(bits_of(w.w_bf16), w.importance.numpy(), pr, p, with_intermediates=True)
    return p, packed, inter


def device_packed_numpy(pk) -> dict:
    """The GPU packed buffers as numpy arrays with the oracle's dtypes."""
    return {
        "val_dense": pk.val_dense.cpu().numpy().view(np.uint16),
        "idx_dense": pk.idx_dense.cpu().numpy(),
        "val_24": pk.val_24.cpu().numpy().view(np.uint16),
        "meta_24": pk.meta_24.cpu().numpy().view(np.uint64),
        "idx_24": pk.idx_24.cpu().numpy(),
    }


def assert_packed_equal(got: dict, want: dict) -> None:
    for k in ("idx_dense", "idx_24", "meta_24", "val_dense", "val_24"):
        g, w = got[k], want[k]
        assert g.shape == w.shape, (k, g.shape, w.shape)
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            raise AssertionError(f"{k}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"got {g[tuple(bad[0])]} want {w[tuple(bad[0])]}")


# Accuracy bar for Y (bf16 output, fp32 accumulation):
#   |Y - Y_o| <= 1e-2 * (|W_hat| |X|) elementwise, and ||Y - Y_o||_F / ||Y_o||_F <= 5e-3.
ELEM_TOL = 1e-2
FRO_TOL = 5e-3


def check_y(y_gpu: torch.Tensor, y_ref: np.ndarray, scale: np.ndarray, what: str = "") -> dict:
    y = y_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bound = ELEM_TOL * scale
    worst = float(np.max(err - bound)) if err.size else 0.0
    assert np.all(err <= bound), f"{what}: elementwise bound exceeded by {worst:.3e}"
    nref = float(np.linalg.norm(y_ref))
    fro = float(np.linalg.norm(y - y_ref)) / nref if nref > 0 else float(np.linalg.norm(y))
    assert fro <= FRO_TOL, f"{what}: relative Frobenius error {fro:.3e}"
    return {"fro": fro, "max_err": float(err.max()) if err.size else 0.0}
