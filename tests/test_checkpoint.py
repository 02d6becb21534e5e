"""Packed-weight checkpoints: a packed weight is packed once and stored (2:4 article, section 5: prune
once, then deploy; FlexHiNM-GP notes, key design 4: the kernel works from stored indices).
state_dict() holds the layout version, the plan's arguments and plain tensors, so torch.save and
torch.load(weights_only=True) round-trip it; loading checks the version and every buffer against the
plan.  The CPU tests build the buffers with the oracle; the GPU test packs on the device."""
import io

import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of

hinm = pytest.importorskip("structured_sparse_gemm_amd")


def _oracle_packed(w):
    p = hinm.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s)
    op = oh.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s)
    b = oh.pack(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), op)
    t = {"val_dense": torch.from_numpy(b["val_dense"].view(np.int16).copy()),
         "idx_dense": torch.from_numpy(b["idx_dense"].astype(np.int32)),
         "val_24": torch.from_numpy(b["val_24"].view(np.int16).copy()),
         "meta_24": torch.from_numpy(b["meta_24"].view(np.int64).copy()),
         "idx_24": torch.from_numpy(b["idx_24"].astype(np.int32))}
    return hinm.HinmPacked(p, **t)


def _roundtrip(sd):
    buf = io.BytesIO()
    torch.save(sd, buf)
    buf.seek(0)
    return torch.load(buf, weights_only=True)


def test_packed_roundtrip_bit_exact():
    w = synth.small(256, 512, 64, 0.75, 0.55, 8, seed=5)
    pk = _oracle_packed(w)
    back = hinm.HinmPacked.from_state_dict(_roundtrip(pk.state_dict()))
    assert back.plan == pk.plan
    for k in ("val_dense", "idx_dense", "val_24", "meta_24", "idx_24"):
        assert torch.equal(getattr(back, k), getattr(pk, k)), k


def test_packed_load_rejects_other_versions_and_shapes():
    w = synth.small(128, 256, 32, 0.75, 0.5, 8, seed=6)
    sd = _oracle_packed(w).state_dict()
    with pytest.raises(ValueError, match="layout version"):
        hinm.HinmPacked.from_state_dict(dict(sd, format_version=hinm.HINM_FORMAT_VERSION + 1))
    with pytest.raises(ValueError, match="idx_24"):
        hinm.HinmPacked.from_state_dict(dict(sd, idx_24=sd["idx_24"][:, 1:]))
    with pytest.raises(ValueError, match="meta_24"):
        hinm.HinmPacked.from_state_dict(dict(sd, meta_24=sd["meta_24"].to(torch.int32)))
    with pytest.raises(ValueError, match="val_dense"):       # plan arguments that give other buffer sizes
        hinm.HinmPacked.from_state_dict(dict(sd, v_s=0.6))
    with pytest.raises(ValueError):
        hinm.HinmPacked.from_state_dict({"format": "something else"})


def test_per_tile_packed_roundtrip():
    w = synth.small(256, 512, 64, 0.75, 0.55, 8, seed=7)
    v = [0.55, 0.6, 0.5, 0.7]
    p = hinm.plan_tiles(w.cout, w.cin, 64, 0.75, v)
    plans = oh.plan_tiles(w.cout, w.cin, 64, 0.75, v)
    b = oh.pack_tiles(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), plans)
    pk = hinm.HinmTPacked(p, torch.from_numpy(b["tiles"].astype(np.int32)),
                          torch.from_numpy(b["val_dense"].view(np.int16).copy()),
                          torch.from_numpy(b["idx_dense"].astype(np.int32)),
                          torch.from_numpy(b["val_24"].view(np.int16).copy()),
                          torch.from_numpy(b["meta_24"].view(np.int64).copy()),
                          torch.from_numpy(b["idx_24"].astype(np.int32)))
    sd = _roundtrip(pk.state_dict())
    back = hinm.HinmTPacked.from_state_dict(sd)
    assert back.plan.v_s == tuple(v) and np.array_equal(back.plan.tiles, p.tiles)
    for k in ("tiles", "val_dense", "idx_dense", "val_24", "meta_24", "idx_24"):
        assert torch.equal(getattr(back, k), getattr(pk, k)), k
    bad = dict(sd, tiles=sd["tiles"].clone())
    bad["tiles"][1, 0] += 1
    with pytest.raises(ValueError, match="tile table"):
        hinm.HinmTPacked.from_state_dict(bad)


@pytest.mark.gpu
def test_device_packed_roundtrip_same_product():
    dev = torch.device("cuda:0")
    w = synth.small(512, 1024, 64, 0.75, 0.55, 64, seed=8)
    pk = hinm.pack(w.w_bf16.to(dev), w.importance.to(dev), 64, w.t_s, w.v_s, w.perm.to(dev))
    sd = _roundtrip({k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in pk.state_dict().items()})
    back = hinm.HinmPacked.from_state_dict(sd, device=dev)
    x = w.x_bf16.to(dev)
    print("[checkpoint] product from the reloaded packed weight", flush=True)
    y0, y1 = hinm.spmm(pk, x), hinm.spmm(back, x)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
