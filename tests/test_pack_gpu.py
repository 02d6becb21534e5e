"""hinm_pack on the GPU against the CPU oracle: every packed buffer bit-exact."""
import json
import os

import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import assert_packed_equal, device_packed_numpy, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_pack(w: synth.Workload, v_s=None, identity=False):
    dev = torch.device("cuda:0")
    perm = None if identity else w.perm.to(dev)
    return hinm.pack(w.w_bf16.to(dev), w.importance.to(dev), w.tile_rows, w.t_s,
                     w.v_s if v_s is None else v_s, perm)


def check(w, v_s=None, identity=False):
    print(f"[pack] {w.name} {w.cout}x{w.cin} R={w.tile_rows} t_s={w.t_s} v_s={w.v_s if v_s is None else v_s}",
          flush=True)
    pk = gpu_pack(w, v_s, identity)
    torch.cuda.synchronize()
    p, want, _ = oracle_pack(w, v_s, None if identity else "given")
    assert (pk.plan.n_dense, pk.plan.n_24, pk.plan.n_pruned) == (p.n_dense, p.n_24, p.n_pruned)
    assert_packed_equal(device_packed_numpy(pk), want)
    return pk


def test_pack_tiny():
    check(synth.tiny())


def test_pack_tiny_identity_perm():
    check(synth.tiny(), identity=True)


def test_pack_q_proj():
    check(synth.q_proj(batch=1))


def test_pack_up_proj():
    check(synth.up_proj(batch=1))


def test_pack_down_proj():
    check(synth.down_proj(batch=1))


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_pack_down_proj_sweep(idx):
    g = json.load(open(os.path.join(GOLDEN, "down_proj_boundary.json")))["results"][idx]
    w = synth.down_proj_sweep(g["t_s"], batch=1)
    pk = check(w, v_s=g["v_s"])
    assert (pk.plan.n_dense, pk.plan.n_24, pk.plan.n_pruned) == (g["n_dense"], g["n_24"], g["n_pruned"])


@pytest.mark.parametrize("layer,proj", [(0, 0), (13, 4), (31, 6)])
def test_pack_stack_layers(layer, proj):
    check(synth.stack_layer(layer, proj, batch=1))


@pytest.mark.parametrize("args", [
    (64, 100, 16, 0.5, 0.25),     # ragged region counts, one 16-row tile
    (96, 132, 48, 0.6, 0.3),      # tile_rows 48 (not a multiple of 64)
    (128, 256, 64, 0.0, 0.0),     # fully dense
    (128, 256, 64, 0.75, 0.75),   # no 2:4 region (p_s = 0)
    (128, 256, 64, 0.75, 0.5),    # no dense region (p_s = 1)
    (160, 4, 32, 0.5, 0.0),       # a single group of four
    (64, 300, 64, 0.9, 0.85),     # high sparsity
])
def test_pack_edge_shapes(args):
    cout, cin, R, t, v = args
    check(synth.small(cout, cin, R, t, v, 1, seed=cout + cin))


def test_pack_ties_and_zeros():
    """Integer importance with many ties and zero/-0.0 entries; the tie rules decide."""
    w = synth.small(128, 192, 32, 0.6, 0.3, 1, seed=5)
    rng = np.random.default_rng(5)
    imp = rng.integers(0, 3, size=(128, 192)).astype(np.float32)
    imp[rng.random((128, 192)) < 0.1] = -0.0
    w.importance = torch.from_numpy(imp)
    check(w)


def test_pack_rejects_bad_perm():
    w = synth.small(64, 128, 32, 0.5, 0.25, 1, seed=3)
    bad = w.perm.clone()
    bad[1, 5] = bad[1, 6]
    with pytest.raises(hinm.HinmError) as e:
        hinm.pack(w.w_bf16.cuda(), w.importance.cuda(), 32, 0.5, 0.25, bad.cuda())
    assert e.value.name == "HINM_EPERM"
    bad = w.perm.clone()
    bad[0, 0] = 128
    with pytest.raises(hinm.HinmError) as e:
        hinm.pack(w.w_bf16.cuda(), w.importance.cuda(), 32, 0.5, 0.25, bad.cuda())
    assert e.value.name == "HINM_EPERM"


@pytest.mark.parametrize("value", [-1.0, float("nan"), float("inf")])
def test_pack_rejects_bad_importance(value):
    w = synth.small(64, 128, 32, 0.5, 0.25, 1, seed=3)
    imp = w.importance.clone()
    imp[7, 9] = value
    with pytest.raises(hinm.HinmError) as e:
        hinm.pack(w.w_bf16.cuda(), imp.cuda(), 32, 0.5, 0.25, w.perm.cuda())
    assert e.value.name == "HINM_EIMPORTANCE"


def test_pack_deterministic():
    w = synth.small(256, 512, 64, 0.7, 0.45, 1, seed=8)
    a = device_packed_numpy(gpu_pack(w))
    b = device_packed_numpy(gpu_pack(w))
    assert_packed_equal(a, b)
