"""The structured-sparse MFMA (SMFMAC) operand layouts that the packed 2:4 format relies on, pinned on the
device by one bare instruction per shape (16x16x64 in the decode kernels, 32x32x32 in the prefill) against
the plain 2:4 product on the host.

The 2:4 structured-sparsity article (section 3) fixes what is computed: two kept weights in every group of
four consecutive input positions, two bits of position per kept element.  The packed format stores, per
row and group g, the two kept values in position order and the nibble i0 | i1 << 2 at bits 4g of a 64-bit
word; the probe (tests/probe/smfmac_probe.hip, built by __graft_entry__.build()) moves that logical form
into the lane layout the product kernels use.  Small integers make every product and sum exact in fp32, so
the comparison is exact."""
import ctypes
import os

import numpy as np
import pytest
import torch

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libsmfmac_probe.so")
DEV = torch.device("cuda:0")
# the six ways to keep two of four positions, as (i0, i1) with i0 < i1
PATTERNS = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)])
SHAPES = {16: (16, 64, 16), 32: (32, 32, 32)}      # rows, positions, columns


def _lib():
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.smfmac_probe.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4
    lib.smfmac_probe.restype = ctypes.c_int
    return lib


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16)


def make_case(shape, seed, dense=False):
    """A block in the packed logical form and its plain 2:4 product (int64)."""
    rows, kpos, cols = SHAPES[shape]
    rng = np.random.default_rng(seed)
    groups = kpos // 4
    vals = rng.integers(-4, 5, size=(rows, groups, 2))
    sel = np.zeros((rows, groups), dtype=np.int64) if dense else rng.integers(0, 6, size=(rows, groups))
    i0, i1 = PATTERNS[sel, 0], PATTERNS[sel, 1]
    nib = (i0 | (i1 << 2)).astype(np.uint64)
    meta = np.zeros(rows, dtype=np.uint64)
    for g in range(groups):
        meta |= nib[:, g] << np.uint64(4 * g)
    b = rng.integers(-4, 5, size=(kpos, cols))
    w = np.zeros((rows, kpos), dtype=np.int64)
    r = np.arange(rows)[:, None]
    g = np.arange(groups)[None, :]
    w[r, 4 * g + i0] = vals[:, :, 0]
    w[r, 4 * g + i1] = vals[:, :, 1]
    return vals.reshape(rows, 2 * groups), meta, b, w @ b


def test_reference_is_two_of_four():
    """The host side of the probe: every group keeps exactly two positions, all six patterns occur, and
    the dense pattern (0, 1) puts the values at positions 4q and 4q + 1."""
    for shape in SHAPES:
        a, meta, b, want = make_case(shape, 1)
        rows, kpos, _ = SHAPES[shape]
        nibs = [(int(m) >> (4 * g)) & 0xF for m in meta for g in range(kpos // 4)]
        assert set(nibs) == {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}
        a, meta, b, want = make_case(shape, 2, dense=True)
        assert all(int(m) == int("4" * (kpos // 4), 16) for m in meta)
        w = np.zeros((rows, kpos), dtype=np.int64)
        w[:, 0::4], w[:, 1::4] = a[:, 0::2], a[:, 1::2]
        assert np.array_equal(w @ b, want)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [16, 32])
def test_smfmac_layout(shape):
    lib = _lib()
    rows, kpos, cols = SHAPES[shape]
    for seed in range(6):
        dense = seed == 5
        a, meta, b, want = make_case(shape, 100 * shape + seed, dense=dense)
        da = _bf16_bits(a).to(DEV)
        dm = torch.from_numpy(meta.view(np.int64)).to(DEV)
        db = _bf16_bits(b).to(DEV)
        dd = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=DEV)
        print(f"[probe]  smfmac {shape} seed={seed} dense={dense}", flush=True)
        rc = lib.smfmac_probe(shape, da.data_ptr(), dm.data_ptr(), db.data_ptr(), dd.data_ptr())
        assert rc == 0, f"HIP error {rc}"
        got = dd.cpu().numpy()
        assert np.array_equal(got, want.astype(np.float32)), (shape, seed, np.argwhere(got != want)[:5])
