"""Python binding of libhinm: hierarchical N:M sparse weight x dense activation on MI355X.

Argument marshalling only.  Every step of the pack and of the product runs in
the HIP kernels of ``libhinm.so``; PyTorch supplies device memory and the
current HIP stream.  If the library is not built, every call raises: there is
no fallback path.

    packed = pack(w_bf16, importance, tile_rows, t_s, v_s, perm=None)
    y = spmm(packed, x_bf16)          # y = (W (.) M) x, bf16 [cout, batch]
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhinm.so")

HINM_ABI_VERSION = 2
HINM_PACKED_WINDOWED = 1     # flags bit: block-diagonal perms (blocks of 64), see include/hinm.h
HINM_FORMAT_VERSION = 1       # packed-buffer layout version (include/hinm.h)
HINM_NOALLOC_SCRATCH_BYTES = 65536 + (32 << 20)   # hinm_spmm_noalloc's device array (include/hinm.h)
STATUS = {0: "HINM_OK", 1: "HINM_EINVAL", 2: "HINM_ESHAPE", 3: "HINM_EPERM", 4: "HINM_EIMPORTANCE",
          5: "HINM_EALIGN", 6: "HINM_EWORKSPACE", 7: "HINM_EHIP", 8: "HINM_EDEVICE"}

# Every symbol the C ABI exports (include/hinm.h).
EXPORTS = ("hinm_abi_version", "hinm_plan", "hinm_pack_workspace_bytes", "hinm_pack",
           "hinm_spmm_workspace_bytes", "hinm_spmm", "hinm_spmm_rows", "hinm_translate_indices",
           "hinm_boundary_workspace_bytes", "hinm_boundary_search", "hinm_plan_tiles",
           "hinm_pack_tiles_workspace_bytes", "hinm_pack_tiles", "hinm_spmm_tiles_workspace_bytes",
           "hinm_spmm_tiles", "hinm_boundary_search_tiles", "hinm_gyro_workspace_bytes", "hinm_gyro_permute",
           "hinm_set_option", "hinm_get_option", "hinm_spmm_noalloc", "hinm_spmm_group_workspace_bytes",
           "hinm_spmm_group", "hinm_status_str", "hinm_last_error")

# Launch-shape options (hinm_set_option): name -> HINM_OPT_* key.
OPTIONS = {"decode_path": 1, "decode_wgs": 2, "prefill_nt": 3, "prefill_splits": 4, "prefill_path": 5,
           "prefill_per_xcd": 6, "prefill_tb_group": 7, "prefill_stagger": 8}


class HinmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class PlanT(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("cout", ctypes.c_int32), ("cin", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("n_tiles", ctypes.c_int32), ("z", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("n_dense", ctypes.c_int32), ("n_24", ctypes.c_int32),
                ("n_pruned", ctypes.c_int32), ("n_dense_pad", ctypes.c_int32), ("n_24_pad", ctypes.c_int32),
                ("kb_dense", ctypes.c_int32), ("kb_24", ctypes.c_int32),
                ("t_s", ctypes.c_double), ("v_s", ctypes.c_double), ("p_s", ctypes.c_double),
                ("bytes_val_dense", ctypes.c_int64), ("bytes_idx_dense", ctypes.c_int64),
                ("bytes_val_24", ctypes.c_int64), ("bytes_meta_24", ctypes.c_int64),
                ("bytes_idx_24", ctypes.c_int64)]


class PackedT(ctypes.Structure):
    _fields_ = [("plan", PlanT), ("val_dense", ctypes.c_void_p), ("idx_dense", ctypes.c_void_p),
                ("val_24", ctypes.c_void_p), ("meta_24", ctypes.c_void_p), ("idx_24", ctypes.c_void_p),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class TPlanT(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("cout", ctypes.c_int32), ("cin", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("n_tiles", ctypes.c_int32), ("z", ctypes.c_int32),
                ("max_n_dense_pad", ctypes.c_int32), ("max_n_24_pad", ctypes.c_int32),
                ("dense_blocks", ctypes.c_int32), ("blocks_24", ctypes.c_int32), ("t_s", ctypes.c_double),
                ("bytes_val_dense", ctypes.c_int64), ("bytes_idx_dense", ctypes.c_int64),
                ("bytes_val_24", ctypes.c_int64), ("bytes_meta_24", ctypes.c_int64),
                ("bytes_idx_24", ctypes.c_int64), ("bytes_tiles", ctypes.c_int64)]


class TPackedT(ctypes.Structure):
    _fields_ = [("plan", TPlanT), ("tiles", ctypes.c_void_p), ("val_dense", ctypes.c_void_p),
                ("idx_dense", ctypes.c_void_p), ("val_24", ctypes.c_void_p), ("meta_24", ctypes.c_void_p),
                ("idx_24", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Loads libhinm.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python structured_sparse_gemm_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        P, S, I64, I32, D, VP = (ctypes.POINTER(PlanT), ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_double, ctypes.c_void_p)
        sig = {
            "hinm_abi_version": ([], ctypes.c_int),
            "hinm_plan": ([I64, I64, I32, D, D, P], ctypes.c_int),
            "hinm_pack_workspace_bytes": ([P, ctypes.POINTER(S)], ctypes.c_int),
            "hinm_pack": ([P, VP, I64, VP, I64, VP, ctypes.POINTER(PackedT), VP, S, VP], ctypes.c_int),
            "hinm_spmm_workspace_bytes": ([P, I64, ctypes.POINTER(S)], ctypes.c_int),
            "hinm_spmm": ([ctypes.POINTER(PackedT), VP, I64, I64, VP, I64, VP, S, VP], ctypes.c_int),
            "hinm_spmm_rows": ([ctypes.POINTER(PackedT), VP, I64, I64, VP, I64, VP, VP, S, VP], ctypes.c_int),
            "hinm_translate_indices": ([ctypes.POINTER(PackedT), VP, VP, S, VP], ctypes.c_int),
            "hinm_boundary_workspace_bytes": ([I64, I64, I32, ctypes.POINTER(S)], ctypes.c_int),
            "hinm_plan_tiles": ([I64, I64, I32, D, ctypes.POINTER(D), ctypes.POINTER(TPlanT), ctypes.POINTER(I32)],
                                ctypes.c_int),
            "hinm_pack_tiles_workspace_bytes": ([ctypes.POINTER(TPlanT), ctypes.POINTER(S)], ctypes.c_int),
            "hinm_pack_tiles": ([ctypes.POINTER(TPlanT), VP, I64, VP, I64, VP, ctypes.POINTER(TPackedT), VP, S, VP],
                                ctypes.c_int),
            "hinm_spmm_tiles_workspace_bytes": ([ctypes.POINTER(TPlanT), I64, ctypes.POINTER(S)], ctypes.c_int),
            "hinm_spmm_tiles": ([ctypes.POINTER(TPackedT), VP, I64, I64, VP, I64, VP, S, VP], ctypes.c_int),
            "hinm_boundary_search_tiles": ([I64, I64, I32, D, D, VP, I64, VP, VP, S, ctypes.POINTER(D),
                                            ctypes.POINTER(I32), VP], ctypes.c_int),
            "hinm_boundary_search": ([I64, I64, I32, D, D, VP, I64, VP, VP, S, ctypes.POINTER(D),
                                      ctypes.POINTER(D), ctypes.POINTER(D), I32, ctypes.POINTER(I32), VP],
                                     ctypes.c_int),
            "hinm_gyro_workspace_bytes": ([P, I32, ctypes.POINTER(S)], ctypes.c_int),
            "hinm_gyro_permute": ([P, VP, I64, VP, I32, I32, I32, VP, VP, ctypes.POINTER(D), VP, S, VP],
                                  ctypes.c_int),
            "hinm_set_option": ([ctypes.c_int, I64], ctypes.c_int),
            "hinm_spmm_noalloc": ([ctypes.POINTER(PackedT), VP, I64, I64, VP, I64, VP], ctypes.c_int),
            "hinm_spmm_group_workspace_bytes": ([ctypes.c_int, VP, I64, ctypes.POINTER(S)], ctypes.c_int),
            "hinm_spmm_group": ([ctypes.c_int, VP, VP, I64, I64, VP, VP, VP, S, VP], ctypes.c_int),
            "hinm_get_option": ([ctypes.c_int, ctypes.POINTER(I64)], ctypes.c_int),
            "hinm_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "hinm_last_error": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = args, res
        if lib.hinm_abi_version() != HINM_ABI_VERSION:
            raise ImportError("libhinm ABI version mismatch")
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise HinmError(status, library().hinm_last_error().decode())


@dataclasses.dataclass(frozen=True)
class Plan:
    cout: int
    cin: int
    tile_rows: int
    n_tiles: int
    z: int
    groups: int
    n_dense: int
    n_24: int
    n_pruned: int
    n_dense_pad: int
    n_24_pad: int
    t_s: float
    v_s: float
    p_s: float
    bytes_val_dense: int
    bytes_idx_dense: int
    bytes_val_24: int
    bytes_meta_24: int
    bytes_idx_24: int
    raw: PlanT = dataclasses.field(repr=False, compare=False)

    @property
    def packed_bytes(self) -> int:
        return (self.bytes_val_dense + self.bytes_idx_dense + self.bytes_val_24 + self.bytes_meta_24
                + self.bytes_idx_24)


def plan(cout: int, cin: int, tile_rows: int, t_s: float, v_s: float) -> Plan:
    """Region counts (host only, needs no GPU)."""
    raw = PlanT()
    _check(library().hinm_plan(cout, cin, tile_rows, float(t_s), float(v_s), ctypes.byref(raw)))
    kw = {f.name: getattr(raw, f.name) for f in dataclasses.fields(Plan) if f.name != "raw"}
    return Plan(raw=raw, **kw)


@dataclasses.dataclass
class HinmPacked:
    """A packed weight: the plan and its five device buffers (torch tensors)."""

    plan: Plan
    val_dense: torch.Tensor   # int16 bits of bf16 [T, n_dense_pad/32, R, 32]
    idx_dense: torch.Tensor   # int32 [T, n_dense_pad]
    val_24: torch.Tensor      # int16 bits of bf16 [T, n_24_pad/64, R, 32]
    meta_24: torch.Tensor     # int64 bits of uint64 [T, n_24_pad/64, R]
    idx_24: torch.Tensor      # int32 [T, n_24_pad]
    flags: int = 0            # HINM_PACKED_* bits (set by pack)

    def struct(self) -> PackedT:
        """The C view of this weight (built once; the tensors must not be replaced afterwards)."""
        st = self.__dict__.get("_struct")
        if st is None:
            def ptr(t):
                return t.data_ptr() if t.numel() else None
            st = PackedT(self.plan.raw, ptr(self.val_dense), ptr(self.idx_dense), ptr(self.val_24),
                         ptr(self.meta_24), ptr(self.idx_24), self.flags, 0)
            self.__dict__["_struct"] = st
            self.__dict__["_ws_need"] = {}
        return st

    @property
    def device(self) -> torch.device:
        return self.idx_24.device

    def nbytes(self) -> int:
        return self.plan.packed_bytes

    def state_dict(self) -> dict:
        """Plain tensors and numbers (torch.save / torch.load(weights_only=True) round-trip them): the
        layout version, the plan's arguments and the five buffers."""
        p = self.plan
        return {"format": "hinm-packed", "format_version": HINM_FORMAT_VERSION, "cout": p.cout, "cin": p.cin,
                "tile_rows": p.tile_rows, "t_s": p.t_s, "v_s": p.v_s, "flags": int(self.flags),
                **{k: getattr(self, k) for k in _BUFFERS}}

    @classmethod
    def from_state_dict(cls, sd: dict, device=None) -> "HinmPacked":
        """Rebuilds a packed weight from state_dict() output: checks the layout version, recomputes the
        plan from its arguments and checks every buffer's dtype and shape against it."""
        _check_format(sd, "hinm-packed")
        p = plan(int(sd["cout"]), int(sd["cin"]), int(sd["tile_rows"]), float(sd["t_s"]), float(sd["v_s"]))
        T, R = p.n_tiles, p.tile_rows
        want = {"val_dense": ((T, p.n_dense_pad // 32, R, 32), torch.int16),
                "idx_dense": ((T, p.n_dense_pad), torch.int32),
                "val_24": ((T, p.n_24_pad // 64, R, 32), torch.int16),
                "meta_24": ((T, p.n_24_pad // 64, R), torch.int64),
                "idx_24": ((T, p.n_24_pad), torch.int32)}
        return cls(p, **_checked_buffers(sd, want, device), flags=int(sd.get("flags", 0)))


_BUFFERS = ("val_dense", "idx_dense", "val_24", "meta_24", "idx_24")


def _check_format(sd: dict, kind: str) -> None:
    if not isinstance(sd, dict) or sd.get("format") != kind:
        raise ValueError(f"not a stored {kind} weight")
    if sd.get("format_version") != HINM_FORMAT_VERSION:
        raise ValueError(f"stored layout version {sd.get('format_version')!r}, this library reads "
                         f"{HINM_FORMAT_VERSION}: pack the weight again")


def _checked_buffers(sd: dict, want: dict, device) -> dict:
    out = {}
    for k, (shape, dtype) in want.items():
        t = sd.get(k)
        if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape):
            got = (None if not isinstance(t, torch.Tensor) else (t.dtype, tuple(t.shape)))
            raise ValueError(f"stored buffer {k}: expected {dtype} {tuple(shape)}, found {got}")
        t = t.contiguous()
        out[k] = t.to(device) if device is not None else t
    return out


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(device: torch.device) -> int:
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _empty(shape, dtype, device):
    # 256-byte aligned by the caching allocator; zero-size buffers stay empty.
    return torch.empty(shape, dtype=dtype, device=device)


def pack_workspace_bytes(p: Plan) -> int:
    n = ctypes.c_size_t()
    _check(library().hinm_pack_workspace_bytes(ctypes.byref(p.raw), ctypes.byref(n)))
    return n.value


def alloc_packed(p: Plan, device) -> HinmPacked:
    T, R = p.n_tiles, p.tile_rows
    return HinmPacked(
        p,
        _empty((T, p.n_dense_pad // 32, R, 32), torch.int16, device),
        _empty((T, p.n_dense_pad), torch.int32, device),
        _empty((T, p.n_24_pad // 64, R, 32), torch.int16, device),
        _empty((T, p.n_24_pad // 64, R), torch.int64, device),
        _empty((T, p.n_24_pad), torch.int32, device))


def pack(w: torch.Tensor, importance: torch.Tensor, tile_rows: int, t_s: float, v_s: float,
         perm: Optional[torch.Tensor] = None) -> HinmPacked:
    """Packs a bf16 weight [cout, cin] on its device (synchronous).

    importance: fp32 [cout, cin] (finite, >= 0); perm: int32 [cout/tile_rows, cin]
    or None for the identity, perm[t][j] = original column at position j of tile t.
    """
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_cuda:
        raise ValueError("w must be a 2-D bf16 CUDA tensor")
    if importance.dtype != torch.float32 or importance.shape != w.shape or importance.device != w.device:
        raise ValueError("importance must be fp32 with the shape and device of w")
    if w.stride(1) != 1 or importance.stride(1) != 1:
        raise ValueError("w and importance must have unit column stride")
    cout, cin = w.shape
    p = plan(cout, cin, tile_rows, t_s, v_s)
    if perm is not None:
        if perm.dtype != torch.int32 or perm.shape != (p.n_tiles, cin) or perm.device != w.device:
            raise ValueError(f"perm must be int32 [{p.n_tiles}, {cin}] on the device of w")
        perm = perm.contiguous()
    out = alloc_packed(p, w.device)
    ws = torch.empty(pack_workspace_bytes(p), dtype=torch.uint8, device=w.device)
    st = out.struct()
    with torch.cuda.device(w.device):
        _check(library().hinm_pack(ctypes.byref(p.raw), w.data_ptr(), w.stride(0), importance.data_ptr(),
                                   importance.stride(0), perm.data_ptr() if perm is not None else None,
                                   ctypes.byref(st), ws.data_ptr(), ws.numel(), _stream_ptr(w.device)))
    out.flags = int(st.flags)
    return out


@dataclasses.dataclass
class TilePlan:
    """Per-tile region counts (hinm_plan_tiles): shared fields, buffer sizes and the tile table."""

    raw: TPlanT = dataclasses.field(repr=False)
    tiles: "np.ndarray"          # int32 [n_tiles, 4]: first dense block, n_dense, first 2:4 block, n_24
    v_s: tuple

    def __getattr__(self, name):
        raw = self.__dict__.get("raw")
        if raw is not None and name in dict(TPlanT._fields_):
            return getattr(raw, name)
        raise AttributeError(name)

    @property
    def packed_bytes(self) -> int:
        r = self.raw
        return r.bytes_val_dense + r.bytes_idx_dense + r.bytes_val_24 + r.bytes_meta_24 + r.bytes_idx_24


def plan_tiles(cout: int, cin: int, tile_rows: int, t_s: float, v_s) -> TilePlan:
    """Per-tile plan (host only): tile t uses v_s[t]."""
    import numpy as np
    v = [float(x) for x in v_s]
    raw = TPlanT()
    n_tiles = cout // tile_rows if tile_rows > 0 else 0
    if len(v) != n_tiles:
        raise ValueError(f"{n_tiles} per-tile v_s values are needed, got {len(v)}")
    arr = (ctypes.c_double * max(1, len(v)))(*v)
    tiles = (ctypes.c_int32 * max(1, 4 * n_tiles))()
    _check(library().hinm_plan_tiles(cout, cin, tile_rows, float(t_s), arr, ctypes.byref(raw), tiles))
    return TilePlan(raw=raw, tiles=np.ctypeslib.as_array(tiles)[:4 * n_tiles].reshape(n_tiles, 4).copy(),
                    v_s=tuple(v))


@dataclasses.dataclass
class HinmTPacked:
    """A packed weight with per-tile counts: the plan, the device tile table and five device buffers."""

    plan: TilePlan
    tiles: torch.Tensor       # int32 [T, 4] on the device
    val_dense: torch.Tensor   # int16 bits of bf16 [dense_blocks, R, 32]
    idx_dense: torch.Tensor   # int32 [dense_blocks * 32]
    val_24: torch.Tensor      # int16 bits of bf16 [blocks_24, R, 32]
    meta_24: torch.Tensor     # int64 bits of uint64 [blocks_24, R]
    idx_24: torch.Tensor      # int32 [blocks_24 * 64]

    def struct(self) -> TPackedT:
        st = self.__dict__.get("_struct")
        if st is None:
            def ptr(t):
                return t.data_ptr() if t.numel() else None
            st = TPackedT(self.plan.raw, ptr(self.tiles), ptr(self.val_dense), ptr(self.idx_dense),
                          ptr(self.val_24), ptr(self.meta_24), ptr(self.idx_24))
            self.__dict__["_struct"] = st
            self.__dict__["_ws_need"] = {}
        return st

    @property
    def device(self) -> torch.device:
        return self.tiles.device

    def nbytes(self) -> int:
        return self.plan.packed_bytes

    def state_dict(self) -> dict:
        """As HinmPacked.state_dict, with the per-tile v_s and the tile table."""
        p = self.plan
        return {"format": "hinm-packed-tiles", "format_version": HINM_FORMAT_VERSION, "cout": p.cout,
                "cin": p.cin, "tile_rows": p.tile_rows, "t_s": p.t_s,
                "v_s": torch.tensor(p.v_s, dtype=torch.float64), "tiles": self.tiles,
                **{k: getattr(self, k) for k in _BUFFERS}}

    @classmethod
    def from_state_dict(cls, sd: dict, device=None) -> "HinmTPacked":
        _check_format(sd, "hinm-packed-tiles")
        v = sd.get("v_s")
        if not isinstance(v, torch.Tensor):
            raise ValueError("stored per-tile v_s missing")
        p = plan_tiles(int(sd["cout"]), int(sd["cin"]), int(sd["tile_rows"]), float(sd["t_s"]), v.tolist())
        R = p.tile_rows
        want = {"tiles": ((p.n_tiles, 4), torch.int32),
                "val_dense": ((p.dense_blocks, R, 32), torch.int16),
                "idx_dense": ((p.dense_blocks * 32,), torch.int32),
                "val_24": ((p.blocks_24, R, 32), torch.int16),
                "meta_24": ((p.blocks_24, R), torch.int64),
                "idx_24": ((p.blocks_24 * 64,), torch.int32)}
        bufs = _checked_buffers(sd, want, device)
        if not np.array_equal(bufs["tiles"].cpu().numpy(), p.tiles):
            raise ValueError("stored tile table does not match the per-tile plan")
        return cls(p, **bufs)


def pack_tiles(w: torch.Tensor, importance: torch.Tensor, tile_rows: int, t_s: float, v_s,
               perm: Optional[torch.Tensor] = None) -> HinmTPacked:
    """Packs a bf16 weight with one v_s per tile (hinm_pack_tiles, synchronous)."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_cuda:
        raise ValueError("w must be a 2-D bf16 CUDA tensor")
    if importance.dtype != torch.float32 or importance.shape != w.shape or importance.device != w.device:
        raise ValueError("importance must be fp32 with the shape and device of w")
    if w.stride(1) != 1 or importance.stride(1) != 1:
        raise ValueError("w and importance must have unit column stride")
    cout, cin = w.shape
    p = plan_tiles(cout, cin, tile_rows, t_s, v_s)
    if perm is not None:
        if perm.dtype != torch.int32 or perm.shape != (p.n_tiles, cin) or perm.device != w.device:
            raise ValueError(f"perm must be int32 [{p.n_tiles}, {cin}] on the device of w")
        perm = perm.contiguous()
    dev, R = w.device, tile_rows
    out = HinmTPacked(p, torch.from_numpy(p.tiles).to(dev),
                      _empty((p.dense_blocks, R, 32), torch.int16, dev), _empty((p.dense_blocks * 32,), torch.int32, dev),
                      _empty((p.blocks_24, R, 32), torch.int16, dev), _empty((p.blocks_24, R), torch.int64, dev),
                      _empty((p.blocks_24 * 64,), torch.int32, dev))
    n = ctypes.c_size_t()
    _check(library().hinm_pack_tiles_workspace_bytes(ctypes.byref(p.raw), ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
    st = out.struct()
    with torch.cuda.device(dev):
        _check(library().hinm_pack_tiles(ctypes.byref(p.raw), w.data_ptr(), w.stride(0), importance.data_ptr(),
                                         importance.stride(0), perm.data_ptr() if perm is not None else None,
                                         ctypes.byref(st), ws.data_ptr(), ws.numel(), _stream_ptr(dev)))
    return out


def spmm_tiles_workspace_bytes(p: TilePlan, batch: int) -> int:
    n = ctypes.c_size_t()
    _check(library().hinm_spmm_tiles_workspace_bytes(ctypes.byref(p.raw), batch, ctypes.byref(n)))
    return n.value


def spmm_workspace_bytes(p: Plan, batch: int) -> int:
    n = ctypes.c_size_t()
    _check(library().hinm_spmm_workspace_bytes(ctypes.byref(p.raw), batch, ctypes.byref(n)))
    return n.value


_ws_cache = {}
_ws_retired = []
_opt_gen = 0


def get_option(name: str) -> int:
    """Current value of a launch-shape option (see OPTIONS and hinm_set_option)."""
    v = ctypes.c_int64()
    _check(library().hinm_get_option(OPTIONS[name], ctypes.byref(v)))
    return v.value


def set_option(name: str, value: int) -> None:
    """Sets a process-wide launch-shape option (hinm_set_option)."""
    global _opt_gen
    _check(library().hinm_set_option(OPTIONS[name], int(value)))
    _opt_gen += 1          # workspace sizes remembered per weight depend on the options


class options:
    """Context manager: ``with options(prefill_splits=2): ...`` sets options and restores them on exit."""

    def __init__(self, **kw):
        for k in kw:
            if k not in OPTIONS:
                raise KeyError(f"unknown option {k!r}; known: {sorted(OPTIONS)}")
        self.kw = kw
        self.saved = {}

    def __enter__(self):
        for k, v in self.kw.items():
            self.saved[k] = get_option(k)
            set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            set_option(k, v)
        return False


def _workspace(device: torch.device, stream: int, nbytes: int) -> Optional[torch.Tensor]:
    """The default workspace of (device, stream): zero-filled when made, at least nbytes.

    One per stream, because a workspace holds the split reduction's arrival
    counters and partial sums, so products that may overlap (different
    streams) must not share one.  A buffer that is outgrown is kept alive, not
    freed: HIP graphs captured earlier, or work still queued, may name it.
    """
    if nbytes == 0:
        return None
    key = (device.index, stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _ws_retired.append(buf)
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def spmm(packed: HinmPacked, x: torch.Tensor, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None, out_rows: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = (W (.) M) X: x bf16 [cin, batch] (row stride >= batch), returns bf16 [cout, batch].

    With ``out_rows`` (int32 [cout] on the device, a permutation), row r of the
    product is written to row out_rows[r] of Y (hinm_spmm_rows).
    Asynchronous on the current stream.  ``workspace`` (uint8, device, zero-filled before its first use) may
    be given; otherwise each stream has its own default workspace, so products on different streams may
    overlap.  The per-call host work is kept to argument checks and one C call, so that small products are
    not bound by Python.
    """
    p = packed.plan
    dev = x.device
    tiled = isinstance(packed, HinmTPacked)
    if tiled and out_rows is not None:
        raise ValueError("out_rows is not supported with per-tile counts")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[0] != p.cin or dev != packed.idx_24.device:
        raise ValueError(f"x must be bf16 [{p.cin}, batch] on {packed.device}")
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    batch = x.shape[1]
    if out is None:
        out = torch.empty((p.cout, batch), dtype=torch.bfloat16, device=dev)
    elif out.dtype != torch.bfloat16 or out.shape != (p.cout, batch) or out.stride(1) != 1 or out.device != dev:
        raise ValueError(f"out must be bf16 [{p.cout}, {batch}] with unit column stride on {dev}")
    if out_rows is not None and (out_rows.dtype != torch.int32 or out_rows.shape != (p.cout,)
                                 or not out_rows.is_contiguous() or out_rows.device != dev):
        raise ValueError(f"out_rows must be a contiguous int32 [{p.cout}] tensor on {dev}")
    st = packed.struct()
    need_cache = packed.__dict__["_ws_need"]
    need = need_cache.get((batch, _opt_gen))
    if need is None:
        need = need_cache[(batch, _opt_gen)] = (spmm_tiles_workspace_bytes(p, batch) if tiled else
                                                spmm_workspace_bytes(p, batch))
    stream = _stream_ptr(dev)
    if workspace is None:
        workspace = _workspace(dev, stream, need)
    lib = library()
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_n = workspace.numel() if workspace is not None else 0
    ldx = max(x.stride(0), batch) if batch else 0
    ldy = max(out.stride(0), batch) if batch else 0
    if tiled:
        call, args = lib.hinm_spmm_tiles, (ctypes.byref(st), x.data_ptr(), batch, ldx, out.data_ptr(), ldy, ws_ptr,
                                           ws_n, stream)
    elif out_rows is None:
        call, args = lib.hinm_spmm, (ctypes.byref(st), x.data_ptr(), batch, ldx, out.data_ptr(), ldy, ws_ptr, ws_n,
                                     stream)
    else:
        call, args = lib.hinm_spmm_rows, (ctypes.byref(st), x.data_ptr(), batch, ldx, out.data_ptr(), ldy,
                                          out_rows.data_ptr(), ws_ptr, ws_n, stream)
    if dev.index is None or dev.index == torch.cuda.current_device():
        _check(call(*args))
    else:
        with torch.cuda.device(dev):
            _check(call(*args))
    return out


class Group:
    """Several packed weights that multiply the same activations (hinm_spmm_group), e.g. the q, k and v
    projections of a layer.  Holds the C array of weight pointers; the weights must stay alive."""

    def __init__(self, packed):
        self.packed = list(packed)
        if not 1 <= len(self.packed) <= 8:
            raise ValueError("a group holds 1 to 8 packed weights")
        if any(isinstance(p, HinmTPacked) for p in self.packed):
            raise ValueError("groups take uniform packed weights (pack, not pack_tiles)")
        self.structs = [p.struct() for p in self.packed]
        self.ptrs = (ctypes.c_void_p * len(self.structs))(*[ctypes.addressof(st) for st in self.structs])
        self._need = {}

    def workspace_bytes(self, batch: int) -> int:
        key = (batch, _opt_gen)
        if key not in self._need:
            n = ctypes.c_size_t()
            _check(library().hinm_spmm_group_workspace_bytes(len(self.packed), self.ptrs, batch, ctypes.byref(n)))
            self._need[key] = n.value
        return self._need[key]


def spmm_group(group: Group, x: torch.Tensor, outs=None, workspace: Optional[torch.Tensor] = None):
    """[(W_g (.) M_g) X for g in the group]: x bf16 [cin, batch]; returns (or fills) one bf16 [cout_g, batch]
    output per weight.  Asynchronous on the current stream; workspace as in spmm."""
    ws0 = group.packed[0]
    p0 = ws0.plan
    dev = x.device
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[0] != p0.cin or dev != ws0.device or x.stride(1) != 1:
        raise ValueError(f"x must be bf16 [{p0.cin}, batch] with unit column stride on {ws0.device}")
    batch = x.shape[1]
    if outs is None:
        outs = [torch.empty((pk.plan.cout, batch), dtype=torch.bfloat16, device=dev) for pk in group.packed]
    for pk, o in zip(group.packed, outs):
        if o.dtype != torch.bfloat16 or o.shape != (pk.plan.cout, batch) or o.stride(1) != 1 or o.device != dev:
            raise ValueError(f"each output must be bf16 [cout, {batch}] with unit column stride on {dev}")
    if len(outs) != len(group.packed):
        raise ValueError("one output per weight")
    need = group.workspace_bytes(batch)
    stream = _stream_ptr(dev)
    if workspace is None:
        workspace = _workspace(dev, stream, need)
    ys = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    ldys = (ctypes.c_int64 * len(outs))(*[max(o.stride(0), batch) if batch else 0 for o in outs])
    ldx = max(x.stride(0), batch) if batch else 0
    with torch.cuda.device(dev):
        _check(library().hinm_spmm_group(len(outs), group.ptrs, x.data_ptr(), batch, ldx, ys, ldys,
                                         workspace.data_ptr() if workspace is not None else None,
                                         workspace.numel() if workspace is not None else 0, stream))
    return outs


def spmm_noalloc(packed: HinmPacked, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Y = (W (.) M) X into ``out`` through hinm_spmm_noalloc: no workspace, no device allocation (the
    scratch is the library's own device array, shared by every call on the device, so calls on different
    streams of one device must not overlap).  x bf16 [cin, batch], out bf16 [cout, batch], both with unit
    column stride.  Asynchronous on the current stream."""
    p = packed.plan
    dev = x.device
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[0] != p.cin or dev != packed.device or x.stride(1) != 1:
        raise ValueError(f"x must be bf16 [{p.cin}, batch] with unit column stride on {packed.device}")
    batch = x.shape[1]
    if out.dtype != torch.bfloat16 or out.shape != (p.cout, batch) or out.stride(1) != 1 or out.device != dev:
        raise ValueError(f"out must be bf16 [{p.cout}, {batch}] with unit column stride on {dev}")
    ldx = max(x.stride(0), batch) if batch else 0
    ldy = max(out.stride(0), batch) if batch else 0
    with torch.cuda.device(dev):
        _check(library().hinm_spmm_noalloc(ctypes.byref(packed.struct()), x.data_ptr(), batch, ldx, out.data_ptr(),
                                           ldy, _stream_ptr(dev)))
    return out


def translate_indices(packed: HinmPacked, mapping: torch.Tensor) -> HinmPacked:
    """Rewrites the packed index lists in place through ``mapping`` (int32 [cin] permutation on the device):
    index i becomes mapping[i], pads stay -1 (hinm_translate_indices).  Synchronous; returns ``packed``."""
    p = packed.plan
    dev = packed.idx_24.device
    if mapping.dtype != torch.int32 or mapping.shape != (p.cin,) or not mapping.is_contiguous() or mapping.device != dev:
        raise ValueError(f"mapping must be a contiguous int32 [{p.cin}] tensor on {dev}")
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = packed.struct()
        _check(library().hinm_translate_indices(ctypes.byref(st), mapping.data_ptr(), ws.data_ptr(),
                                                ws.numel(), _stream_ptr(dev)))
    packed.flags = int(st.flags)
    return packed


def boundary_search(importance: torch.Tensor, perm: Optional[torch.Tensor], tile_rows: int, t_s: float,
                    step: float = 0.01, trace_cap: int = 256):
    """Device boundary search for v_s (hinm_boundary_search).  importance fp32 [cout, cin] and perm int32
    [n_tiles, cin] (or None) on the device.  Returns (v_s, [(v, R_total), ...] of the grid points visited)."""
    if importance.dtype != torch.float32 or importance.dim() != 2 or importance.stride(1) != 1:
        raise ValueError("importance must be float32 [cout, cin] with unit column stride")
    cout, cin = importance.shape
    dev = importance.device
    if perm is not None and (perm.dtype != torch.int32 or not perm.is_contiguous() or perm.device != dev):
        raise ValueError("perm must be a contiguous int32 tensor on the importance's device")
    lib = library()
    n = ctypes.c_size_t()
    _check(lib.hinm_boundary_workspace_bytes(cout, cin, tile_rows, ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
    v = ctypes.c_double()
    tv = (ctypes.c_double * trace_cap)()
    tr = (ctypes.c_double * trace_cap)()
    tl = ctypes.c_int32()
    with torch.cuda.device(dev):
        _check(lib.hinm_boundary_search(cout, cin, tile_rows, float(t_s), float(step), importance.data_ptr(),
                                        importance.stride(0), perm.data_ptr() if perm is not None else None,
                                        ws.data_ptr(), ws.numel(), ctypes.byref(v), tv, tr, trace_cap,
                                        ctypes.byref(tl), _stream_ptr(dev)))
    k = min(tl.value, trace_cap)
    return v.value, [(tv[i], tr[i]) for i in range(k)]


def gyro_permute(importance: torch.Tensor, perm: torch.Tensor, tile_rows: int, t_s: float, v_s: float,
                 rounds: int, cluster_size: int, kmeans_iters: int, sample, init):
    """In-tile input-channel gyro permutation (hinm_gyro_permute), synchronous.

    importance fp32 [cout, cin] and perm int32 [n_tiles, cin] on the device; sample uint8
    [rounds, n_tiles, groups] and init int32 [rounds, n_tiles, n_clusters] (numpy, host).
    Returns (new perm tensor, cost trace float64 numpy [rounds + 1, n_tiles]); perm is not modified.
    """
    if importance.dtype != torch.float32 or importance.dim() != 2 or importance.stride(1) != 1:
        raise ValueError("importance must be float32 [cout, cin] with unit column stride")
    cout, cin = importance.shape
    dev = importance.device
    p = plan(cout, cin, tile_rows, t_s, v_s)
    if perm.dtype != torch.int32 or perm.shape != (p.n_tiles, cin) or perm.device != dev:
        raise ValueError(f"perm must be int32 [{p.n_tiles}, {cin}] on the importance's device")
    out = perm.clone().contiguous()
    sample = np.ascontiguousarray(sample, dtype=np.uint8)
    init = np.ascontiguousarray(init, dtype=np.int32)
    lib = library()
    n = ctypes.c_size_t()
    _check(lib.hinm_gyro_workspace_bytes(ctypes.byref(p.raw), int(cluster_size), ctypes.byref(n)))
    ws = torch.empty(max(1, n.value), dtype=torch.uint8, device=dev)
    trace = np.zeros((rounds + 1, p.n_tiles), dtype=np.float64)
    with torch.cuda.device(dev):
        _check(lib.hinm_gyro_permute(ctypes.byref(p.raw), importance.data_ptr(), importance.stride(0),
                                     out.data_ptr(), int(rounds), int(cluster_size), int(kmeans_iters),
                                     sample.ctypes.data if sample.size else None,
                                     init.ctypes.data if init.size else None,
                                     trace.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), ws.data_ptr(),
                                     ws.numel(), _stream_ptr(dev)))
    return out, trace


def boundary_search_tiles(importance: torch.Tensor, perm: Optional[torch.Tensor], tile_rows: int, t_s: float,
                          step: float = 0.01):
    """Per-tile device boundary search (hinm_boundary_search_tiles).  Returns (v_s per tile, grid points per tile)."""
    if importance.dtype != torch.float32 or importance.dim() != 2 or importance.stride(1) != 1:
        raise ValueError("importance must be float32 [cout, cin] with unit column stride")
    cout, cin = importance.shape
    dev = importance.device
    if perm is not None and (perm.dtype != torch.int32 or not perm.is_contiguous() or perm.device != dev):
        raise ValueError("perm must be a contiguous int32 tensor on the importance's device")
    lib = library()
    n = ctypes.c_size_t()
    _check(lib.hinm_boundary_workspace_bytes(cout, cin, tile_rows, ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev)
    T = cout // tile_rows
    v = (ctypes.c_double * max(1, T))()
    pts = (ctypes.c_int32 * max(1, T))()
    with torch.cuda.device(dev):
        _check(lib.hinm_boundary_search_tiles(cout, cin, tile_rows, float(t_s), float(step), importance.data_ptr(),
                                              importance.stride(0), perm.data_ptr() if perm is not None else None,
                                              ws.data_ptr(), ws.numel(), v, pts, _stream_ptr(dev)))
    return [v[i] for i in range(T)], [pts[i] for i in range(T)]


__all__ = ["HinmError", "HinmPacked", "Plan", "plan", "pack", "spmm", "spmm_noalloc", "Group", "spmm_group", "set_option", "get_option", "options",
           "OPTIONS", "translate_indices", "boundary_search", "plan_tiles", "pack_tiles", "boundary_search_tiles",
           "HinmTPacked", "TilePlan", "spmm_tiles_workspace_bytes", "alloc_packed",
           "pack_workspace_bytes",
           "spmm_workspace_bytes", "library", "LIB_PATH", "EXPORTS"]
