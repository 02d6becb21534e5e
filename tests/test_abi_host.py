"""The C ABI on a host without a GPU: exports, region counts, host-side errors."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle.hinm as oh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
hinm = pytest.importorskip("structured_sparse_gemm_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hinm.LIB_PATH):
        pytest.skip("libhinm.so is not built (run __graft_entry__.build())")
    return hinm.library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hinm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hinm_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(hinm.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.hinm_abi_version() == hinm.HINM_ABI_VERSION == 2


@pytest.mark.parametrize("shape", [(128, 256, 32, 0.75, 0.5), (4096, 4096, 64, 0.5, 0.25),
                                   (11008, 4096, 64, 0.75, 0.55), (4096, 11008, 64, 0.75, 0.55),
                                   (4096, 11008, 64, 0.6, 0.4), (64, 4, 16, 0.5, 0.0), (16, 8, 16, 0.0, 0.0)])
def test_plan_matches_oracle(lib, shape):
    p = hinm.plan(*shape)
    o = oh.plan(*shape)
    for f in ("cout", "cin", "tile_rows", "n_tiles", "z", "groups", "n_dense", "n_24", "n_pruned",
              "n_dense_pad", "n_24_pad"):
        assert getattr(p, f) == getattr(o, f), f
    T, R = o.n_tiles, o.tile_rows
    assert p.bytes_val_dense == T * o.n_dense_pad * R * 2
    assert p.bytes_val_24 == T * o.n_24_pad // 2 * R * 2
    assert p.bytes_meta_24 == T * o.n_24_pad // 64 * R * 8


def test_plan_matches_oracle_random(lib):
    rng = np.random.default_rng(99)
    for _ in range(2000):
        cin = 4 * int(rng.integers(1, 6000))
        t = float(rng.uniform(0, 0.999))
        v = float(rng.uniform(max(0, 2 * t - 1), t))
        if rng.random() < 0.1:
            v = t
        p, o = hinm.plan(64, cin, 64, t, v), oh.plan(64, cin, 64, t, v)
        assert (p.z, p.n_dense, p.n_24, p.n_pruned) == (o.z, o.n_dense, o.n_24, o.n_pruned), (cin, t, v)


@pytest.mark.parametrize("args,status", [
    ((64, 256, 24, 0.5, 0.25), "HINM_ESHAPE"),
    ((100, 256, 64, 0.5, 0.25), "HINM_ESHAPE"),
    ((64, 254, 64, 0.5, 0.25), "HINM_ESHAPE"),
    ((0, 256, 64, 0.5, 0.25), "HINM_ESHAPE"),
    ((64, 256, 64, 0.5, 0.6), "HINM_EINVAL"),
    ((64, 256, 64, 0.75, 0.4), "HINM_EINVAL"),
    ((64, 256, 64, 1.0, 0.99), "HINM_EINVAL"),
    ((64, 256, 64, float("nan"), 0.0), "HINM_EINVAL"),
    ((64, 256, 64, 0.5, float("inf")), "HINM_EINVAL"),
])
def test_plan_errors(lib, args, status):
    with pytest.raises(hinm.HinmError) as e:
        hinm.plan(*args)
    assert e.value.name == status
    assert lib.hinm_last_error().decode()


def test_status_strings(lib):
    for s in range(9):
        assert lib.hinm_status_str(s).decode().startswith(hinm.STATUS[s])


def _fake_packed(p, base=1 << 20):
    """A packed struct whose pointers are never dereferenced (host checks fail first)."""
    return hinm.PackedT(p.raw, base, base, base, base, base)


def test_spmm_host_errors(lib):
    p = hinm.plan(4096, 4096, 64, 0.5, 0.25)
    pk = _fake_packed(p)
    call = lambda **kw: lib.hinm_spmm(ctypes.byref(kw.get("pk", pk)), kw.get("x", 4096), kw.get("batch", 16),
                                      kw.get("ldx", 16), kw.get("y", 4096), kw.get("ldy", 16),
                                      kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(batch=-1) == 2
    assert call(ldx=8) == 2
    assert call(ldy=8) == 2
    assert call(x=None) == 1
    assert call(x=4097) == 5
    assert call(pk=_fake_packed(p, base=(1 << 20) + 8)) == 5
    assert call(pk=hinm.PackedT(p.raw, None, None, None, None, None)) == 1
    # the prefill path runs without a workspace; the split decode path needs one
    assert hinm.spmm_workspace_bytes(p, 2048) == 0
    assert hinm.spmm_workspace_bytes(p, 16) > 0
    # tile_rows 48 takes the generic path, which splits K through the workspace
    p48 = hinm.plan(96 * 8, 4096, 48, 0.5, 0.25)
    need = hinm.spmm_workspace_bytes(p48, 100)
    assert need > 0
    pk48 = _fake_packed(p48)
    assert call(pk=pk48, batch=100, ldx=100, ldy=100, ws=None, wsb=0) == 6
    assert call(pk=pk48, batch=100, ldx=100, ldy=100, ws=1 << 20, wsb=need - 1) == 6
    assert call(pk=pk48, batch=100, ldx=100, ldy=100, ws=(1 << 20) + 16, wsb=need) == 5
    assert call(batch=0, ldx=0, ldy=0) == 0          # empty batch is a no-op
    bad = hinm.PlanT.from_buffer_copy(p.raw)
    bad.n_dense += 1
    assert call(pk=hinm.PackedT(bad, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)) == 1
    bad = hinm.PlanT.from_buffer_copy(p.raw)
    bad.abi_version = hinm.HINM_ABI_VERSION + 1
    assert call(pk=hinm.PackedT(bad, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)) == 1


def test_spmm_rows_and_translate_host_errors(lib):
    """The output-row and index-translation entry points check their extra arguments on the host."""
    p = hinm.plan(4096, 4096, 64, 0.5, 0.25)
    pk = _fake_packed(p)
    rows = lambda **kw: lib.hinm_spmm_rows(ctypes.byref(kw.get("pk", pk)), kw.get("x", 4096), kw.get("batch", 2048),
                                           kw.get("ldx", 2048), kw.get("y", 4096), kw.get("ldy", 2048),
                                           kw.get("out_rows", 1 << 20), kw.get("ws", None), kw.get("wsb", 0), None)
    assert rows(out_rows=None) == 1
    assert rows(out_rows=(1 << 20) + 2) == 5
    assert rows(batch=-1) == 2                      # then everything hinm_spmm checks
    assert rows(x=None) == 1
    assert rows(batch=0, ldx=0, ldy=0) == 0
    tr = lambda **kw: lib.hinm_translate_indices(ctypes.byref(kw.get("pk", pk)), kw.get("map", 1 << 20),
                                                 kw.get("ws", 1 << 20), kw.get("wsb", 256), None)
    assert tr(map=None) == 1
    assert tr(map=(1 << 20) + 2) == 5
    assert tr(ws=None) == 6
    assert tr(wsb=255) == 6
    assert tr(ws=(1 << 20) + 16) == 5
    assert tr(pk=hinm.PackedT(p.raw, None, None, None, None, None)) == 1
    bad = hinm.PlanT.from_buffer_copy(p.raw)
    bad.n_24 += 4
    assert tr(pk=hinm.PackedT(bad, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)) == 1


def test_boundary_search_host_errors(lib):
    n = ctypes.c_size_t()
    assert lib.hinm_boundary_workspace_bytes(4096, 11008, 64, ctypes.byref(n)) == 0
    T, C = 64, 11008
    assert n.value >= T * C * (8 + 4 + 1) + 2 * T * C * 4
    assert lib.hinm_boundary_workspace_bytes(4096, 11007, 64, ctypes.byref(n)) == 2   # cin % 4
    v = ctypes.c_double()
    tv, tr, tl = (ctypes.c_double * 4)(), (ctypes.c_double * 4)(), ctypes.c_int32()
    lib.hinm_boundary_workspace_bytes(4096, 11008, 64, ctypes.byref(n))
    call = lambda **kw: lib.hinm_boundary_search(
        kw.get("cout", 4096), kw.get("cin", 11008), 64, kw.get("t_s", 0.7), kw.get("step", 0.01),
        kw.get("imp", 1 << 20), kw.get("ldi", 11008), kw.get("perm", None), kw.get("ws", 1 << 20),
        kw.get("wsb", n.value), ctypes.byref(v), kw.get("tv", tv), kw.get("tr", tr), kw.get("cap", 4),
        ctypes.byref(tl), None)
    assert call(imp=None) == 1
    assert call(step=0.0) == 1
    assert call(step=float("nan")) == 1
    assert call(cap=-1) == 1
    assert call(tv=None) == 1
    assert call(t_s=1.0) == 1
    assert call(ldi=11000) == 2
    assert call(imp=(1 << 20) + 2) == 5
    assert call(ws=None) == 6
    assert call(wsb=n.value - 1) == 6
    assert call(ws=(1 << 20) + 16) == 5


def test_pack_host_errors(lib):
    p = hinm.plan(128, 256, 32, 0.75, 0.5)
    wsb = hinm.pack_workspace_bytes(p)
    assert wsb >= p.n_tiles * p.cin * 9
    out = _fake_packed(p)
    call = lambda **kw: lib.hinm_pack(ctypes.byref(p.raw), kw.get("w", 1 << 20), kw.get("ldw", 256),
                                      kw.get("imp", 1 << 20), kw.get("ldi", 256), kw.get("perm", None),
                                      ctypes.byref(kw.get("out", out)), kw.get("ws", 1 << 20),
                                      kw.get("wsb", wsb), None)
    assert call(w=None) == 1
    assert call(ldw=255) == 2
    assert call(imp=(1 << 20) + 2) == 5
    assert call(ws=None) == 6
    assert call(wsb=wsb - 1) == 6
    assert call(ws=(1 << 20) + 64) == 5
    assert call(out=hinm.PackedT(p.raw, None, None, None, None, None)) == 1


def test_workspace_sizes(lib):
    counters = 16384 * 4
    p = hinm.plan(11008, 4096, 64, 0.75, 0.55)
    for b in (0, 2048, 4096):                  # 1376 and 2752 work items: no K split
        assert hinm.spmm_workspace_bytes(p, b) == 0
    assert hinm.spmm_workspace_bytes(p, 65) == 0        # 172 items of 128 tokens: more than 128, no split
    # 128 items of 128 tokens: split 4 ways; per item and split 256 threads x 32 fp32 partials
    assert hinm.spmm_workspace_bytes(hinm.plan(4096, 11008, 64, 0.75, 0.55), 200) == counters + 4 * 128 * 256 * 128
    for b in (1, 16, 64):
        assert hinm.spmm_workspace_bytes(p, b) % 4 == 0
    q = hinm.plan(4096, 4096, 64, 0.5, 0.25)   # 64 items at batch 128: split 4 ways
    assert hinm.spmm_workspace_bytes(q, 128) == counters + 4 * 64 * 256 * 128
    assert hinm.spmm_workspace_bytes(q, 512) == 0     # 256 items: no split
    with hinm.options(prefill_splits=1):
        assert hinm.spmm_workspace_bytes(q, 128) == 0
    assert hinm.spmm_workspace_bytes(q, 128) == counters + 4 * 64 * 256 * 128
    p = hinm.plan(96, 4096, 48, 0.75, 0.55)
    assert hinm.spmm_workspace_bytes(p, 200) % 256 == 0


def test_plan_tiles_matches_oracle():
    """Per-tile counts and block offsets equal the oracle's per-tile plan, on random shapes and v_s."""
    import oracle.hinm as oh
    rng = np.random.default_rng(5)
    for _ in range(200):
        R = int(rng.choice([16, 32, 64]))
        T = int(rng.integers(1, 9))
        cin = 4 * int(rng.integers(1, 600))
        t_s = float(rng.uniform(0, 0.95))
        lo = max(0.0, 2 * t_s - 1)
        v = [float(x) for x in rng.uniform(lo, t_s, T)]
        tp = hinm.plan_tiles(T * R, cin, R, t_s, v)
        plans = oh.plan_tiles(T * R, cin, R, t_s, v)
        kd = ks = 0
        for t, pl in enumerate(plans):
            assert tuple(tp.tiles[t]) == (kd, pl.n_dense, ks, pl.n_24)
            kd += pl.n_dense_pad // 32
            ks += pl.n_24_pad // 64
        assert (tp.dense_blocks, tp.blocks_24) == (kd, ks)
        assert tp.max_n_dense_pad == max(pl.n_dense_pad for pl in plans)
        assert tp.max_n_24_pad == max(pl.n_24_pad for pl in plans)
        assert tp.z == plans[0].z
        assert tp.bytes_val_24 == ks * R * 64 and tp.bytes_meta_24 == ks * R * 8 and tp.bytes_idx_dense == kd * 128


def test_tiles_host_errors(lib):
    v = (ctypes.c_double * 4)(0.5, 0.55, 0.6, 0.8)          # 0.8 > t_s
    raw, tiles = hinm.TPlanT(), (ctypes.c_int32 * 16)()
    assert lib.hinm_plan_tiles(256, 512, 64, 0.75, v, ctypes.byref(raw), tiles) == 1
    assert b"tile 3" in lib.hinm_last_error()
    assert lib.hinm_plan_tiles(256, 512, 64, 0.75, None, ctypes.byref(raw), tiles) == 1
    tp = hinm.plan_tiles(256, 512, 64, 0.75, [0.5, 0.55, 0.6, 0.7])
    n = ctypes.c_size_t()
    assert lib.hinm_pack_tiles_workspace_bytes(ctypes.byref(tp.raw), ctypes.byref(n)) == 0
    assert n.value >= 4 * 512 * 9
    assert lib.hinm_spmm_tiles_workspace_bytes(ctypes.byref(tp.raw), 2048, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.hinm_spmm_tiles_workspace_bytes(ctypes.byref(tp.raw), 16, ctypes.byref(n)) == 0
    bad = hinm.TPlanT.from_buffer_copy(tp.raw)
    bad.blocks_24 += 1                                      # sizes no longer consistent
    assert lib.hinm_pack_tiles_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == 1
    bad = hinm.TPlanT.from_buffer_copy(tp.raw)
    bad.z += 1
    assert lib.hinm_spmm_tiles_workspace_bytes(ctypes.byref(bad), 16, ctypes.byref(n)) == 1
    pk = hinm.TPackedT(tp.raw, None, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    call = lambda **kw: lib.hinm_spmm_tiles(ctypes.byref(kw.get("pk", pk)), 1 << 20, kw.get("batch", 16), 16,
                                            1 << 20, 16, kw.get("ws", 1 << 20), 1 << 24, None)
    assert call() == 1                                      # no tile table
    pk2 = hinm.TPackedT(tp.raw, (1 << 20) + 2, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    assert call(pk=pk2) == 5
    pk3 = hinm.TPackedT(tp.raw, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    assert call(pk=pk3, batch=-1) == 2
    out = hinm.TPackedT(tp.raw, None, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    assert lib.hinm_pack_tiles(ctypes.byref(tp.raw), 1 << 20, 512, 1 << 20, 512, None, ctypes.byref(out),
                               1 << 20, 1 << 24, None) == 1


def test_gyro_host_errors(lib):
    p = hinm.plan(128, 256, 32, 0.75, 0.5)          # 32 groups per tile, 4 tiles
    n = ctypes.c_size_t()
    assert lib.hinm_gyro_workspace_bytes(ctypes.byref(p.raw), 0, ctypes.byref(n)) == 1
    assert lib.hinm_gyro_workspace_bytes(ctypes.byref(p.raw), 8, ctypes.byref(n)) == 0
    G, T, N, rounds = p.groups, p.n_tiles, 4, 2           # N = ceil(32 / 8)
    assert G == 32 and T == 4
    sample = np.zeros((rounds, T, G), np.uint8)
    init = np.tile(np.arange(N, dtype=np.int32), (rounds, T, 1))
    trace = (ctypes.c_double * ((rounds + 1) * T))()

    def call(**kw):
        s = kw.get("sample", sample)
        i = kw.get("init", init)
        return lib.hinm_gyro_permute(ctypes.byref(p.raw), kw.get("imp", 1 << 20), kw.get("ldi", 256),
                                     kw.get("perm", 1 << 21), kw.get("rounds", rounds), kw.get("cs", 8),
                                     kw.get("iters", 2), s.ctypes.data if s is not None else None,
                                     i.ctypes.data if i is not None else None, trace, kw.get("ws", 1 << 22),
                                     kw.get("wsb", n.value), None)
    assert call(ws=None) == 6                        # the valid draws pass every check before the workspace one
    assert call(imp=None) == 1
    assert call(perm=None) == 1
    assert call(rounds=-1) == 1
    assert call(cs=0) == 1
    assert call(iters=0) == 1
    assert call(sample=None) == 1
    bad = sample.copy()
    bad[1, 2, 5] = 4
    assert call(sample=bad) == 1                     # a position outside 0..3
    dup = init.copy()
    dup[0, 1, 2] = dup[0, 1, 0]
    assert call(init=dup) == 1                       # centroids must start at distinct groups
    oob = init.copy()
    oob[1, 3, 1] = G
    assert call(init=oob) == 1
    assert call(ldi=255) == 2
    assert call(imp=(1 << 20) + 2) == 5
    assert call(ws=None) == 6
    assert call(wsb=n.value - 1) == 6
    assert call(ws=(1 << 22) + 16) == 5


def test_options_set_get_and_reject(lib):
    """Launch options through the C ABI: read back what was set, refuse unknown keys and out-of-range
    values (leaving the option unchanged), and the workspace size follows the setting."""
    import ctypes
    v = ctypes.c_int64()
    for name, key in hinm.OPTIONS.items():
        assert lib.hinm_get_option(key, ctypes.byref(v)) == 0
        before = v.value
        assert lib.hinm_set_option(key, -3) == 1
        assert lib.hinm_get_option(key, ctypes.byref(v)) == 0 and v.value == before
        assert hinm.get_option(name) == before
    assert lib.hinm_set_option(0, 1) == 1 and lib.hinm_set_option(len(hinm.OPTIONS) + 1, 1) == 1
    assert lib.hinm_get_option(2, None) == 1
    q = hinm.plan(4096, 4096, 64, 0.5, 0.25)
    base = hinm.spmm_workspace_bytes(q, 128)
    with hinm.options(prefill_splits=2, prefill_nt=128):
        assert hinm.get_option("prefill_splits") == 2
        assert hinm.spmm_workspace_bytes(q, 128) == 16384 * 4 + 2 * 64 * 256 * 128
    assert hinm.get_option("prefill_splits") == 0 and hinm.spmm_workspace_bytes(q, 128) == base
    with pytest.raises(hinm.HinmError):
        hinm.set_option("prefill_nt", 192)
    with pytest.raises(KeyError):
        hinm.options(no_such_option=1)


def test_noalloc_host_checks(lib):
    """hinm_spmm_noalloc's host-side checks, before any launch: a NULL weight, batch 0 (a no-op), every
    default launch shape of the configured workloads fits the static scratch array, and a product whose
    scratch need exceeds it (only under forced options) is refused with HINM_EWORKSPACE."""
    import ctypes
    assert lib.hinm_spmm_noalloc(None, 16, 16, 16, 16, 16, None) == 1
    for cout, cin, R, t, v in ((4096, 4096, 64, 0.5, 0.25), (11008, 4096, 64, 0.75, 0.55),
                               (4096, 11008, 64, 0.75, 0.55), (2048, 4096, 64, 0.75, 0.55),
                               (960, 1024, 48, 0.5, 0.25), (128, 256, 32, 0.75, 0.5)):
        p = hinm.plan(cout, cin, R, t, v)
        for b in (1, 16, 17, 33, 64, 65, 100, 128, 129, 256, 300, 1000, 1024, 2048, 3000, 4096):
            assert hinm.spmm_workspace_bytes(p, b) <= hinm.HINM_NOALLOC_SCRATCH_BYTES, (cout, cin, b)
    p = hinm.plan(11008, 4096, 64, 0.75, 0.55)
    pk = hinm.PackedT(p.raw, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20)
    assert lib.hinm_spmm_noalloc(ctypes.byref(pk), 1 << 20, 0, 0, 1 << 20, 0, None) == 0
    with hinm.options(prefill_splits=4):
        # 1376 items of 256 tokens, each split 4 ways: 344 MiB of partials
        assert hinm.spmm_workspace_bytes(p, 2048) > hinm.HINM_NOALLOC_SCRATCH_BYTES
        assert lib.hinm_spmm_noalloc(ctypes.byref(pk), 1 << 20, 2048, 2048, 1 << 20, 2048, None) == 6
        assert b"allocation-free" in lib.hinm_last_error()


def test_group_host_errors(lib):
    """hinm_spmm_group's host-side checks (before any launch): weight count, NULL entries, unequal cin
    or tile_rows, NULL outputs, ldy below the batch; batch 0 is a no-op."""
    import ctypes
    p1 = hinm.plan(256, 1024, 64, 0.75, 0.55)
    p2 = hinm.plan(128, 1024, 64, 0.5, 0.25)
    p3 = hinm.plan(128, 512, 64, 0.5, 0.25)
    fake = 1 << 20
    k1, k2, k3 = (hinm.PackedT(p.raw, fake, fake, fake, fake, fake) for p in (p1, p2, p3))
    arr = lambda *ks: (ctypes.c_void_p * len(ks))(*[ctypes.addressof(k) for k in ks])
    ys = (ctypes.c_void_p * 2)(fake, fake)
    ldy = (ctypes.c_int64 * 2)(16, 16)
    n = ctypes.c_size_t()
    assert lib.hinm_spmm_group_workspace_bytes(0, arr(k1), 16, ctypes.byref(n)) == 1
    assert lib.hinm_spmm_group_workspace_bytes(9, arr(*([k1] * 9)), 16, ctypes.byref(n)) == 1
    assert lib.hinm_spmm_group_workspace_bytes(2, arr(k1, k2), 16, ctypes.byref(n)) == 0
    assert n.value >= max(hinm.spmm_workspace_bytes(p1, 16), hinm.spmm_workspace_bytes(p2, 16))
    assert lib.hinm_spmm_group(2, arr(k1, k3), fake, 16, 16, ys, ldy, None, 0, None) == 2     # unequal cin
    assert lib.hinm_spmm_group(2, None, fake, 16, 16, ys, ldy, None, 0, None) == 1
    assert lib.hinm_spmm_group(2, arr(k1, k2), fake, 16, 16, None, ldy, None, 0, None) == 1
    assert lib.hinm_spmm_group(2, arr(k1, k2), fake, 16, 16, ys, (ctypes.c_int64 * 2)(16, 8), None, 0, None) == 2
    assert lib.hinm_spmm_group(2, arr(k1, k2), fake, 16, 16, (ctypes.c_void_p * 2)(fake, None), ldy, None, 0,
                               None) == 1
    assert lib.hinm_spmm_group(2, arr(k1, k2), fake, 0, 0, ys, (ctypes.c_int64 * 2)(0, 0), None, 0, None) == 0
    bad = hinm.PackedT(p2.raw, fake, None, fake, fake, fake)
    assert lib.hinm_spmm_group(2, arr(k1, bad), fake, 16, 16, ys, ldy, None, 0, None) == 1


def test_group_size_limits(lib):
    """hinm_spmm_group takes 1 to 8 weights; other counts fail on the host before any launch."""
    p = hinm.plan(4096, 4096, 64, 0.5, 0.25)
    pks = [_fake_packed(p) for _ in range(9)]
    ptrs = (ctypes.c_void_p * 9)(*[ctypes.addressof(k) for k in pks])
    ys = (ctypes.c_void_p * 9)(*([1 << 20] * 9))
    ldys = (ctypes.c_int64 * 9)(*([16] * 9))
    for n in (0, 9, -1):
        assert lib.hinm_spmm_group(n, ptrs, 1 << 20, 16, 16, ys, ldys, None, 0, None) == 1
        assert "weights" in lib.hinm_last_error().decode()
    with pytest.raises(ValueError):
        hinm.Group([object()] * 9)


@pytest.mark.parametrize("rblocks", [64, 200, 257, 300, 344, 511, 512])
def test_split_decode_workspace_follows_the_split_rule(lib, rblocks):
    """The split decode's partial-sum planes, read back through the workspace query: a power-of-two split
    for about 256 workgroups (each keeping >= 4 K-blocks); when row blocks x splits fall strictly between 256
    and 512, the last row blocks take twice the splits (two planes more than one split needs), at every
    batch up to 64."""
    cout, cin = 64 * rblocks, 2048
    p = hinm.plan(cout, cin, 64, 0.75, 0.55)
    nblk = p.n_dense_pad // 32 + p.n_24_pad // 64
    splits = 1
    while splits < 64 and rblocks * splits * 2 <= 256 and nblk // (splits * 2) >= 4:
        splits *= 2
    mixed = rblocks * splits < 512 < 2 * rblocks * splits and nblk // (2 * splits) >= 4
    planes = 2 * splits if mixed else splits
    for b, nt in ((1, 16), (16, 16), (17, 32), (32, 32), (40, 64), (64, 64)):
        want = 0 if planes == 1 else 65536 + planes * cout * nt * 4
        assert hinm.spmm_workspace_bytes(p, b) == want, (rblocks, b)


@pytest.mark.parametrize("rblocks,batch,mixed", [(150, 200, True), (150, 129, True), (150, 128, False),
                                                 (100, 200, False), (255, 200, True), (172, 512, False)])
def test_prefill_workspace_follows_the_two_count_rule(lib, rblocks, batch, mixed):
    """The batch > 64 kernel's two split counts, read back through the workspace query: with 128-token
    items in two or more token blocks and between 256 and 512 items, each XCD's first items run whole and
    the rest in two halves (so that the XCD has one piece per workgroup of 64), and partial sums are kept
    for the halved items only; otherwise no workspace (more than 128 items, one split)."""
    cout, cin = 64 * rblocks, 2048
    p = hinm.plan(cout, cin, 64, 0.75, 0.55)
    got = hinm.spmm_workspace_bytes(p, batch)
    if not mixed:
        assert got == 0
        return
    items = rblocks * -(-batch // 128)
    n_half = 0
    for x in range(8):
        nx = (x + 1) * items // 8 - x * items // 8
        n_half += nx - min(nx, max(0, 2 * nx - 64))
    assert got == 65536 + 2 * n_half * 256 * 128
