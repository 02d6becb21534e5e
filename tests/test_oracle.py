"""Pins of the CPU oracle against what the pages and mathematics fix (CPU only).

Every check here is independent of the oracle's own code path: closed forms,
invariants, brute force over tiny inputs, special cases that reduce to a
library routine, and a fixture worked by hand from the pages' rules.  The
mutation tests at the end plant plausible mistakes in the oracle (on the CPU)
and confirm that a pin catches each one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.hinm as oh
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(w_bf16: torch.Tensor) -> np.ndarray:
    return w_bf16.contiguous().view(torch.int16).numpy().view(np.uint16)


def run_pack(w: synth.Workload, v_s=None):
    p = oh.plan(w.cout, w.cin, w.tile_rows, w.t_s, w.v_s if v_s is None else v_s)
    packed, inter = oh.pack(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), p,
                            with_intermediates=True)
    return p, packed, inter


# --------------------------------------------------------------------------------------
# Closed form of the region counts (FlexHiNM-GP notes, key design 1)
# --------------------------------------------------------------------------------------

def check_counts(cin, t_s, v_s):
    p = oh.plan(64, cin, 64, t_s, v_s)
    assert p.n_dense + p.n_24 + p.n_pruned == cin
    assert p.n_24 % 4 == 0 and min(p.n_dense, p.n_24, p.n_pruned) >= 0
    # 2:4 vectors lose half their entries: zeros = pruned + n_24 / 2 exactly.
    assert 2 * p.z == 2 * p.n_pruned + p.n_24
    assert abs(Fraction(p.z, cin) - Fraction(t_s)) <= Fraction(1, 2 * cin)
    # The page's identity t = v + (1 - v) p / 2 holds exactly for the realised fractions.
    v_eff = Fraction(p.n_pruned, cin)
    if p.n_dense + p.n_24:
        p_eff = Fraction(p.n_24, p.n_dense + p.n_24)
        assert v_eff + (1 - v_eff) * p_eff / 2 == Fraction(p.z, cin)
    assert abs(p.n_pruned - v_s * cin) <= 1.5 + 1e-9
    assert abs(p.n_24 - 2 * (t_s - v_s) * cin) <= 2 + 1e-9
    return p


def test_counts_closed_form_random():
    rng = np.random.default_rng(7)
    for _ in range(400):
        cin = 4 * int(rng.integers(1, 3000))
        t = float(rng.uniform(0, 0.99))
        lo = max(0.0, 2 * t - 1)
        v = float(rng.uniform(lo, t))
        check_counts(cin, t, v)


def test_counts_exact_when_integral():
    # When t*cin and (t - v)*cin/2 are integers the realised fractions equal the page's.
    for cin, t, v in [(4096, 0.5, 0.25), (4096, 0.75, 0.5), (256, 0.75, 0.5), (1024, 0.625, 0.375)]:
        p = check_counts(cin, t, v)
        assert p.n_pruned == v * cin
        assert abs(p.n_24 / (p.n_24 + p.n_dense) - 2 * (t - v) / (1 - v)) < 1e-12
        assert abs(p.p_s - 2 * (t - v) / (1 - v)) < 1e-15


def test_counts_endpoints():
    # v = t gives p = 0 (no 2:4 region, vector pruning only);
    # v = 2t - 1 gives p = 1 (no dense region: HiNM-V, vector pruning then uniform 2:4).
    for cin, t in [(4096, 0.75), (11008, 0.75), (256, 0.6), (4096, 0.5)]:
        p = oh.plan(64, cin, 64, t, t)
        assert p.n_24 == 0 and p.n_dense == cin - p.z
        p = oh.plan(64, cin, 64, t, max(0.0, 2 * t - 1))
        assert p.n_dense <= 2, p   # only rounding slack remains
        if (t * cin) % 1 == 0 and ((1 - t) * cin) % 2 == 0:
            assert p.n_dense == 0


def test_counts_of_the_workloads():
    # The region counts of the LLaMA-7B-shaped workloads follow from the same formula.
    assert (lambda p: (p.n_dense, p.n_24, p.n_pruned))(oh.plan(128, 256, 32, 0.75, 0.5)) == (0, 128, 128)
    assert (lambda p: (p.n_dense, p.n_24, p.n_pruned))(oh.plan(4096, 4096, 64, 0.5, 0.25)) == (1024, 2048, 1024)
    assert (lambda p: (p.n_dense, p.n_24, p.n_pruned))(oh.plan(11008, 4096, 64, 0.75, 0.55)) == (204, 1640, 2252)
    assert (lambda p: (p.n_dense, p.n_24, p.n_pruned))(oh.plan(4096, 11008, 64, 0.75, 0.55)) == (550, 4404, 6054)


@pytest.mark.parametrize("args", [
    (64, 256, 48, 0.5, 0.25),    # tile_rows not a multiple of 16... 48 is; cout % 48 != 0
    (64, 254, 64, 0.5, 0.25),    # cin % 4
    (64, 256, 64, 0.5, 0.6),     # v > t
    (64, 256, 64, 0.75, 0.4),    # v < 2t - 1
    (64, 256, 64, 1.0, 0.99),    # t = 1
    (64, 256, 64, float("nan"), 0.0),
])
def test_plan_rejects(args):
    with pytest.raises(oracle.OracleError):
        oh.plan(*args)


# --------------------------------------------------------------------------------------
# Hand-worked fixture
# --------------------------------------------------------------------------------------

def handworked():
    g = json.load(open(os.path.join(GOLDEN, "handworked_16x8.json")))
    R, C = g["cout"], g["cin"]
    w = np.array([[(r + 1) + c / 8 for c in range(C)] for r in range(R)], dtype=np.float32)
    base = np.array(g["base"], dtype=np.float32)
    d = np.tile(base, (R, 1))
    a, b = g["odd_row_swap"]
    d[1::2, a], d[1::2, b] = base[b], base[a]
    x = np.array([[c + 1, (-1) ** c] for c in range(C)], dtype=np.float64)
    return g, w, d, x


def test_handworked_fixture():
    g, w, d, x = handworked()
    p = oh.plan(g["cout"], g["cin"], g["tile_rows"], g["t_s"], g["v_s"])
    for k, v in g["counts"].items():
        assert getattr(p, k) == v, k
    wb = bits_of(torch.from_numpy(w).to(torch.bfloat16))
    packed, inter = oh.pack(wb, d, np.array([g["perm"]]), p, with_intermediates=True)
    assert inter["scores"][0].tolist() == g["scores"]
    reg = inter["regions"][0]
    assert sorted(np.nonzero(reg == oh.DENSE)[0].tolist()) == g["dense"]
    assert sorted(np.nonzero(reg == oh.TWO_FOUR)[0].tolist()) == g["two_four"]
    assert sorted(np.nonzero(reg == oh.PRUNED)[0].tolist()) == g["pruned"]
    assert packed["idx_dense"][0, :2].tolist() == g["idx_dense"]
    assert (packed["idx_dense"][0, 2:] == -1).all()
    assert packed["idx_24"][0, :4].tolist() == g["idx_24"]
    assert (packed["idx_24"][0, 4:] == -1).all()
    meta = packed["meta_24"][0, 0]
    assert all(int(meta[r]) == int(g["meta_even"], 16) for r in range(0, 16, 2))
    assert all(int(meta[r]) == int(g["meta_odd"], 16) for r in range(1, 16, 2))
    for r in range(16):
        cols = g["val24_even_cols"] if r % 2 == 0 else g["val24_odd_cols"]
        assert packed["val_24"][0, 0, r, :2].tolist() == [int(wb[r, c]) for c in cols]
        assert (packed["val_24"][0, 0, r, 2:] == 0).all()
        assert packed["val_dense"][0, 0, r, :2].tolist() == [int(wb[r, 3]), int(wb[r, 7])]
        kept = g["kept_even"] if r % 2 == 0 else g["kept_odd"]
        assert np.nonzero(inter["mask"][r])[0].tolist() == kept
    # Y by a brute-force sum over the hand-derived kept set.
    y = oh.spmm(oh.unpack(packed, p), x)
    for r in range(16):
        kept = g["kept_even"] if r % 2 == 0 else g["kept_odd"]
        for n in range(2):
            assert y[r, n] == math.fsum(float(w[r, c]) * x[c, n] for c in kept)


# --------------------------------------------------------------------------------------
# Invariants and brute force
# --------------------------------------------------------------------------------------

def check_sparsity(p, inter):
    kept = inter["mask"].sum(axis=1)
    assert (kept == p.cin - p.z).all()
    assert p.cout * p.cin - int(inter["mask"].sum()) == p.cout * p.z   # achieved sparsity is Z/cin exactly


def check_region_order(p, inter):
    s, reg = inter["scores"], inter["regions"]
    for t in range(p.n_tiles):
        sd, s4, sp = s[t][reg[t] == oh.DENSE], s[t][reg[t] == oh.TWO_FOUR], s[t][reg[t] == oh.PRUNED]
        assert sd.size == p.n_dense and s4.size == p.n_24 and sp.size == p.n_pruned
        if sd.size and s4.size:
            assert sd.min() >= s4.max()
        if s4.size and sp.size:
            assert s4.min() >= sp.max()
        if sd.size and sp.size:
            assert sd.min() >= sp.max()


def check_24(p, packed, d, perm):
    """Exactly two kept per group; the kept pair maximises retained importance."""
    if p.groups == 0:
        return
    nib_all = []
    for t in range(p.n_tiles):
        for q in range(p.n_24_pad // 4):
            kb, ql = divmod(q, 16)
            nib = (packed["meta_24"][t, kb] >> np.uint64(4 * ql)) & np.uint64(0xF)
            if q >= p.groups:
                assert (nib == oh.PAD_NIBBLE).all()
                assert (packed["val_24"][t, kb, :, 2 * ql:2 * ql + 2] == 0).all()
                continue
            nib_all.append(nib)
            cols = packed["idx_24"][t, 4 * q:4 * q + 4]
            rows = np.arange(t * p.tile_rows, (t + 1) * p.tile_rows)
            a = d[np.ix_(rows, cols)].astype(np.float64)
            i0, i1 = (nib & np.uint64(3)).astype(int), (nib >> np.uint64(2)).astype(int)
            assert (i0 < i1).all()
            best = np.max([a[:, u] + a[:, v] for u, v in itertools.combinations(range(4), 2)], axis=0)
            got = a[np.arange(len(rows)), i0] + a[np.arange(len(rows)), i1]
            assert np.array_equal(got, best)
    u = np.unique(np.concatenate(nib_all)).tolist()
    assert set(u) <= set(oh.LEGAL_NIBBLES)


def test_invariants_random_small():
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        cin = 4 * int(rng.integers(8, 40))
        t = float(rng.uniform(0.3, 0.9))
        v = float(rng.uniform(max(0, 2 * t - 1), t))
        w = synth.small(64, cin, 32, t, v, 3, seed)
        p, packed, inter = run_pack(w)
        check_sparsity(p, inter)
        check_region_order(p, inter)
        check_24(p, packed, w.importance.numpy(), w.perm.numpy())
        assert np.array_equal(oh.unpack(packed, p), oh.masked_weight(bits_of(w.w_bf16), inter["mask"]))


def test_workload_tiny_invariants():
    w = synth.tiny()
    p, packed, inter = run_pack(w)
    check_sparsity(p, inter)
    check_region_order(p, inter)
    check_24(p, packed, w.importance.numpy(), w.perm.numpy())


def test_regions_brute_force():
    """Kept set = max-sum subset; dense set = max-sum subset of the kept ones (ties: lowest columns)."""
    rng = np.random.default_rng(3)
    for trial in range(40):
        cin = 12
        t = float(rng.choice([0.5, 0.625, 0.75]))
        v = float(rng.uniform(max(0, 2 * t - 1), t))
        p = oh.plan(16, cin, 16, t, v)
        # integer-valued importance makes ties frequent
        d = rng.integers(0, 3, size=(16, cin)).astype(np.float32)
        s = oh.vector_scores(d, p)[0]
        reg = oh.regions(s[None, :], p)[0]

        def best_subset(cands, k):
            best = None
            for sub in itertools.combinations(sorted(cands), k):
                key = (sum(s[list(sub)]), [-c for c in sub])
                if best is None or key > best[0]:
                    best = (key, sub)
            return set(best[1])
        kept = best_subset(range(cin), cin - p.n_pruned)
        dense = best_subset(kept, p.n_dense)
        assert set(np.nonzero(reg != oh.PRUNED)[0].tolist()) == kept
        assert set(np.nonzero(reg == oh.DENSE)[0].tolist()) == dense


def test_scores_brute_force():
    rng = np.random.default_rng(5)
    d = rng.random((32, 8), dtype=np.float32) * np.float32(1e3)
    p = oh.plan(32, 8, 16, 0.5, 0.25)
    s = oh.vector_scores(d, p)
    for t in range(2):
        for c in range(8):
            acc = 0.0
            for r in range(16):
                acc += float(d[16 * t + r, c])
            assert s[t, c] == acc


def test_topk_special_case():
    """t=0.5, v=0, identity perm, D=|W|: the mask is the plain 2:4 top-2 of the N:M article."""
    w = synth.small(64, 128, 32, 0.5, 0.0, 2, 11, identity_perm=True)
    p, packed, inter = run_pack(w)
    assert p.n_24 == 128 and p.n_dense == 0 and p.n_pruned == 0
    wf = w.w_bf16.to(torch.float32)
    wr = wf.view(64, 32, 4)
    _, top = torch.topk(wr.abs(), k=2, dim=-1)
    ref = torch.zeros_like(wr).scatter_(-1, top, 1.0).view(64, 128).bool().numpy()
    # Compare groups whose four magnitudes are distinct, so the library's unspecified
    # tie order cannot matter; almost every group qualifies.
    srt = np.sort(wr.abs().numpy(), axis=-1)
    tie_free = (np.diff(srt, axis=-1) > 0).all(axis=-1)          # [64, 32]
    assert tie_free.mean() > 0.95
    got = inter["mask"].reshape(64, 32, 4)[tie_free]
    assert np.array_equal(got, ref.reshape(64, 32, 4)[tie_free])


def test_permutation_invariance():
    """Relabelling input channels (W columns, D columns, X rows, perm) leaves Y unchanged."""
    w = synth.small(128, 96, 32, 0.6, 0.3, 5, 21)
    p, packed, inter = run_pack(w)
    x = synth.as_f64(w.x_bf16)
    y = oh.spmm(oh.unpack(packed, p), x)
    rng = np.random.default_rng(1)
    sig = rng.permutation(w.cin)
    inv = np.argsort(sig)
    wb2 = bits_of(w.w_bf16)[:, sig]
    d2 = w.importance.numpy()[:, sig]
    perm2 = inv[w.perm.numpy()]
    packed2 = oh.pack(wb2, d2, perm2, p)
    y2 = oh.spmm(oh.unpack(packed2, p), x[sig])
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_no_24_region_independent_of_perm():
    w = synth.small(64, 64, 32, 0.5, 0.5, 4, 2)
    p, packed, inter = run_pack(w)
    assert p.n_24 == 0
    other = np.stack([np.random.default_rng(t).permutation(64) for t in range(2)])
    packed2 = oh.pack(bits_of(w.w_bf16), w.importance.numpy(), other, p)
    x = synth.as_f64(w.x_bf16)
    assert np.array_equal(oh.spmm(oh.unpack(packed, p), x), oh.spmm(oh.unpack(packed2, p), x))


def test_dense_special_case_matches_library_gemm():
    w = synth.small(64, 64, 32, 0.0, 0.0, 7, 4)
    p, packed, inter = run_pack(w)
    assert p.n_dense == 64 and p.z == 0
    x = synth.as_f64(w.x_bf16)
    y = oh.spmm(oh.unpack(packed, p), x)
    ref = torch.matmul(w.w_bf16.to(torch.float64), w.x_bf16.to(torch.float64)).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-15)


def test_gemm_brute_force():
    w = synth.small(32, 16, 16, 0.5, 0.25, 3, 9)
    p, packed, inter = run_pack(w)
    wh = oh.unpack(packed, p)
    x = synth.as_f64(w.x_bf16)
    y = oh.spmm(wh, x)
    for r in range(32):
        for n in range(3):
            ref = math.fsum(wh[r, c] * x[c, n] for c in range(16))
            assert abs(y[r, n] - ref) <= 1e-14 * max(1.0, abs(ref))


def test_pack_rejects_bad_inputs():
    w = synth.small(64, 32, 32, 0.5, 0.25, 1, 0)
    p = oh.plan(64, 32, 32, 0.5, 0.25)
    bad = w.perm.numpy().copy()
    bad[1, 0] = bad[1, 1]
    with pytest.raises(oracle.OracleError):
        oh.pack(bits_of(w.w_bf16), w.importance.numpy(), bad, p)
    d = w.importance.numpy().copy()
    d[3, 3] = -1.0
    with pytest.raises(oracle.OracleError):
        oh.pack(bits_of(w.w_bf16), d, w.perm.numpy(), p)
    d[3, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oh.pack(bits_of(w.w_bf16), d, w.perm.numpy(), p)


# --------------------------------------------------------------------------------------
# Boundary search (FlexHiNM-GP notes, key design 1)
# --------------------------------------------------------------------------------------

def test_boundary_search_rule_and_grid():
    """Early stop = last grid point before the first strict decrease, and near the grid max.

    The FlexHiNM-GP notes claim the objective is concave (proof in an appendix
    that is not on the page), which would make the early stop the grid argmax.
    On these synthetic weights it is concave only up to wiggles of about 1e-4
    relative near its plateau, so the check is the stopping rule itself plus a
    bound on the gap to the full scan.
    """
    w = synth.draw("dps", 256, 704, 64, 0.7, None, 1, 5, n_outliers=35, importance="sq")
    v, trace = oh.boundary_search(w.importance.numpy(), w.perm.numpy(), w.cout, w.cin, 64, 0.7)
    grid = oh.boundary_grid(w.importance.numpy(), w.perm.numpy(), w.cout, w.cin, 64, 0.7)
    assert trace[0][0] == 0.7 and trace == grid[:len(trace)]
    k = next((i for i in range(len(grid) - 1) if grid[i + 1][1] < grid[i][1]), len(grid) - 1)
    pv = oh.plan(w.cout, w.cin, 64, 0.7, v)
    pk = oh.plan(w.cout, w.cin, 64, 0.7, grid[k][0])
    assert (pv.n_dense, pv.n_24, pv.n_pruned) == (pk.n_dense, pk.n_24, pk.n_pruned)
    assert v == pk.n_pruned / w.cin
    # the snapped value re-plans to the same counts
    assert oh.plan(w.cout, w.cin, 64, 0.7, v).n_24 == pv.n_24
    best = max(r for _, r in grid)
    assert grid[k][1] >= (1 - 1e-3) * best
    # coarse concavity: the objective rises from v = t_s, then falls toward v = 2 t_s - 1
    assert grid[0][1] < grid[k][1] and grid[-1][1] < grid[k][1]


def test_boundary_first_group_never_loses():
    """With one 2:4 group per tile, R_total cannot fall below its value at v_s = t_s.

    The single group holds the two weakest dense vectors and the two strongest
    pruned ones; keeping the top two of four per row retains at least what the
    two dense vectors held.  A planted sign or index mistake breaks this.
    """
    rng = np.random.default_rng(17)
    for trial in range(10):
        cin, t = 64, 0.5
        d = (rng.random((64, cin)) ** 3).astype(np.float32)
        perm = np.stack([rng.permutation(cin)])
        p0 = oh.plan(64, cin, 64, t, t)
        p1 = oh.plan(64, cin, 64, t, t - 2 / cin)
        assert p1.groups == 1
        assert oh.retained_importance(d, perm, p1) >= oh.retained_importance(d, perm, p0)


def test_retained_importance_brute_force():
    w = synth.small(32, 16, 16, 0.5, 0.25, 1, 13, importance="sq")
    p, packed, inter = run_pack(w)
    d = w.importance.numpy().astype(np.float64)
    m = inter["mask"]
    # retained importance = sum of importance over kept entries (dense vectors entirely).
    assert oh.retained_importance(w.importance.numpy(), w.perm.numpy(), p) == pytest.approx(
        float(np.sum(d[m])), rel=1e-12)


# --------------------------------------------------------------------------------------
# Mutation tests: a planted mistake in the oracle must trip a pin.
# --------------------------------------------------------------------------------------

def _mut_regions_ascending(s, p):
    reg = np.full((p.n_tiles, p.cin), oh.PRUNED, dtype=np.uint8)
    for t in range(p.n_tiles):
        order = np.argsort(s[t], kind="stable")          # wrong sign
        reg[t, order[:p.n_dense]] = oh.DENSE
        reg[t, order[p.n_dense:p.n_dense + p.n_24]] = oh.TWO_FOUR
    return reg


def _mut_select24_smallest(d, idx_s, p):
    sel = np.zeros((p.cout, p.groups, 2), dtype=np.int64)
    for t in range(p.n_tiles):
        rows = slice(t * p.tile_rows, (t + 1) * p.tile_rows)
        a = np.asarray(d, np.float32)[rows][:, idx_s[t, :p.n_24]].reshape(p.tile_rows, p.groups, 4)
        sel[rows] = np.sort(np.argsort(a, axis=-1, kind="stable")[..., :2], axis=-1)
    return sel


def _mut_scores_drop_last_row(d, p):
    d3 = np.asarray(d, np.float32).reshape(p.n_tiles, p.tile_rows, p.cin)
    return d3[:, :-1, :].astype(np.float64).sum(axis=1)


def _mut_index_lists_ignore_perm(reg, perm, p):
    ident = np.tile(np.arange(p.cin), (p.n_tiles, 1))
    return oracle.hinm.__dict__["_orig_index_lists"](reg, ident, p)


@pytest.mark.parametrize("name,fn", [
    ("regions", _mut_regions_ascending),
    ("select24", _mut_select24_smallest),
    ("vector_scores", _mut_scores_drop_last_row),
])
def test_mutations_are_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oh, name, fn)
    caught = False
    try:
        test_invariants_random_small()
        test_handworked_fixture()
        test_scores_brute_force()
    except AssertionError:
        caught = True
    assert caught, f"planted mistake in {name} went unnoticed"


def test_mutation_perm_ignored_is_caught(monkeypatch):
    monkeypatch.setattr(oh, "_orig_index_lists", oh.index_lists, raising=False)
    monkeypatch.setattr(oh, "index_lists", _mut_index_lists_ignore_perm)
    with pytest.raises(AssertionError):
        test_handworked_fixture()


def test_mutation_transposed_product_is_caught(monkeypatch):
    monkeypatch.setattr(oh, "spmm", lambda w, x: (np.asarray(x, np.float64).T @ np.asarray(w, np.float64).T).T[:, ::-1])
    with pytest.raises(AssertionError):
        test_gemm_brute_force()


# --------------------------------------------------------------------------------------
# Output-channel permutation at write-out and cross-layer index translation
# (FlexHiNM-GP notes, key designs 2 and 4; highlights)
# --------------------------------------------------------------------------------------

def test_scatter_rows_brute_force():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((7, 3))
    out_rows = rng.permutation(7)
    res = oh.scatter_rows(y, out_rows)
    for r in range(7):
        assert np.array_equal(res[out_rows[r]], y[r])
    assert np.array_equal(oh.scatter_rows(y, np.arange(7)), y)
    with pytest.raises(ValueError):
        oh.scatter_rows(y, np.array([0, 0, 1, 2, 3, 4, 5]))


def test_translate_indices_brute_force():
    rng = np.random.default_rng(4)
    mapping = rng.permutation(12)
    idx = np.array([[3, -1, 0, 11], [7, 7, -1, -1]])
    out = oh.translate_indices(idx, mapping)
    for (i, j), v in np.ndenumerate(idx):
        assert out[i, j] == (-1 if v < 0 else mapping[v])
    with pytest.raises(ValueError):
        oh.translate_indices(idx, np.zeros(12, dtype=np.int64))


def test_two_layer_chain_permuted_storage():
    """Layer A writes its rows through out_rows = sigma; layer B, whose indices are translated by
    mapping = sigma (channel c is stored at row sigma[c]), reads the stored activations and produces
    exactly the product over activations in channel order.  Integer-valued inputs keep every sum exact."""
    rng = np.random.default_rng(5)
    wa = synth.small(64, 32, 32, 0.5, 0.25, 4, 31)
    wb = synth.small(32, 64, 32, 0.5, 0.25, 4, 32)
    pa, packed_a, _ = run_pack(wa)
    pb, packed_b, _ = run_pack(wb)
    x = rng.integers(-3, 4, size=(32, 4)).astype(np.float64)
    wa_hat = np.round(oh.unpack(packed_a, pa) * 8)      # small integers: exact float64 sums
    ya = oh.spmm(wa_hat, x)                              # activations in channel order [64 x 4]
    sigma = rng.permutation(64)
    stored = oh.scatter_rows(ya, sigma)                  # row sigma[c] holds channel c
    pk_t = dict(packed_b)
    pk_t["idx_dense"] = oh.translate_indices(packed_b["idx_dense"], sigma)
    pk_t["idx_24"] = oh.translate_indices(packed_b["idx_24"], sigma)
    wb_hat = np.round(oh.unpack(packed_b, pb) * 8)
    wb_hat_t = np.round(oh.unpack(pk_t, pb) * 8)         # columns moved to the stored rows
    assert np.array_equal(oh.spmm(wb_hat_t, stored), oh.spmm(wb_hat, ya))
    # the translation is not the identity, so the check above is not vacuous
    assert not np.array_equal(wb_hat_t, wb_hat)


def test_mutation_translate_inverse_is_caught(monkeypatch):
    orig = oh.translate_indices
    monkeypatch.setattr(oh, "translate_indices", lambda idx, m: orig(idx, np.argsort(m)))
    with pytest.raises(AssertionError):
        test_two_layer_chain_permuted_storage()


def test_mutation_scatter_as_gather_is_caught(monkeypatch):
    monkeypatch.setattr(oh, "scatter_rows", lambda y, r: np.asarray(y)[np.asarray(r)])
    with pytest.raises(AssertionError):
        test_scatter_rows_brute_force()
    with pytest.raises(AssertionError):
        test_two_layer_chain_permuted_storage()


# --------------------------------------------------------------------------------------
# Per-tile v_s (FlexHiNM-GP notes, "整体框架": region ratios decided inside each tile)
# --------------------------------------------------------------------------------------

def test_pack_tiles_equal_v_is_the_uniform_pack():
    """With one v_s for every tile the per-tile layout is the uniform layout with the tile axis folded."""
    w = synth.small(256, 512, 64, 0.75, 0.55, 4, 71)
    p, packed, inter = run_pack(w)
    plans = oh.plan_tiles(w.cout, w.cin, 64, 0.75, [0.55] * p.n_tiles)
    pt, it = oh.pack_tiles(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), plans, with_intermediates=True)
    nkd, nks = p.n_dense_pad // 32, p.n_24_pad // 64
    assert np.array_equal(pt["val_dense"], packed["val_dense"].reshape(-1, 64, 32))
    assert np.array_equal(pt["idx_dense"], packed["idx_dense"].reshape(-1))
    assert np.array_equal(pt["val_24"], packed["val_24"].reshape(-1, 64, 32))
    assert np.array_equal(pt["meta_24"], packed["meta_24"].reshape(-1, 64))
    assert np.array_equal(pt["idx_24"], packed["idx_24"].reshape(-1))
    assert np.array_equal(pt["tiles"][:, 0], np.arange(p.n_tiles) * nkd)
    assert np.array_equal(pt["tiles"][:, 2], np.arange(p.n_tiles) * nks)
    assert np.array_equal(it["mask"], inter["mask"])


def test_pack_tiles_invariants_random_v():
    """Random per-tile v_s: every row keeps cin - z entries, each tile has its closed-form counts, every
    2:4 group keeps exactly two, and the unpacked weight is W on the mask."""
    rng = np.random.default_rng(72)
    cout, cin, R, t_s = 192, 256, 32, 0.7
    w = synth.small(cout, cin, R, t_s, 0.5, 3, 73)
    lo = 2 * t_s - 1
    v = [float(x) for x in rng.uniform(max(0.0, lo), t_s, cout // R)]
    plans = oh.plan_tiles(cout, cin, R, t_s, v)
    pk, inter = oh.pack_tiles(bits_of(w.w_bf16), w.importance.numpy(), w.perm.numpy(), plans,
                              with_intermediates=True)
    m = inter["mask"]
    z = math.floor(t_s * cin + 0.5)
    assert np.all(m.sum(axis=1) == cin - z)
    assert len({(pl.n_dense, pl.n_24) for pl in plans}) > 1          # the counts really differ
    for t, pl in enumerate(plans):
        g = math.floor((t_s - v[t]) * cin / 2 + 0.5)
        g = max(0, min(g, min(z, cin - z) // 2))
        assert (pl.n_24, pl.n_pruned, pl.n_dense) == (4 * g, z - 2 * g, cin - z - 2 * g)
        assert tuple(pk["tiles"][t, [1, 3]]) == (pl.n_dense, pl.n_24)
        # each 2:4 group of the tile keeps exactly two per row
        kd, _, ks, n24 = pk["tiles"][t]
        cols = pk["idx_24"][64 * ks:64 * ks + n24].reshape(-1, 4)
        rows = m[t * R:(t + 1) * R]
        for grp in cols:
            assert np.all(rows[:, grp].sum(axis=1) == 2)
    wh = oh.unpack_tiles(pk, plans)
    assert np.array_equal(wh, oh.masked_weight(bits_of(w.w_bf16), m))


def test_boundary_search_tiles_single_tile_is_the_search():
    w = synth.draw("bt1", 64, 256, 64, 0.7, None, 1, 74, n_outliers=12, importance="sq")
    v1, tr1 = oh.boundary_search(w.importance.numpy(), w.perm.numpy(), 64, 256, 64, 0.7)
    vt, trt = oh.boundary_search_tiles(w.importance.numpy(), w.perm.numpy(), 64, 256, 64, 0.7)
    assert vt == [v1] and trt == [tr1]


def test_boundary_search_tiles_stop_rule_brute_force():
    """Each tile's v_s obeys the stop rule on its own retained importance, recomputed here by brute force
    (every kept element summed one by one)."""
    w = synth.draw("bt2", 96, 64, 32, 0.6, None, 1, 75, n_outliers=4, importance="sq")
    d, perm = w.importance.numpy(), w.perm.numpy()
    vs, traces = oh.boundary_search_tiles(d, perm, 96, 64, 32, 0.6)

    def r_tile(t, v):
        pl = oh.plan(32, 64, 32, 0.6, v)
        _, inter = oh.pack(bits_of(w.w_bf16)[32 * t:32 * t + 32], d[32 * t:32 * t + 32], perm[t:t + 1], pl,
                           with_intermediates=True)
        m = inter["mask"]
        sub = d[32 * t:32 * t + 32].astype(np.float64)
        scores = sub.sum(axis=0)
        dense = inter["regions"][0] == oh.DENSE
        return math.fsum(scores[dense]) + math.fsum(sub[m & ~dense[None, :]].tolist())

    for t in range(3):
        tr = traces[t]
        for v, r in tr:
            assert abs(r - r_tile(t, v)) <= 1e-9 * abs(r)
        # the trace ends at the first strict decrease (or at the end of the grid); the rule returns the
        # point before that decrease
        stopped = len(tr) > 1 and tr[-1][1] < tr[-2][1]
        assert all(tr[k][1] >= tr[k - 1][1] for k in range(1, len(tr) - (1 if stopped else 0)))
        vb = tr[-2][0] if stopped else tr[-1][0]
        assert vs[t] == oh.plan(32, 64, 32, 0.6, vb).n_pruned / 64


# ---------------------------------------------------------------------------
# In-tile input-channel gyro permutation (oracle/gyro.py)
# ---------------------------------------------------------------------------
import itertools

import oracle.gyro as og


def test_hungarian_brute_force_and_library():
    rng = np.random.default_rng(70)
    for n in range(1, 7):
        for _ in range(5):
            c = rng.random((n, n))
            col = og.hungarian(c)
            assert sorted(col.tolist()) == list(range(n))
            best = min(sum(c[i, pi[i]] for i in range(n)) for pi in itertools.permutations(range(n)))
            assert abs(sum(c[i, col[i]] for i in range(n)) - best) <= 1e-12
    from scipy.optimize import linear_sum_assignment
    for n in (17, 40):
        c = rng.random((n, n))
        r, k = linear_sum_assignment(c)
        col = og.hungarian(c)
        assert abs(c[np.arange(n), col].sum() - c[r, k].sum()) <= 1e-9


def test_hungarian_ties_lowest_column():
    # all costs equal: every assignment is optimal; the rule gives row i -> column i
    assert og.hungarian(np.ones((4, 4))).tolist() == [0, 1, 2, 3]


def test_balanced_kmeans_recovers_blobs():
    rng = np.random.default_rng(71)
    n, size, dim = 5, 6, 8
    centers = rng.normal(0, 100, (n, dim))
    pts = np.concatenate([centers[k] + rng.normal(0, 0.1, (size, dim)) for k in range(n)])
    perm = rng.permutation(n * size)
    pts = pts[perm]
    truth = (perm // size)
    init = np.array([np.nonzero(truth == k)[0][0] for k in range(n)])
    caps = og.capacities(n * size, n)
    label = og.balanced_kmeans(pts, init, 4, caps)
    assert np.bincount(label, minlength=n).tolist() == caps.tolist()
    assert np.array_equal(label, truth)


def test_balanced_kmeans_capacities_hold():
    rng = np.random.default_rng(72)
    for g, s in ((10, 3), (23, 4), (7, 7), (9, 1)):
        pts = rng.random((g, 5))
        n = og.n_clusters(g, s)
        caps = og.capacities(g, n)
        assert caps.sum() == g and caps.max() - caps.min() <= 1
        label = og.balanced_kmeans(pts, rng.choice(g, n, replace=False), 3, caps)
        assert np.bincount(label, minlength=n).tolist() == caps.tolist()


def test_pair_cost_is_what_the_24_selection_drops():
    """The group cost equals the importance the pack's own 2:4 selection leaves out (select24 is an
    argsort-based path, not pair_cost)."""
    rng = np.random.default_rng(73)
    p = oh.plan(64, 96, 32, 0.75, 0.5)
    d = rng.random((64, 96)).astype(np.float32)
    perm = np.stack([rng.permutation(96) for _ in range(2)])
    reg = oh.regions(oh.vector_scores(d, p), p)
    _, idx_s = oh.index_lists(reg, perm, p)
    sel = oh.select24(d, idx_s, p)
    for t in range(2):
        rows = slice(32 * t, 32 * t + 32)
        cols = idx_s[t, :p.n_24].reshape(p.groups, 4)
        a = d[rows][:, cols.reshape(-1)].reshape(32, p.groups, 4).astype(np.float64)
        kept = np.take_along_axis(a, sel[rows], axis=-1).sum(axis=-1)
        dropped = (a.sum(axis=-1) - kept).sum(axis=0)
        assert np.allclose(og.group_costs(d[rows], cols), dropped, rtol=1e-12, atol=1e-12)


def _gyro_case(seed, cout=128, cin=96, R=32, t=0.75, v=0.5, rounds=3, s=3, iters=2):
    rng = np.random.default_rng(seed)
    d = (rng.random((cout, cin)) ** 3).astype(np.float32)
    p = oh.plan(cout, cin, R, t, v)
    perm = np.stack([rng.permutation(cin) for _ in range(p.n_tiles)])
    n = og.n_clusters(p.groups, s)
    sample, init = synth.gyro_draws(seed, rounds, p.n_tiles, p.groups, n)
    new, trace = og.gyro_permutation(d, perm, p, rounds, s, iters, sample, init)
    return d, p, perm, new, trace


def test_gyro_rounds_never_raise_the_cost_and_keep_the_regions():
    for seed in range(4):
        d, p, perm, new, trace = _gyro_case(80 + seed)
        assert np.all(np.diff(trace, axis=0) <= 0)
        assert np.any(trace[-1] < trace[0])
        reg = oh.regions(oh.vector_scores(d, p), p)
        for t in range(p.n_tiles):
            assert sorted(new[t].tolist()) == list(range(p.cin))
            fixed = reg[t][perm[t]] != oh.TWO_FOUR
            assert np.array_equal(new[t][fixed], perm[t][fixed])           # dense and pruned stay put
            assert sorted(new[t][~fixed].tolist()) == sorted(perm[t][~fixed].tolist())


def test_gyro_trace_is_the_retained_importance_gain():
    """R_24 after minus R_24 before equals the pruning cost removed (retained_importance is the boundary
    search's objective, computed through the pack's select24)."""
    d, p, perm, new, trace = _gyro_case(85)
    gain = oh.retained_importance(d, new, p) - oh.retained_importance(d, perm, p)
    assert gain >= 0
    assert abs(gain - (trace[0].sum() - trace[-1].sum())) <= 1e-9 * max(1.0, trace[0].sum())


def test_gyro_one_cluster_round_is_the_brute_force_optimum():
    """One cluster holding every group: the round's cost is the least over all ways of putting the drawn
    columns back (brute force over G! assignments)."""
    rng = np.random.default_rng(86)
    d_tile = (rng.random((16, 20)) ** 2).astype(np.float32)
    cols = rng.permutation(20)[:16].reshape(4, 4)
    sample = rng.integers(0, 4, 4)
    new = og.gyro_round(d_tile, cols, sample, np.array([0]), cluster_size=8, iters=2)
    drawn = cols[np.arange(4), sample]
    best = np.inf
    for pi in itertools.permutations(range(4)):
        c = cols.copy()
        for j in range(4):
            c[j, sample[j]] = drawn[pi[j]]
        best = min(best, og.total_cost(og.group_costs(d_tile, c)))
    assert abs(og.total_cost(og.group_costs(d_tile, new)) - best) <= 1e-12


def test_gyro_no_24_region_is_a_no_op():
    rng = np.random.default_rng(87)
    d = rng.random((64, 64)).astype(np.float32)
    p = oh.plan(64, 64, 32, 0.75, 0.75)
    perm = np.stack([rng.permutation(64) for _ in range(2)])
    new, trace = og.gyro_permutation(d, perm, p, 2, 4, 2, np.zeros((2, 2, 0), np.uint8), np.zeros((2, 2, 0), np.int32))
    assert np.array_equal(new, perm) and not trace.any()


def test_mutation_gyro_largest_two_is_caught(monkeypatch):
    """A cost that drops the two largest instead of the two smallest fails the select24 pin."""
    def wrong(vals):
        s = np.sort(np.asarray(vals, dtype=np.float32), axis=-1)
        per_row = s[..., 2].astype(np.float64) + s[..., 3].astype(np.float64)
        acc = np.zeros(per_row.shape[:-1])
        for r in range(per_row.shape[-1]):
            acc = acc + per_row[..., r]
        return acc
    monkeypatch.setattr(og, "pair_cost", wrong)
    with pytest.raises(AssertionError):
        test_pair_cost_is_what_the_24_selection_drops()


def test_mutation_gyro_maximising_assignment_is_caught(monkeypatch):
    orig = og.hungarian
    monkeypatch.setattr(og, "hungarian", lambda c: orig(-np.asarray(c)))
    with pytest.raises(AssertionError):
        test_gyro_one_cluster_round_is_the_brute_force_optimum()


def _kmeans_cases():
    with open(os.path.join(GOLDEN, "gyro_kmeans_handworked.json")) as f:
        return json.load(f)["cases"]


def test_balanced_kmeans_handworked():
    """Hand-worked cases (tests/golden/gyro_kmeans_handworked.json): the centroid update changes the
    second assignment step, squared euclidean and L1 distances pick different clusters, and equal
    distances go to the lower cluster and the lower point first."""
    for c in _kmeans_cases():
        label = og.balanced_kmeans(np.array(c["points"], dtype=np.float64), np.array(c["init"]), c["iters"],
                                   np.array(c["caps"], dtype=np.int64))
        assert label.tolist() == c["labels"], c["name"]


def test_mutation_kmeans_without_update_is_caught(monkeypatch):
    def frozen(points, init, iters, caps):
        cents = points[np.asarray(init, dtype=np.int64)].copy()
        label = None
        for _ in range(iters):
            label = og.balanced_assign(og.sq_dist(points, cents), caps)
        return label
    monkeypatch.setattr(og, "balanced_kmeans", frozen)
    with pytest.raises(AssertionError):
        test_balanced_kmeans_handworked()


def test_mutation_kmeans_l1_distance_is_caught(monkeypatch):
    monkeypatch.setattr(og, "sq_dist", lambda p, c: np.abs(p[:, None, :] - c[None, :, :]).sum(axis=-1))
    with pytest.raises(AssertionError):
        test_balanced_kmeans_handworked()


@pytest.mark.parametrize("reverse", ["cluster", "point"])
def test_mutation_kmeans_reversed_tie_order_is_caught(monkeypatch, reverse):
    def assign(dist, caps):
        g, n = dist.shape
        qs, ks = np.repeat(np.arange(g), n), np.tile(np.arange(n), g)
        keys = (-ks, qs, dist.reshape(-1)) if reverse == "cluster" else (ks, -qs, dist.reshape(-1))
        label, room = np.full(g, -1, dtype=np.int64), caps.copy()
        for e in np.lexsort(keys):
            if label[qs[e]] < 0 and room[ks[e]] > 0:
                label[qs[e]] = ks[e]
                room[ks[e]] -= 1
        return label
    monkeypatch.setattr(og, "balanced_assign", assign)
    with pytest.raises(AssertionError):
        test_balanced_kmeans_handworked()
