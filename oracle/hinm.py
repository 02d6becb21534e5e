"""Step-by-step CPU oracle of the HiNM (hierarchical N:M) pack and product.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py (cpu_baseline, cpu_baseline_boundary), never by the
product path.

Sources (cited by page title and section; the pages are the FlexHiNM-GP paper
notes, an article on N:M block sparsity, an article on 2:4 structured
sparsity, the PermLLM summary and a course page on structured pruning):

* FlexHiNM-GP notes, one-line summary and "整体框架" (framework): every
  output-channel tile of W is split into a dense (4:4) region, a 2:4 region
  and a fully pruned (0:4) region of whole column vectors.
* FlexHiNM-GP notes, key design 1 (boundary search): the closed form
  t_s = v_s + (1 - v_s) * p_s * 0.5, hence p_s = 2 (t_s - v_s) / (1 - v_s),
  and a 1-D search on v_s that maximises the retained importance
  R_total = R_dense + R_24, starting at v_s = t_s and stopping at the first
  decrease.
* FlexHiNM-GP notes, "亮点与洞察" (highlights): high-importance vectors stay
  dense, medium ones go 2:4, low ones are pruned whole.
* FlexHiNM-GP notes, key designs 2 and 4: permutation reorders channels
  without changing the result; the kernel gathers input rows through
  precomputed N:M indices, with the permutation folded into the index.
* N:M block-sparsity article, section 2 (definition): keep N of every M
  consecutive weights along the input dimension, chosen by magnitude.
* 2:4 structured-sparsity article, section 3: exactly 2 kept per group of 4,
  groups independent, 2 bits of position per kept element (6 legal
  patterns); section 5: the forward uses W (.) M.
* PermLLM summary, problem definition (W in R^{Cout x Cin}, W_hat = W P) and
  the mask rule on permuted importance (top-N per group of M).

Readings where the pages are silent or ambiguous (each one is listed in the
design notes of the repository):

* a "vector" is the column segment W[tR:tR+R, c] of one tile;
* the region counts are the same in every tile and rounded half-up:
  Z = floor(t_s*Cin + 1/2), g = floor((t_s - v_s)*Cin/2 + 1/2) clamped to
  [0, floor(min(Z, Cin - Z)/2)], n_24 = 4g, n_pruned = Z - 2g,
  n_dense = Cin - Z - 2g;
* a vector's score is the float64 sum of its importance over the tile's rows,
  accumulated in ascending row order from +0.0; columns rank by
  (-score, column); dense = first n_dense, 2:4 = next n_24, rest pruned;
* perm[t][j] is the original column placed at position j of tile t; the
  index lists keep perm order; 2:4 groups are 4 consecutive entries of the
  2:4 list;
* in a group, the two kept entries are the first two by (-importance,
  position); metadata nibble = i0 | i1 << 2 with i0 < i1;
* the boundary search steps v_s by 0.01 (the page's adaptive step terms are
  taken as zero) and snaps the result to n_pruned / Cin.

Packed layout (this library's own format; padding to whole K-blocks):

* val_dense  uint16 (bf16 bits) [T][n_dense_pad/32][R][32]
* idx_dense  int32              [T][n_dense_pad]          (pad = -1)
* val_24     uint16 (bf16 bits) [T][n_24_pad/64][R][32]   (2 per group, i0 then i1)
* meta_24    uint64             [T][n_24_pad/64][R]       (nibble q at bits 4q)
* idx_24     int32              [T][n_24_pad]             (pad = -1)

Pad values are +0 (0x0000), pad nibbles 0x4, pad indices -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

DENSE, TWO_FOUR, PRUNED = 2, 1, 0
KB_DENSE = 32          # dense-region K-block: 32 columns
KB_24 = 64             # 2:4-region K-block: 64 positions = 16 groups
PAD_NIBBLE = 0x4       # i0 = 0, i1 = 1
# The six ways to keep 2 of 4 (2:4 article, section 3): i0 | i1 << 2, i0 < i1.
LEGAL_NIBBLES = (0x4, 0x8, 0xC, 0x9, 0xD, 0xE)


class OracleError(ValueError):
    """An argument the method does not define (bad shape, range or permutation)."""


@dataclasses.dataclass(frozen=True)
class Plan:
    cout: int
    cin: int
    tile_rows: int
    n_tiles: int
    t_s: float
    v_s: float
    p_s: float
    z: int            # zeros per row
    groups: int       # 2:4 groups per tile row
    n_dense: int
    n_24: int
    n_pruned: int
    n_dense_pad: int
    n_24_pad: int


def plan(cout: int, cin: int, tile_rows: int, t_s: float, v_s: float) -> Plan:
    """Region counts of one weight (FlexHiNM-GP notes, key design 1, closed form)."""
    if cout <= 0 or cin <= 0 or tile_rows <= 0:
        raise OracleError("sizes must be positive")
    if tile_rows % 16 or cout % tile_rows:
        raise OracleError("tile_rows must be a multiple of 16 dividing cout")
    if cin % 4:
        raise OracleError("cin must be a multiple of 4 (groups of 4 along the input dim)")
    if not (math.isfinite(t_s) and math.isfinite(v_s)):
        raise OracleError("t_s, v_s must be finite")
    if not (0.0 <= t_s < 1.0):
        raise OracleError("t_s must lie in [0, 1)")
    if not (max(0.0, 2.0 * t_s - 1.0) <= v_s <= t_s):
        raise OracleError("v_s must lie in [max(0, 2 t_s - 1), t_s] so that p_s is in [0, 1]")
    z = math.floor(t_s * cin + 0.5)
    g = math.floor((t_s - v_s) * cin / 2.0 + 0.5)
    g = max(0, min(g, min(z, cin - z) // 2))
    n_24 = 4 * g
    n_pruned = z - 2 * g
    n_dense = cin - z - 2 * g
    p_s = 2.0 * (t_s - v_s) / (1.0 - v_s)
    return Plan(cout, cin, tile_rows, cout // tile_rows, t_s, v_s, p_s, z, g, n_dense, n_24,
                n_pruned, -(-n_dense // KB_DENSE) * KB_DENSE, -(-n_24 // KB_24) * KB_24)


def _check_perm(perm: np.ndarray, p: Plan) -> None:
    if perm.shape != (p.n_tiles, p.cin):
        raise OracleError(f"perm must have shape {(p.n_tiles, p.cin)}")
    want = np.arange(p.cin)
    for t in range(p.n_tiles):
        if not np.array_equal(np.sort(perm[t]), want):
            raise OracleError(f"perm[{t}] is not a permutation of 0..cin-1")


def _check_importance(d: np.ndarray, p: Plan) -> None:
    if d.shape != (p.cout, p.cin):
        raise OracleError("importance must have shape (cout, cin)")
    if not np.all(np.isfinite(d)) or np.any(d < 0):
        raise OracleError("importance must be finite and >= 0")


def vector_scores(d: np.ndarray, p: Plan) -> np.ndarray:
    """Score of every column vector of every tile: s[t][c] = sum_r D[tR+r][c].

    Accumulated in float64, rows in ascending order, starting from +0.0
    (FlexHiNM-GP notes, key design 2: the objective is the retained importance
    ||M (.) D||; a vector's share of it is the sum over its rows).
    """
    d3 = np.asarray(d, dtype=np.float32).reshape(p.n_tiles, p.tile_rows, p.cin)
    s = np.zeros((p.n_tiles, p.cin), dtype=np.float64)
    for r in range(p.tile_rows):
        s = s + d3[:, r, :].astype(np.float64)
    return s


def regions(s: np.ndarray, p: Plan) -> np.ndarray:
    """Region of every column in every tile (FlexHiNM-GP notes, highlights).

    Rank by (-score, column): first n_dense dense, next n_24 2:4, rest pruned.
    """
    reg = np.full((p.n_tiles, p.cin), PRUNED, dtype=np.uint8)
    for t in range(p.n_tiles):
        order = np.argsort(-s[t], kind="stable")
        reg[t, order[:p.n_dense]] = DENSE
        reg[t, order[p.n_dense:p.n_dense + p.n_24]] = TWO_FOUR
    return reg


def index_lists(reg: np.ndarray, perm: np.ndarray, p: Plan) -> Tuple[np.ndarray, np.ndarray]:
    """Kept-vector index lists in permuted order, padded with -1.

    idx_x[t] = [perm[t][j] for ascending j if region of perm[t][j] is x]
    (FlexHiNM-GP notes, key design 2 and 4: the input permutation is folded
    into the index the kernel gathers through; PermLLM summary: W_hat = W P).
    """
    idx_d = np.full((p.n_tiles, p.n_dense_pad), -1, dtype=np.int32)
    idx_s = np.full((p.n_tiles, p.n_24_pad), -1, dtype=np.int32)
    for t in range(p.n_tiles):
        r = reg[t][perm[t]]
        dl = perm[t][r == DENSE]
        sl = perm[t][r == TWO_FOUR]
        assert dl.size == p.n_dense and sl.size == p.n_24
        idx_d[t, :p.n_dense] = dl
        idx_s[t, :p.n_24] = sl
    return idx_d, idx_s


def select24(d: np.ndarray, idx_s: np.ndarray, p: Plan) -> np.ndarray:
    """Kept positions (i0 < i1) of every 2:4 group of every row: [cout][groups][2].

    Group q of tile t covers columns idx_s[t][4q..4q+3].  In each row the two
    entries with the largest importance are kept, ties to the lower position
    (2:4 article, section 3; N:M article, section 2; PermLLM summary, mask on
    permuted importance).
    """
    sel = np.zeros((p.cout, p.groups, 2), dtype=np.int64)
    if p.groups == 0:
        return sel
    for t in range(p.n_tiles):
        rows = slice(t * p.tile_rows, (t + 1) * p.tile_rows)
        cols = idx_s[t, :p.n_24]
        a = np.asarray(d, dtype=np.float32)[rows][:, cols].reshape(p.tile_rows, p.groups, 4)
        order = np.argsort(-a, axis=-1, kind="stable")[..., :2]
        sel[rows] = np.sort(order, axis=-1)
    return sel


def mask_from(idx_d: np.ndarray, idx_s: np.ndarray, sel: np.ndarray, p: Plan) -> np.ndarray:
    """Boolean mask M [cout][cin]: dense columns of the tile plus the chosen 2:4 entries."""
    m = np.zeros((p.cout, p.cin), dtype=bool)
    for t in range(p.n_tiles):
        rows = np.arange(t * p.tile_rows, (t + 1) * p.tile_rows)
        m[np.ix_(rows, idx_d[t, :p.n_dense])] = True
        if p.groups:
            grp = idx_s[t, :p.n_24].reshape(p.groups, 4)
            for e in range(2):
                cols = grp[np.arange(p.groups)[None, :], sel[rows, :, e]]
                m[rows[:, None], cols] = True
    return m


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the upper half of an fp32 word)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def serialize(w_bits: np.ndarray, idx_d: np.ndarray, idx_s: np.ndarray, sel: np.ndarray,
              p: Plan) -> Dict[str, np.ndarray]:
    """Write the packed buffers in this library's layout (see the module docstring)."""
    R, T = p.tile_rows, p.n_tiles
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    val_d = np.zeros((T, p.n_dense_pad // KB_DENSE, R, KB_DENSE), dtype=np.uint16)
    val_s = np.zeros((T, p.n_24_pad // KB_24, R, 32), dtype=np.uint16)
    meta = np.zeros((T, p.n_24_pad // KB_24, R), dtype=np.uint64)
    for t in range(T):
        base = t * R
        for j in range(p.n_dense):
            kb, k = divmod(j, KB_DENSE)
            val_d[t, kb, :, k] = w_bits[base:base + R, idx_d[t, j]]
        for q in range(p.n_24_pad // 4):
            kb, ql = divmod(q, KB_24 // 4)
            if q < p.groups:
                i0 = sel[base:base + R, q, 0]
                i1 = sel[base:base + R, q, 1]
                c0 = idx_s[t, 4 * q + i0]
                c1 = idx_s[t, 4 * q + i1]
                rows = np.arange(base, base + R)
                val_s[t, kb, :, 2 * ql] = w_bits[rows, c0]
                val_s[t, kb, :, 2 * ql + 1] = w_bits[rows, c1]
                nib = (i0 | (i1 << 2)).astype(np.uint64)
            else:
                nib = np.full(R, PAD_NIBBLE, dtype=np.uint64)
            meta[t, kb, :] |= nib << np.uint64(4 * ql)
    return {"val_dense": val_d, "idx_dense": idx_d.copy(), "val_24": val_s, "meta_24": meta,
            "idx_24": idx_s.copy()}


def pack(w_bits: np.ndarray, importance: np.ndarray, perm: Optional[np.ndarray], p: Plan,
         with_intermediates: bool = False):
    """The whole pack: scores, regions, index lists, 2:4 selection, serialisation.

    ``w_bits`` are the bf16 bit patterns of W [cout][cin]; ``importance`` is
    fp32 [cout][cin]; ``perm`` int [n_tiles][cin] or None for the identity.
    """
    d = np.asarray(importance, dtype=np.float32)
    _check_importance(d, p)
    if perm is None:
        perm = np.tile(np.arange(p.cin, dtype=np.int64), (p.n_tiles, 1))
    perm = np.asarray(perm, dtype=np.int64)
    _check_perm(perm, p)
    s = vector_scores(d, p)
    reg = regions(s, p)
    idx_d, idx_s = index_lists(reg, perm, p)
    sel = select24(d, idx_s, p)
    packed = serialize(w_bits, idx_d, idx_s, sel, p)
    if with_intermediates:
        return packed, {"scores": s, "regions": reg, "sel": sel,
                        "mask": mask_from(idx_d, idx_s, sel, p)}
    return packed


def masked_weight(w_bits: np.ndarray, m: np.ndarray) -> np.ndarray:
    """W (.) M in float64 (2:4 article, section 5)."""
    return np.where(m, bf16_bits_to_f64(w_bits), 0.0)


def unpack(packed: Dict[str, np.ndarray], p: Plan) -> np.ndarray:
    """Rebuild the dense masked weight [cout][cin] (float64) from the packed buffers."""
    R = p.tile_rows
    w = np.zeros((p.cout, p.cin), dtype=np.float64)
    vd = bf16_bits_to_f64(packed["val_dense"])
    vs = bf16_bits_to_f64(packed["val_24"])
    for t in range(p.n_tiles):
        rows = np.arange(t * R, (t + 1) * R)
        for j in range(p.n_dense_pad):
            c = packed["idx_dense"][t, j]
            if c >= 0:
                w[rows, c] += vd[t, j // KB_DENSE, :, j % KB_DENSE]
        for q in range(p.n_24_pad // 4):
            kb, ql = divmod(q, KB_24 // 4)
            nib = (packed["meta_24"][t, kb, :] >> np.uint64(4 * ql)) & np.uint64(0xF)
            i0 = (nib & np.uint64(3)).astype(np.int64)
            i1 = (nib >> np.uint64(2)).astype(np.int64)
            c0 = packed["idx_24"][t, 4 * q + i0]
            c1 = packed["idx_24"][t, 4 * q + i1]
            ok0, ok1 = c0 >= 0, c1 >= 0
            w[rows[ok0], c0[ok0]] += vs[t, kb, ok0, 2 * ql]
            w[rows[ok1], c1[ok1]] += vs[t, kb, ok1, 2 * ql + 1]
    return w


def spmm(w_hat: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Y = W_hat . X as a dense float64 product (the method computes exactly this)."""
    return np.asarray(w_hat, dtype=np.float64) @ np.asarray(x, dtype=np.float64)


def plan_tiles(cout: int, cin: int, tile_rows: int, t_s: float, v_s_tiles) -> List[Plan]:
    """Per-tile region counts: the closed form of key design 1 at each tile's own v_s.

    FlexHiNM-GP notes, "整体框架": the ratio of the three regions is decided
    inside each output-channel tile.  t_s is shared, so every row of every
    tile keeps cin - z entries; only the dense / 2:4 split moves.  Each
    returned plan describes one tile (cout = tile_rows).
    """
    if tile_rows <= 0 or cout % tile_rows:
        raise OracleError("tile_rows must divide cout")
    v = [float(x) for x in v_s_tiles]
    if len(v) != cout // tile_rows:
        raise OracleError("one v_s per tile is needed")
    return [plan(tile_rows, cin, tile_rows, t_s, vt) for vt in v]


def pack_tiles(w_bits: np.ndarray, importance: np.ndarray, perm: Optional[np.ndarray], plans: List[Plan],
               with_intermediates: bool = False):
    """Pack with per-tile counts.  Tiles are independent (scores, regions,
    index lists and 2:4 groups never cross a tile), so tile t is packed on its
    own and the buffers of the tiles are laid end to end: the K-blocks of
    tile t follow those of tile t-1.  ``tiles`` [T][4] holds, per tile, the
    first dense block, n_dense, the first 2:4 block and n_24.
    """
    R = plans[0].tile_rows
    T = len(plans)
    cin = plans[0].cin
    w_bits = np.asarray(w_bits)
    d = np.asarray(importance, dtype=np.float32)
    if perm is None:
        perm = np.tile(np.arange(cin, dtype=np.int64), (T, 1))
    perm = np.asarray(perm, dtype=np.int64)
    parts, masks = [], []
    tiles = np.zeros((T, 4), dtype=np.int64)
    kd = ks = 0
    for t, pt in enumerate(plans):
        rows = slice(t * R, (t + 1) * R)
        pk, inter = pack(w_bits[rows], d[rows], perm[t:t + 1], pt, with_intermediates=True)
        parts.append(pk)
        masks.append(inter["mask"])
        tiles[t] = (kd, pt.n_dense, ks, pt.n_24)
        kd += pt.n_dense_pad // KB_DENSE
        ks += pt.n_24_pad // KB_24
    packed = {
        "val_dense": np.concatenate([q["val_dense"][0] for q in parts], axis=0),
        "idx_dense": np.concatenate([q["idx_dense"][0] for q in parts], axis=0),
        "val_24": np.concatenate([q["val_24"][0] for q in parts], axis=0),
        "meta_24": np.concatenate([q["meta_24"][0] for q in parts], axis=0),
        "idx_24": np.concatenate([q["idx_24"][0] for q in parts], axis=0),
        "tiles": tiles,
    }
    if with_intermediates:
        return packed, {"mask": np.concatenate(masks, axis=0)}
    return packed


def unpack_tiles(packed: Dict[str, np.ndarray], plans: List[Plan]) -> np.ndarray:
    """Dense masked weight [cout][cin] (float64) from per-tile packed buffers."""
    R, cin = plans[0].tile_rows, plans[0].cin
    w = np.zeros((R * len(plans), cin), dtype=np.float64)
    for t, pt in enumerate(plans):
        kd, _, ks, _ = (int(v) for v in packed["tiles"][t])
        nkd, nks = pt.n_dense_pad // KB_DENSE, pt.n_24_pad // KB_24
        one = {"val_dense": packed["val_dense"][None, kd:kd + nkd],
               "idx_dense": packed["idx_dense"][None, KB_DENSE * kd:KB_DENSE * (kd + nkd)],
               "val_24": packed["val_24"][None, ks:ks + nks],
               "meta_24": packed["meta_24"][None, ks:ks + nks],
               "idx_24": packed["idx_24"][None, KB_24 * ks:KB_24 * (ks + nks)]}
        w[t * R:(t + 1) * R] = unpack(one, pt)
    return w


def boundary_search_tiles(d: np.ndarray, perm: np.ndarray, cout: int, cin: int, tile_rows: int, t_s: float,
                          step: float = 0.01) -> Tuple[List[float], List[List[Tuple[float, float]]]]:
    """Key design 1's search run inside each tile on its own: tile t's retained
    importance R_t(v) decides tile t's v_s (same grid and stop rule as
    boundary_search, which is this search with one tile)."""
    d = np.asarray(d, dtype=np.float32)
    perm = np.asarray(perm)
    vs, traces = [], []
    for t in range(cout // tile_rows):
        rows = slice(t * tile_rows, (t + 1) * tile_rows)
        v, tr = boundary_search(d[rows], perm[t:t + 1], tile_rows, cin, tile_rows, t_s, step)
        vs.append(v)
        traces.append(tr)
    return vs, traces


def scatter_rows(y: np.ndarray, out_rows: np.ndarray) -> np.ndarray:
    """Output-channel permutation undone at write-out: result[out_rows[r]] = y[r].

    FlexHiNM-GP notes, key design 2: output channels are permuted before
    pruning, and the permutation costs nothing at run time because it is
    applied where the data moves anyway (highlights).  ``out_rows`` must be a
    permutation of 0..cout-1.
    """
    y = np.asarray(y)
    out_rows = np.asarray(out_rows, dtype=np.int64)
    if out_rows.shape != (y.shape[0],) or not np.array_equal(np.sort(out_rows), np.arange(y.shape[0])):
        raise ValueError("out_rows must be a permutation of 0..cout-1")
    res = np.empty_like(y)
    res[out_rows] = y
    return res


def translate_indices(idx: np.ndarray, mapping: np.ndarray) -> np.ndarray:
    """Cross-layer index translation: every index i >= 0 becomes mapping[i]; pads (-1) stay.

    FlexHiNM-GP notes, key design 2: the translation between one layer's
    output order and the next layer's input order is folded into the HiNM
    indices; key design 4: the kernel gathers X rows through those indices.
    With mapping[c] = the row at which channel c is stored, gathering through
    the translated indices reads the same values as gathering channel rows
    through the original ones.
    """
    idx = np.asarray(idx)
    mapping = np.asarray(mapping, dtype=np.int64)
    n = mapping.shape[0]
    if not np.array_equal(np.sort(mapping), np.arange(n)):
        raise ValueError("mapping must be a permutation")
    out = idx.copy()
    keep = idx >= 0
    out[keep] = mapping[idx[keep]]
    return out


def retained_importance(d: np.ndarray, perm: np.ndarray, p: Plan,
                        s: Optional[np.ndarray] = None) -> float:
    """R_total = R_dense + R_24 for the allocation that ``p`` defines.

    R_dense sums the scores of the dense vectors; R_24 sums, over every row
    and 2:4 group, the importance of the two kept entries (FlexHiNM-GP notes,
    key design 1).  Pruned vectors retain nothing.
    """
    d = np.asarray(d, dtype=np.float32)
    if s is None:
        s = vector_scores(d, p)
    reg = regions(s, p)
    idx_d, idx_s = index_lists(reg, np.asarray(perm, dtype=np.int64), p)
    total = 0.0
    for t in range(p.n_tiles):
        total += float(np.sum(s[t, idx_d[t, :p.n_dense]]))
    if p.groups:
        sel = select24(d, idx_s, p)
        for t in range(p.n_tiles):
            rows = slice(t * p.tile_rows, (t + 1) * p.tile_rows)
            a = d[rows][:, idx_s[t, :p.n_24]].reshape(p.tile_rows, p.groups, 4).astype(np.float64)
            kept = np.take_along_axis(a, sel[rows], axis=-1)
            total += float(np.sum(kept))
    return total


def _v_grid(t_s: float, step: float) -> List[float]:
    lo = max(0.0, 2.0 * t_s - 1.0)
    out, k = [], 0
    while True:
        v = t_s - step * k
        if v < lo - 1e-12:
            break
        out.append(max(v, lo))
        k += 1
    return out


def boundary_search(d: np.ndarray, perm: np.ndarray, cout: int, cin: int, tile_rows: int,
                    t_s: float, step: float = 0.01) -> Tuple[float, List[Tuple[float, float]]]:
    """1-D search on v_s (FlexHiNM-GP notes, key design 1).

    Starts at v_s = t_s and lowers v_s by ``step`` while the retained
    importance does not decrease; at the first strict decrease it returns the
    previous v_s, snapped to n_pruned / cin of its plan.  Returns (v_s, trace).
    """
    p0 = plan(cout, cin, tile_rows, t_s, t_s)
    s = vector_scores(np.asarray(d, dtype=np.float32), p0)
    trace: List[Tuple[float, float]] = []
    best_v, best_r = None, None
    for v in _v_grid(t_s, step):
        r = retained_importance(d, perm, plan(cout, cin, tile_rows, t_s, v), s)
        trace.append((v, r))
        if best_r is not None and r < best_r:
            break
        best_v, best_r = v, r
    pb = plan(cout, cin, tile_rows, t_s, best_v)
    return pb.n_pruned / cin, trace


def boundary_grid(d: np.ndarray, perm: np.ndarray, cout: int, cin: int, tile_rows: int,
                  t_s: float, step: float = 0.01) -> List[Tuple[float, float]]:
    """Retained importance at every grid point (the full scan the early stop relies on)."""
    p0 = plan(cout, cin, tile_rows, t_s, t_s)
    s = vector_scores(np.asarray(d, dtype=np.float32), p0)
    return [(v, retained_importance(d, perm, plan(cout, cin, tile_rows, t_s, v), s))
            for v in _v_grid(t_s, step)]
