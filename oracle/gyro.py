"""CPU oracle of the in-tile input-channel gyro permutation.

TEST INFRASTRUCTURE ONLY: imported by tests/ and the CPU-baseline leg of
bench.py (cpu_baseline_gyro), never by the product path.

Source: FlexHiNM-GP paper notes, key design 2 (陀螺置换, gyro permutation).
The notes state the objective, argmax over the output and input channel
orders of ||M (.) D||, the split into output-channel permutation, vector
pruning and in-tile input-channel permutation, and one round of the latter as
three steps: draw vectors from each tile, cluster them with a balanced
K-means, assign them with the Hungarian algorithm on a pruning-cost matrix
(lower cost is better), repeated over rounds.  The notes give no further
detail; the plain reading implemented here (each choice is listed among the
readings of the pages in the design notes):

* Only the 2:4 region is affected: the dense and pruned sets depend on the
  vector scores alone, while the input order decides which four columns form
  a 2:4 group (group q of a tile = entries 4q..4q+3 of its 2:4 list, the list
  in permuted order).
* Pruning cost of a group = the importance the 2:4 selection drops: per row
  the sum of the two smallest of its four importances, summed over the tile's
  rows.  Per row the two values are added in float64 and the rows in
  ascending order from +0.0.
* One round, per tile:
  1. sampling - from every group q one position sample[q] in 0..3 (drawn by
     the caller); its column is taken out, leaving a hole in group q;
  2. balanced K-means - the drawn columns' importance vectors (float64 over
     the tile's rows) are split into N = ceil(G / S) clusters of sizes
     floor(G / N) or one more (the first G mod N clusters take the extra
     point).  Centroids start at the drawn vectors init[0..N-1] (drawn by the
     caller).  An assignment step gives every point the cluster of its
     nearest centroid under the capacities: all (squared distance, point,
     cluster) triples in increasing order, each point taking the first
     cluster in that order that still has room.  An update step sets every
     centroid to the mean of its members (summed in increasing point order).
     `iters` assignment steps with an update between consecutive ones;
  3. Hungarian - inside every cluster, the drawn columns of its members are
     assigned to the holes of its members so that the summed pruning cost of
     the refilled groups is least.  cost[i][j] = pruning cost of group q_j
     with column a_{q_i} in its hole (members in increasing order).  The
     algorithm is the O(n^3) shortest-augmenting-path form with potentials;
     on equal reduced costs it takes the lowest column index.
  Putting every drawn column back where it came from is one of the
  assignments, so no round increases the tile's pruning cost.
* The output permutation keeps the dense and pruned columns where they were
  and writes the 2:4 columns, in their new list order, into the positions the
  2:4 columns occupied.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from . import hinm as oh


def n_clusters(groups: int, cluster_size: int) -> int:
    return -(-groups // cluster_size) if groups else 0


def capacities(groups: int, n: int) -> np.ndarray:
    base, extra = divmod(groups, n)
    return np.array([base + (1 if k < extra else 0) for k in range(n)], dtype=np.int64)


def pair_cost(vals: np.ndarray) -> np.ndarray:
    """Per-row dropped importance of groups: vals [..., R, 4] float32 ->
    [...] float64, the two smallest of each row added in float64, rows summed
    in ascending order."""
    s = np.sort(np.asarray(vals, dtype=np.float32), axis=-1)
    per_row = s[..., 0].astype(np.float64) + s[..., 1].astype(np.float64)
    acc = np.zeros(per_row.shape[:-1], dtype=np.float64)
    for r in range(per_row.shape[-1]):
        acc = acc + per_row[..., r]
    return acc


def sq_dist(points: np.ndarray, cents: np.ndarray) -> np.ndarray:
    """Squared euclidean distances [G][N], the rows' terms added in ascending order."""
    acc = np.zeros((points.shape[0], cents.shape[0]), dtype=np.float64)
    for r in range(points.shape[1]):
        diff = points[:, r][:, None] - cents[:, r][None, :]
        acc = acc + diff * diff
    return acc


def balanced_assign(dist: np.ndarray, caps: np.ndarray) -> np.ndarray:
    """Every point to the cluster of the first (distance, point, cluster)
    triple in increasing order that still has room."""
    g, n = dist.shape
    qs = np.repeat(np.arange(g), n)
    ks = np.tile(np.arange(n), g)
    order = np.lexsort((ks, qs, dist.reshape(-1)))
    label = np.full(g, -1, dtype=np.int64)
    room = caps.copy()
    for e in order:
        q, k = qs[e], ks[e]
        if label[q] < 0 and room[k] > 0:
            label[q] = k
            room[k] -= 1
    return label


def balanced_kmeans(points: np.ndarray, init: np.ndarray, iters: int, caps: np.ndarray) -> np.ndarray:
    """Cluster labels of the points (float64 [G][R]) after `iters` capacity-bound assignment steps."""
    cents = points[np.asarray(init, dtype=np.int64)].copy()
    label = None
    for it in range(iters):
        label = balanced_assign(sq_dist(points, cents), caps)
        if it + 1 < iters:
            for k in range(cents.shape[0]):
                acc = np.zeros(points.shape[1], dtype=np.float64)
                members = np.nonzero(label == k)[0]
                for q in members:
                    acc = acc + points[q]
                cents[k] = acc / float(members.size)
    return label


def hungarian(cost: np.ndarray) -> np.ndarray:
    """Minimum-cost assignment of an n x n matrix: col[i] is the column of row i.

    Shortest augmenting paths with row and column potentials, one row added
    at a time (Kuhn-Munkres in its O(n^3) form); on equal reduced costs the
    lowest column index is taken.
    """
    n = cost.shape[0]
    inf = float("inf")
    u = [0.0] * (n + 1)
    v = [0.0] * (n + 1)
    match = [0] * (n + 1)          # match[j] = row (1-based) assigned to column j, 0 = free
    way = [0] * (n + 1)
    a = [[0.0] * (n + 1)] + [[0.0] + [float(x) for x in row] for row in cost]
    for i in range(1, n + 1):
        match[0] = i
        j0 = 0
        minv = [inf] * (n + 1)
        used = [False] * (n + 1)
        while True:
            used[j0] = True
            i0 = match[j0]
            delta = inf
            j1 = 0
            for j in range(1, n + 1):
                if not used[j]:
                    cur = a[i0][j] - u[i0] - v[j]
                    if cur < minv[j]:
                        minv[j] = cur
                        way[j] = j0
                    if minv[j] < delta:
                        delta = minv[j]
                        j1 = j
            for j in range(n + 1):
                if used[j]:
                    u[match[j]] += delta
                    v[j] -= delta
                else:
                    minv[j] -= delta
            j0 = j1
            if match[j0] == 0:
                break
        while True:
            j1 = way[j0]
            match[j0] = match[j1]
            j0 = j1
            if j0 == 0:
                break
    col = np.zeros(n, dtype=np.int64)
    for j in range(1, n + 1):
        col[match[j] - 1] = j - 1
    return col


def group_costs(d_tile: np.ndarray, groups_cols: np.ndarray) -> np.ndarray:
    """Pruning cost of every group: d_tile float32 [R][cin], groups_cols [G][4] column indices."""
    vals = d_tile[:, groups_cols]                 # [R][G][4]
    return pair_cost(np.transpose(vals, (1, 0, 2)))


def total_cost(gc: np.ndarray) -> float:
    acc = 0.0
    for c in gc:
        acc = acc + float(c)
    return acc


def gyro_round(d_tile: np.ndarray, cols: np.ndarray, sample: np.ndarray, init: np.ndarray,
               cluster_size: int, iters: int) -> np.ndarray:
    """One round on one tile: cols [G][4] (the 2:4 list as groups) -> new cols."""
    g = cols.shape[0]
    n = n_clusters(g, cluster_size)
    caps = capacities(g, n)
    drawn = cols[np.arange(g), sample]                              # a_q
    points = d_tile[:, drawn].T.astype(np.float64)                  # [G][R]
    label = balanced_kmeans(points, init, iters, caps)
    new = cols.copy()
    for k in range(n):
        members = np.nonzero(label == k)[0]
        m = members.size
        quad = np.repeat(cols[members][None, :, :], m, axis=0)     # [i][j][4]: group q_j ...
        for j in range(m):
            quad[:, j, sample[members[j]]] = drawn[members]        # ... with a_{q_i} in its hole
        vals = d_tile[:, quad]                                      # [R][i][j][4]
        cost = pair_cost(np.transpose(vals, (1, 2, 0, 3)))          # [i][j]
        col_of = hungarian(cost)
        for i in range(m):
            j = col_of[i]
            new[members[j], sample[members[j]]] = drawn[members[i]]
    return new


def gyro_permutation(d: np.ndarray, perm: np.ndarray, p: oh.Plan, rounds: int, cluster_size: int,
                     iters: int, sample: np.ndarray, init: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The in-tile input-channel gyro permutation of every tile.

    d float32 [cout][cin] importance, perm int [n_tiles][cin], sample uint8
    [rounds][n_tiles][groups], init int [rounds][n_tiles][N].  Returns the
    new perm and the pruning cost of every tile before the first round and
    after each round, float64 [rounds + 1][n_tiles].
    """
    d = np.asarray(d, dtype=np.float32)
    perm = np.asarray(perm, dtype=np.int64)
    if rounds < 0 or cluster_size < 1 or iters < 1:
        raise oh.OracleError("rounds >= 0, cluster_size >= 1 and iters >= 1 are required")
    s = oh.vector_scores(d, p)
    reg = oh.regions(s, p)
    _, idx_s = oh.index_lists(reg, perm, p)
    g = p.groups
    trace = np.zeros((rounds + 1, p.n_tiles), dtype=np.float64)
    out = perm.copy()
    for t in range(p.n_tiles):
        d_tile = d[t * p.tile_rows:(t + 1) * p.tile_rows]
        cols = idx_s[t, :p.n_24].reshape(g, 4).astype(np.int64)
        trace[0, t] = total_cost(group_costs(d_tile, cols)) if g else 0.0
        for r in range(rounds):
            if g:
                cols = gyro_round(d_tile, cols, np.asarray(sample[r, t], dtype=np.int64),
                                  np.asarray(init[r, t], dtype=np.int64), cluster_size, iters)
                trace[r + 1, t] = total_cost(group_costs(d_tile, cols))
        if g:
            pos = np.nonzero(reg[t][perm[t]] == oh.TWO_FOUR)[0]     # positions of the 2:4 columns in perm[t]
            out[t, pos] = cols.reshape(-1)
    return out, trace
