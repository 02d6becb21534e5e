// hinm_gyro_permute: the in-tile input-channel gyro permutation (FlexHiNM-GP
// paper notes, key design 2), rounds of
//   1. taking one drawn column out of every 2:4 group of a tile,
//   2. a capacity-bound K-means of the drawn columns' importance vectors,
//   3. a Hungarian assignment of drawn columns to holes inside every cluster,
//      on the pruning cost (the importance the 2:4 selection drops).
// The floating-point work that decides the result (distances, centroids,
// pruning costs) runs on the device in float64 with every sum in a fixed
// order and no fused multiply-adds; the sort of the capacity-bound
// assignment and the Hungarian algorithm run on the host.  Offline work (a
// pruning-time step that produces perm), written for an exactly defined
// result rather than speed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <limits>
#include <functional>
#include <numeric>
#include <thread>
#include <vector>
#include <stdint.h>
#include <string.h>

#include "hinm_internal.h"

using hinm::fail;

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(HINM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Importance of the 2:4 columns, per tile and list position, rows contiguous:
// dc[t][p][r] = D[t R + r][idx24[t][p]].
__global__ __launch_bounds__(256) void gather_cols_kernel(const float* __restrict__ imp, int64_t ldi,
                                                          const int32_t* __restrict__ idx24, int n24, int n24_pad,
                                                          int R, int T, float* __restrict__ dc) {
  const int64_t n = (int64_t)T * n24 * R;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(e % R);
    const int64_t tp = e / R;
    const int p = (int)(tp % n24), t = (int)(tp / n24);
    const int c = idx24[(int64_t)t * n24_pad + p];
    dc[e] = imp[((int64_t)t * R + r) * ldi + c];
  }
}

// The pruning cost of four columns over the tile's rows: per row the two
// smallest importances added in float64, rows added in ascending order.
__device__ inline double quad_cost(const float* a, const float* b, const float* c, const float* d, int R) {
  double acc = 0.0;
  for (int r = 0; r < R; ++r) {
    const float m1 = fminf(a[r], b[r]), M1 = fmaxf(a[r], b[r]);
    const float m2 = fminf(c[r], d[r]), M2 = fmaxf(c[r], d[r]);
    const float lo = fminf(m1, m2), second = fminf(fmaxf(m1, m2), fminf(M1, M2));
    acc = __dadd_rn(acc, __dadd_rn((double)lo, (double)second));
  }
  return acc;
}

// Cost of every current group: cols[t][q][4] list positions.
__global__ __launch_bounds__(256) void group_cost_kernel(const float* __restrict__ dc, const int32_t* __restrict__ cols,
                                                         int n24, int G, int R, int T, double* __restrict__ out) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= (int64_t)T * G) return;
  const int t = (int)(e / G);
  const int32_t* q = cols + e * 4;
  const float* base = dc + (int64_t)t * n24 * R;
  out[e] = quad_cost(base + (int64_t)q[0] * R, base + (int64_t)q[1] * R, base + (int64_t)q[2] * R,
                     base + (int64_t)q[3] * R, R);
}

// Centroids start at drawn vectors: cent[t][k][r] = dc[t][drawn[t][init[t][k]]][r].
__global__ __launch_bounds__(256) void init_cent_kernel(const float* __restrict__ dc, const int32_t* __restrict__ drawn,
                                                        const int32_t* __restrict__ init, int n24, int G, int N, int R,
                                                        int T, double* __restrict__ cent) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= (int64_t)T * N * R) return;
  const int r = (int)(e % R);
  const int64_t tk = e / R;
  const int k = (int)(tk % N), t = (int)(tk / N);
  const int q = init[(int64_t)t * N + k];
  cent[e] = (double)dc[((int64_t)t * n24 + drawn[(int64_t)t * G + q]) * R + r];
}

// Squared distances of the drawn vectors to the centroids, rows in ascending order.
__global__ __launch_bounds__(256) void dist_kernel(const float* __restrict__ dc, const int32_t* __restrict__ drawn,
                                                   const double* __restrict__ cent, int n24, int G, int N, int R, int T,
                                                   double* __restrict__ dist) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= (int64_t)T * G * N) return;
  const int k = (int)(e % N);
  const int64_t tq = e / N;
  const int t = (int)(tq / G);
  const float* x = dc + ((int64_t)t * n24 + drawn[tq]) * R;
  const double* c = cent + ((int64_t)t * N + k) * R;
  double acc = 0.0;
  for (int r = 0; r < R; ++r) {
    const double d = __dsub_rn((double)x[r], c[r]);
    acc = __dadd_rn(acc, __dmul_rn(d, d));
  }
  dist[e] = acc;
}

// Centroid = mean of the members' vectors, members in ascending order.
__global__ __launch_bounds__(256) void update_cent_kernel(const float* __restrict__ dc,
                                                          const int32_t* __restrict__ drawn,
                                                          const int32_t* __restrict__ label, int n24, int G, int N,
                                                          int R, int T, double* __restrict__ cent) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= (int64_t)T * N * R) return;
  const int r = (int)(e % R);
  const int64_t tk = e / R;
  const int k = (int)(tk % N), t = (int)(tk / N);
  double acc = 0.0;
  int n = 0;
  for (int q = 0; q < G; ++q) {
    if (label[(int64_t)t * G + q] != k) continue;
    acc = __dadd_rn(acc, (double)dc[((int64_t)t * n24 + drawn[(int64_t)t * G + q]) * R + r]);
    ++n;
  }
  cent[e] = __ddiv_rn(acc, (double)n);
}

// Cost matrices of the clusters: for cluster k of tile t with members
// memb[moff[k] .. moff[k+1]) (groups, ascending), entry (i, j) is the cost
// of group q_j with the drawn column of q_i in its hole.
__global__ __launch_bounds__(256) void cost_kernel(const float* __restrict__ dc, const int32_t* __restrict__ cols,
                                                   const uint8_t* __restrict__ hole, const int32_t* __restrict__ memb,
                                                   const int32_t* __restrict__ moff, const int64_t* __restrict__ coff,
                                                   int n24, int G, int N, int R, int T, int cap_max,
                                                   double* __restrict__ cost) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t per_tile = (int64_t)N * cap_max * cap_max;
  if (e >= (int64_t)T * per_tile) return;
  const int t = (int)(e / per_tile);
  const int64_t rest = e % per_tile;
  const int k = (int)(rest / ((int64_t)cap_max * cap_max));
  const int i = (int)(rest / cap_max % cap_max), j = (int)(rest % cap_max);
  const int32_t* mo = moff + (int64_t)t * (N + 1);
  const int m = mo[k + 1] - mo[k];
  if (i >= m || j >= m) return;
  const int qi = memb[(int64_t)t * G + mo[k] + i], qj = memb[(int64_t)t * G + mo[k] + j];
  const int32_t* gj = cols + ((int64_t)t * G + qj) * 4;
  const int32_t* gi = cols + ((int64_t)t * G + qi) * 4;
  const int h = hole[(int64_t)t * G + qj];
  const int drawn_i = gi[hole[(int64_t)t * G + qi]];
  int pos[4];
  for (int u = 0; u < 4; ++u) pos[u] = u == h ? drawn_i : gj[u];
  const float* base = dc + (int64_t)t * n24 * R;
  cost[coff[(int64_t)t * (N + 1) + k] + (int64_t)i * m + j] =
      quad_cost(base + (int64_t)pos[0] * R, base + (int64_t)pos[1] * R, base + (int64_t)pos[2] * R,
                base + (int64_t)pos[3] * R, R);
}

// Minimum-cost assignment of an n x n matrix (row-major): col[i] = column of
// row i.  Shortest augmenting paths with row and column potentials, one row
// at a time (Kuhn-Munkres, O(n^3)); on equal reduced costs the lowest column
// index is taken.
void hungarian(const double* a, int n, int* col) {
  const double inf = std::numeric_limits<double>::infinity();
  std::vector<double> u(n + 1, 0.0), v(n + 1, 0.0), minv(n + 1);
  std::vector<int> match(n + 1, 0), way(n + 1, 0);
  std::vector<char> used(n + 1);
  for (int i = 1; i <= n; ++i) {
    match[0] = i;
    int j0 = 0;
    std::fill(minv.begin(), minv.end(), inf);
    std::fill(used.begin(), used.end(), 0);
    for (;;) {
      used[j0] = 1;
      const int i0 = match[j0];
      double delta = inf;
      int j1 = 0;
      for (int j = 1; j <= n; ++j) {
        if (used[j]) continue;
        const double cur = a[(size_t)(i0 - 1) * n + (j - 1)] - u[i0] - v[j];
        if (cur < minv[j]) {
          minv[j] = cur;
          way[j] = j0;
        }
        if (minv[j] < delta) {
          delta = minv[j];
          j1 = j;
        }
      }
      for (int j = 0; j <= n; ++j) {
        if (used[j]) {
          u[match[j]] += delta;
          v[j] -= delta;
        } else {
          minv[j] -= delta;
        }
      }
      j0 = j1;
      if (match[j0] == 0) break;
    }
    for (;;) {
      const int j1 = way[j0];
      match[j0] = match[j1];
      j0 = j1;
      if (j0 == 0) break;
    }
  }
  for (int j = 1; j <= n; ++j) col[match[j] - 1] = j - 1;
}

// Every point to the cluster of the first (distance, point, cluster) triple
// in increasing order that still has room.  Scanning the sorted G x N
// triples is done with a heap holding, for every unassigned point, its
// smallest triple not yet looked at: the heap's minimum is then always the
// next triple of the full scan that concerns an unassigned point, so the
// decisions are the same.
void balanced_assign(const double* dist, int G, int N, const std::vector<int>& caps, int* label) {
  struct Key {
    double d;
    int q, k;
    bool operator>(const Key& o) const {
      if (d != o.d) return d > o.d;
      if (q != o.q) return q > o.q;
      return k > o.k;
    }
  };
  std::vector<int> order((size_t)G * N);        // clusters of each point by (distance, cluster)
  std::vector<int> next(G, 0);
  for (int q = 0; q < G; ++q) {
    int* o = order.data() + (size_t)q * N;
    const double* dq = dist + (size_t)q * N;
    std::iota(o, o + N, 0);
    std::sort(o, o + N, [&](int a, int b) { return dq[a] != dq[b] ? dq[a] < dq[b] : a < b; });
  }
  std::vector<Key> heap;
  heap.reserve(G);
  for (int q = 0; q < G; ++q) {
    const int k = order[(size_t)q * N];
    heap.push_back({dist[(size_t)q * N + k], q, k});
  }
  std::make_heap(heap.begin(), heap.end(), std::greater<Key>());
  std::vector<int> room(caps);
  for (int q = 0; q < G; ++q) label[q] = -1;
  while (!heap.empty()) {
    std::pop_heap(heap.begin(), heap.end(), std::greater<Key>());
    const Key top = heap.back();
    heap.pop_back();
    if (room[top.k] > 0) {
      label[top.q] = top.k;
      --room[top.k];
    } else if (++next[top.q] < N) {
      const int k = order[(size_t)top.q * N + next[top.q]];
      heap.push_back({dist[(size_t)top.q * N + k], top.q, k});
      std::push_heap(heap.begin(), heap.end(), std::greater<Key>());
    }
  }
}

// f(t) for t in [0, T) on up to 16 host threads.
template <class F>
void for_tiles(int T, F f) {
  const int nt = std::max(1, std::min<int>({T, 16, (int)std::thread::hardware_concurrency()}));
  if (nt <= 1) {
    for (int t = 0; t < T; ++t) f(t);
    return;
  }
  std::vector<std::thread> th;
  for (int w = 0; w < nt; ++w)
    th.emplace_back([&, w] {
      for (int t = w; t < T; t += nt) f(t);
    });
  for (auto& x : th) x.join();
}

struct GyroShape {
  int T, cin, R, n24, n24_pad, n_dense_pad, G, N, cap_max;
};

GyroShape gyro_shape(const hinm_plan_t& p, int32_t cluster_size) {
  GyroShape s;
  s.T = p.n_tiles;
  s.cin = p.cin;
  s.R = p.tile_rows;
  s.n24 = p.n_24;
  s.n24_pad = p.n_24_pad;
  s.n_dense_pad = p.n_dense_pad;
  s.G = p.groups;
  s.N = s.G ? (s.G + cluster_size - 1) / cluster_size : 0;
  s.cap_max = s.N ? (s.G + s.N - 1) / s.N : 0;
  return s;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace: [pack stages: flag, scores, regions][idx_dense][idx_24][dc]
// [cols][hole][drawn][label][memb][moff][coff][cent][dist][cost][gcost]
struct GyroWs {
  size_t pack, idx_d, idx_24, dc, cols, hole, drawn, label, memb, moff, coff, cent, dist, cost, gcost, total;
};

GyroWs gyro_ws(const hinm_plan_t& p, const GyroShape& s) {
  GyroWs w;
  size_t pack_bytes = 0;
  hinm_pack_workspace_bytes(&p, &pack_bytes);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  const size_t TG = (size_t)s.T * s.G;
  w.pack = take(pack_bytes);
  w.idx_d = take((size_t)s.T * s.n_dense_pad * 4);
  w.idx_24 = take((size_t)s.T * s.n24_pad * 4);
  w.dc = take((size_t)s.T * s.n24 * s.R * 4);
  w.cols = take(TG * 16);
  w.hole = take(TG);
  w.drawn = take(TG * 4);
  w.label = take(TG * 4);
  w.memb = take(TG * 4);
  w.moff = take((size_t)s.T * (s.N + 1) * 4);
  w.coff = take((size_t)s.T * (s.N + 1) * 8);
  w.cent = take((size_t)s.T * s.N * s.R * 8);
  w.dist = take(TG * s.N * 8);
  w.cost = take((size_t)s.T * s.N * s.cap_max * s.cap_max * 8);
  w.gcost = take(TG * 8);
  w.total = o;
  return w;
}

unsigned blocks_for(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1 << 20)); }

}  // namespace

extern "C" int hinm_gyro_workspace_bytes(const hinm_plan_t* plan, int32_t cluster_size, size_t* bytes) {
  hinm::clear_error();
  int st = hinm::check_plan(plan);
  if (st) return st;
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  if (cluster_size < 1) return fail(HINM_EINVAL, "cluster_size must be >= 1");
  *bytes = gyro_ws(*plan, gyro_shape(*plan, cluster_size)).total;
  return HINM_OK;
}

extern "C" int hinm_gyro_permute(const hinm_plan_t* plan, const float* importance, int64_t ldi, int32_t* perm,
                                 int32_t rounds, int32_t cluster_size, int32_t kmeans_iters, const uint8_t* sample,
                                 const int32_t* init, double* cost_trace, void* workspace, size_t workspace_bytes,
                                 void* stream_) {
  hinm::clear_error();
  int st = hinm::check_plan(plan);
  if (st) return st;
  const hinm_plan_t& p = *plan;
  if (!importance || !perm) return fail(HINM_EINVAL, "importance and perm must be non-NULL");
  if (rounds < 0 || cluster_size < 1 || kmeans_iters < 1)
    return fail(HINM_EINVAL, "rounds >= 0, cluster_size >= 1 and kmeans_iters >= 1 are required");
  if (ldi < p.cin) return fail(HINM_ESHAPE, "ldi=%lld must be >= cin=%d", (long long)ldi, p.cin);
  if (p.cin > (1 << 20)) return fail(HINM_ESHAPE, "cin=%d exceeds the 2^20 supported by the permutation check", p.cin);
  if (!hinm::aligned(importance, 4) || !hinm::aligned(perm, 4))
    return fail(HINM_EALIGN, "importance and perm must be 4-byte aligned");
  const GyroShape s = gyro_shape(p, cluster_size);
  const int T = s.T, G = s.G, N = s.N, R = s.R;
  if (rounds > 0 && G > 0) {
    if (!sample || !init) return fail(HINM_EINVAL, "sample and init must be non-NULL");
    for (int64_t e = 0; e < (int64_t)rounds * T * G; ++e)
      if (sample[e] > 3) return fail(HINM_EINVAL, "sample[%lld] = %d is not a position 0..3", (long long)e, sample[e]);
    std::vector<char> seen(G);
    for (int64_t rt = 0; rt < (int64_t)rounds * T; ++rt) {
      std::fill(seen.begin(), seen.end(), 0);
      for (int k = 0; k < N; ++k) {
        const int q = init[rt * N + k];
        if (q < 0 || q >= G || seen[q])
          return fail(HINM_EINVAL, "init of round %lld, tile %lld: %d is not a distinct group 0..%d",
                      (long long)(rt / T), (long long)(rt % T), q, G - 1);
        seen[q] = 1;
      }
    }
  }
  const GyroWs w = gyro_ws(p, s);
  if (!workspace || workspace_bytes < w.total)
    return fail(HINM_EWORKSPACE, "gyro workspace of %zu bytes given, %zu needed", workspace_bytes, w.total);
  if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  st = hinm::ensure_device();
  if (st) return st;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  int32_t* d_idx24 = reinterpret_cast<int32_t*>(ws + w.idx_24);
  float* d_dc = reinterpret_cast<float*>(ws + w.dc);
  int32_t* d_cols = reinterpret_cast<int32_t*>(ws + w.cols);
  uint8_t* d_hole = reinterpret_cast<uint8_t*>(ws + w.hole);
  int32_t* d_drawn = reinterpret_cast<int32_t*>(ws + w.drawn);
  int32_t* d_label = reinterpret_cast<int32_t*>(ws + w.label);
  int32_t* d_memb = reinterpret_cast<int32_t*>(ws + w.memb);
  int32_t* d_moff = reinterpret_cast<int32_t*>(ws + w.moff);
  int64_t* d_coff = reinterpret_cast<int64_t*>(ws + w.coff);
  double* d_cent = reinterpret_cast<double*>(ws + w.cent);
  double* d_dist = reinterpret_cast<double*>(ws + w.dist);
  double* d_cost = reinterpret_cast<double*>(ws + w.cost);
  double* d_gcost = reinterpret_cast<double*>(ws + w.gcost);

  // Regions and the 2:4 lists (with the perm and importance checks).
  st = hinm::region_lists(p, importance, ldi, perm, reinterpret_cast<int32_t*>(ws + w.idx_d), d_idx24, ws + w.pack,
                          stream);
  if (st) return st;
  if (G == 0) {
    if (cost_trace) std::fill(cost_trace, cost_trace + (size_t)(rounds + 1) * T, 0.0);
    hipError_t e = hipStreamSynchronize(stream);
    return e == hipSuccess ? HINM_OK : hip_fail(e, "gyro");
  }
  hipLaunchKernelGGL(gather_cols_kernel, dim3(blocks_for((int64_t)T * s.n24 * R)), dim3(256), 0, stream, importance,
                     ldi, d_idx24, s.n24, s.n24_pad, R, T, d_dc);

  // Groups as list positions: cols[t][q][u] (group q = list entries 4q..4q+3 at the start).
  std::vector<int32_t> cols((size_t)T * G * 4);
  for (int t = 0; t < T; ++t)
    for (int q = 0; q < G; ++q)
      for (int u = 0; u < 4; ++u) cols[((size_t)t * G + q) * 4 + u] = 4 * q + u;
  std::vector<double> gcost((size_t)T * G);
  auto sum_costs = [&](double* out_row) {
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int q = 0; q < G; ++q) acc += gcost[(size_t)t * G + q];
      out_row[t] = acc;
    }
  };
  hipError_t e = hipMemcpyAsync(d_cols, cols.data(), cols.size() * 4, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "gyro upload");
  if (cost_trace) {
    hipLaunchKernelGGL(group_cost_kernel, dim3(blocks_for((int64_t)T * G)), dim3(256), 0, stream, d_dc, d_cols,
                       s.n24, G, R, T, d_gcost);
    e = hipMemcpyAsync(gcost.data(), d_gcost, gcost.size() * 8, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "gyro group costs");
    sum_costs(cost_trace);
  }

  std::vector<int> caps(N);
  for (int k = 0; k < N; ++k) caps[k] = G / N + (k < G % N ? 1 : 0);
  std::vector<uint8_t> hole((size_t)T * G);
  std::vector<int32_t> drawn((size_t)T * G), label((size_t)T * G), memb((size_t)T * G), moff((size_t)T * (N + 1));
  std::vector<int64_t> coff((size_t)T * (N + 1));
  std::vector<double> dist((size_t)T * G * N), cost((size_t)T * N * s.cap_max * s.cap_max);
  for (int r = 0; r < rounds; ++r) {
    // 1. one drawn column per group
    for (int t = 0; t < T; ++t)
      for (int q = 0; q < G; ++q) {
        const size_t tq = (size_t)t * G + q;
        hole[tq] = sample[((size_t)r * T + t) * G + q];
        drawn[tq] = cols[tq * 4 + hole[tq]];
      }
    e = hipMemcpyAsync(d_hole, hole.data(), hole.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(d_drawn, drawn.data(), drawn.size() * 4, hipMemcpyHostToDevice, stream);
    // 2. capacity-bound K-means of the drawn vectors
    if (e == hipSuccess)
      e = hipMemcpyAsync(d_label, init + (size_t)r * T * N, (size_t)T * N * 4, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "gyro upload");
    hipLaunchKernelGGL(init_cent_kernel, dim3(blocks_for((int64_t)T * N * R)), dim3(256), 0, stream, d_dc, d_drawn,
                       d_label, s.n24, G, N, R, T, d_cent);
    for (int it = 0; it < kmeans_iters; ++it) {
      hipLaunchKernelGGL(dist_kernel, dim3(blocks_for((int64_t)T * G * N)), dim3(256), 0, stream, d_dc, d_drawn,
                         d_cent, s.n24, G, N, R, T, d_dist);
      e = hipMemcpyAsync(dist.data(), d_dist, dist.size() * 8, hipMemcpyDeviceToHost, stream);
      if (e == hipSuccess) e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "gyro distances");
      for_tiles(T, [&](int t) {
        balanced_assign(dist.data() + (size_t)t * G * N, G, N, caps, label.data() + (size_t)t * G);
      });
      if (it + 1 < kmeans_iters) {
        e = hipMemcpyAsync(d_label, label.data(), label.size() * 4, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "gyro upload");
        hipLaunchKernelGGL(update_cent_kernel, dim3(blocks_for((int64_t)T * N * R)), dim3(256), 0, stream, d_dc,
                           d_drawn, d_label, s.n24, G, N, R, T, d_cent);
      }
    }
    // 3. cost matrices of the clusters, Hungarian assignment inside each
    for (int t = 0; t < T; ++t) {
      int32_t* mo = moff.data() + (size_t)t * (N + 1);
      int64_t* co = coff.data() + (size_t)t * (N + 1);
      mo[0] = 0;
      co[0] = 0;
      for (int k = 0; k < N; ++k) {
        int m = 0;
        for (int q = 0; q < G; ++q)
          if (label[(size_t)t * G + q] == k) memb[(size_t)t * G + mo[k] + m++] = q;
        mo[k + 1] = mo[k] + m;
        co[k + 1] = co[k] + (int64_t)m * m;
      }
      for (int k = 0; k <= N; ++k) co[k] += (int64_t)t * N * s.cap_max * s.cap_max;
    }
    e = hipMemcpyAsync(d_memb, memb.data(), memb.size() * 4, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(d_moff, moff.data(), moff.size() * 4, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(d_coff, coff.data(), coff.size() * 8, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "gyro upload");
    hipLaunchKernelGGL(cost_kernel, dim3(blocks_for((int64_t)T * N * s.cap_max * s.cap_max)), dim3(256), 0, stream,
                       d_dc, d_cols, d_hole, d_memb, d_moff, d_coff, s.n24, G, N, R, T, s.cap_max, d_cost);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(cost.data(), d_cost, cost.size() * 8, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "gyro costs");
    for_tiles(T, [&](int t) {
      const int32_t* mo = moff.data() + (size_t)t * (N + 1);
      const int64_t* co = coff.data() + (size_t)t * (N + 1);
      std::vector<int> col_of(s.cap_max);
      for (int k = 0; k < N; ++k) {
        const int m = mo[k + 1] - mo[k];
        const int32_t* mem = memb.data() + (size_t)t * G + mo[k];
        const double* c = cost.data() + co[k];
        hungarian(c, m, col_of.data());
        for (int i = 0; i < m; ++i) {
          const int j = col_of[i];
          const size_t tqj = (size_t)t * G + mem[j];
          cols[tqj * 4 + hole[tqj]] = drawn[(size_t)t * G + mem[i]];
          gcost[tqj] = c[(size_t)i * m + j];
        }
      }
    });
    e = hipMemcpyAsync(d_cols, cols.data(), cols.size() * 4, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "gyro upload");
    if (cost_trace) sum_costs(cost_trace + (size_t)(r + 1) * T);
  }

  // The new perm: the 2:4 columns, in their new list order, go to the
  // positions the 2:4 columns held; every other position keeps its column.
  std::vector<int32_t> hperm((size_t)T * s.cin), list((size_t)T * s.n24_pad);
  e = hipMemcpyAsync(hperm.data(), perm, hperm.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(list.data(), d_idx24, list.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "gyro perm");
  std::vector<char> is24(s.cin);
  for (int t = 0; t < T; ++t) {
    const int32_t* L = list.data() + (size_t)t * s.n24_pad;
    std::fill(is24.begin(), is24.end(), 0);
    for (int pidx = 0; pidx < s.n24; ++pidx) is24[L[pidx]] = 1;
    int32_t* pr = hperm.data() + (size_t)t * s.cin;
    int pidx = 0;
    for (int j = 0; j < s.cin; ++j)
      if (is24[pr[j]]) {
        pr[j] = L[cols[((size_t)t * G + pidx / 4) * 4 + pidx % 4]];
        ++pidx;
      }
  }
  e = hipMemcpyAsync(perm, hperm.data(), hperm.size() * 4, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "gyro perm");
  return HINM_OK;
}
