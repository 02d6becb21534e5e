// hinm_pack: vector scoring, region ranking, permuted index lists, 2:4 top-2
// selection with 2-bit metadata, and the dense-region value gather, for
// gfx950.  A one-time transform of a weight; written for exactness (bit
// identical to the definition) more than speed, but every kernel is a plain
// data-parallel pass with coalesced stores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>
#include <math.h>
#include <stdint.h>

#include "hinm_internal.h"

using hinm::fail;

namespace {

constexpr uint8_t kPruned = 0, kTwoFour = 1, kDense = 2;

// Where tile t's K-blocks and counts are: from the per-tile table
// (first dense block, n_dense, first 2:4 block, n_24) when there is one,
// else the uniform layout (every tile the same counts, tiles end to end).
struct TileDesc {
  int kd0, n_dense, ks0, n_24;
};
__device__ inline TileDesc tile_desc(const int32_t* tiles, int t, int n_dense, int n_dense_pad, int n_24,
                                     int n_24_pad) {
  if (tiles) return {tiles[4 * t], tiles[4 * t + 1], tiles[4 * t + 2], tiles[4 * t + 3]};
  return {t * (n_dense_pad / 32), n_dense, t * (n_24_pad / 64), n_24};
}
constexpr int kFlagPerm = 1, kFlagImportance = 2;
// set when some perm row moves a column out of its aligned block of 64 positions
constexpr int kFlagNotBlock64 = 4;

__global__ void zero_flag_kernel(int* flag) {
  if (threadIdx.x < 64) flag[threadIdx.x] = 0;
}

// Every perm row must hold each of 0..cin-1 once.  One workgroup per tile
// marks seen columns in an LDS bitmap; an out-of-range or repeated entry sets
// the error flag.  cin entries with no repeat cover all cin values.
__global__ __launch_bounds__(1024) void check_perm_kernel(const int32_t* __restrict__ perm, int cin,
                                                          int* __restrict__ flag) {
  extern __shared__ uint32_t seen[];
  const int nw = (cin + 31) >> 5;
  for (int i = threadIdx.x; i < nw; i += blockDim.x) seen[i] = 0u;
  __syncthreads();
  const int32_t* row = perm + (int64_t)blockIdx.x * cin;
  bool bad = false, off_block = false;
  for (int j = threadIdx.x; j < cin; j += blockDim.x) {
    const int c = row[j];
    if (c < 0 || c >= cin) {
      bad = true;
      continue;
    }
    off_block |= (c >> 6) != (j >> 6);
    const uint32_t m = 1u << (c & 31);
    if (atomicOr(&seen[c >> 5], m) & m) bad = true;
  }
  if (bad) atomicOr(flag, kFlagPerm);
  if (off_block) atomicOr(flag, kFlagNotBlock64);
}

// Score of the vector (tile t, column c): sum over the tile's rows of the
// importance, in float64, ascending rows, from +0.0 (one thread per column so
// the order is exactly that).  Also rejects negative or non-finite importance.
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ imp, int64_t ldi, int cin,
                                                     int rows, double* __restrict__ s, int* __restrict__ flag) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
  if (c >= cin) return;
  const float* col = imp + (int64_t)t * rows * ldi + c;
  double acc = 0.0;
  bool bad = false;
  for (int r = 0; r < rows; ++r) {
    const float v = col[(int64_t)r * ldi];
    bad |= !(v >= 0.0f) || isinf(v);
    acc += (double)v;
  }
  if (bad) atomicOr(flag, kFlagImportance);
  s[(int64_t)t * cin + c] = acc;
}

// Region of every column: its rank under (-score, column) decides it.  The
// rank is counted directly, comparing against every column of the tile; the
// loop index is uniform across the wave, so each score is read once per wave.
__global__ __launch_bounds__(256) void regions_kernel(const double* __restrict__ s, int cin, int n_dense,
                                                      int n_24, uint8_t* __restrict__ reg,
                                                      const int32_t* __restrict__ tiles) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
  if (tiles) {
    n_dense = tiles[4 * t + 1];
    n_24 = tiles[4 * t + 3];
  }
  const double* st = s + (int64_t)t * cin;
  const double sc = c < cin ? st[c] : 0.0;
  int rank = 0;
  for (int j = 0; j < cin; ++j) {
    const double sj = st[j];
    rank += (sj > sc) | ((sj == sc) & (j < c));
  }
  if (c < cin) reg[(int64_t)t * cin + c] = rank < n_dense ? kDense : (rank < n_dense + n_24 ? kTwoFour : kPruned);
}

// Index lists in permuted order: walk perm[t][0..cin) and append each column
// to the list of its region (an exclusive prefix count per region).  One
// workgroup of 1024 threads per tile, chunks of 1024 positions.
__global__ __launch_bounds__(1024) void compact_kernel(const int32_t* __restrict__ perm, const uint8_t* __restrict__ reg,
                                                       int cin, int n_dense_pad, int n_24_pad,
                                                       int32_t* __restrict__ idx_d, int32_t* __restrict__ idx_s,
                                                       const int32_t* __restrict__ tiles) {
  __shared__ int wd[16], ws[16];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int32_t* od = idx_d + (int64_t)t * n_dense_pad;
  int32_t* os = idx_s + (int64_t)t * n_24_pad;
  if (tiles) {   // this tile's lists and pads
    od = idx_d + (int64_t)tiles[4 * t] * 32;
    os = idx_s + (int64_t)tiles[4 * t + 2] * 64;
    n_dense_pad = (tiles[4 * t + 1] + 31) / 32 * 32;
    n_24_pad = (tiles[4 * t + 3] + 63) / 64 * 64;
  }
  int base_d = 0, base_s = 0;
  for (int j0 = 0; j0 < cin; j0 += 1024) {
    const int j = j0 + threadIdx.x;
    int c = -1;
    uint8_t r = kPruned;
    if (j < cin) {
      c = perm ? perm[(int64_t)t * cin + j] : j;
      if (c >= 0 && c < cin) r = reg[(int64_t)t * cin + c];
    }
    const uint64_t bd = __ballot(r == kDense), bs = __ballot(r == kTwoFour);
    if (lane == 0) {
      wd[wave] = __popcll(bd);
      ws[wave] = __popcll(bs);
    }
    __syncthreads();
    int pd = base_d + __popcll(bd & below), ps = base_s + __popcll(bs & below);
    int tot_d = 0, tot_s = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < wave) {
        pd += wd[k];
        ps += ws[k];
      }
      tot_d += wd[k];
      tot_s += ws[k];
    }
    if (r == kDense && pd < n_dense_pad) od[pd] = c;
    if (r == kTwoFour && ps < n_24_pad) os[ps] = c;
    base_d += tot_d;
    base_s += tot_s;
    __syncthreads();
  }
  for (int i = min(base_d, n_dense_pad) + threadIdx.x; i < n_dense_pad; i += blockDim.x) od[i] = -1;
  for (int i = min(base_s, n_24_pad) + threadIdx.x; i < n_24_pad; i += blockDim.x) os[i] = -1;
}

// 2:4 encode: one thread per (tile, 64-position block, row), rows fastest so
// the 64-byte value rows and the metadata words are stored contiguously.  In
// each group of four listed columns the first two by (-importance, position)
// are kept; the nibble is i0 | i1 << 2 with i0 < i1 (2:4 article, section 3).
__global__ __launch_bounds__(256) void encode24_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                       const float* __restrict__ imp, int64_t ldi,
                                                       const int32_t* __restrict__ idx_s, int cin, int rows,
                                                       int n_tiles, int groups, int n_24_pad,
                                                       uint16_t* __restrict__ val_s, uint64_t* __restrict__ meta,
                                                       const int32_t* __restrict__ tiles) {
  const int nkb = n_24_pad / 64;   // blocks per tile (the largest, with a tile table)
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tiles * nkb * rows) return;
  const int r = (int)(gid % rows);
  const int64_t tk = gid / rows;
  const int kb = (int)(tk % nkb);
  const int t = (int)(tk / nkb);
  const TileDesc td = tile_desc(tiles, t, 0, 0, groups * 4, n_24_pad);
  if (tiles) {
    if (kb >= (td.n_24 + 63) / 64) return;
    groups = td.n_24 / 4;
  }
  const int blk = td.ks0 + kb;     // this block's index in the 2:4 buffers
  const int64_t grow = (int64_t)t * rows + r;
  const int32_t* il = idx_s + (int64_t)blk * 64;
  uint64_t m = 0;
  uint32_t packed[16];
  for (int g = 0; g < 16; ++g) {
    const int q = kb * 16 + g;
    uint32_t nib = 0x4u, v0 = 0u, v1 = 0u;
    if (q < groups) {
      int cc[4];
      float a[4];
      for (int k = 0; k < 4; ++k) {
        cc[k] = il[4 * g + k];
        a[k] = (cc[k] >= 0 && cc[k] < cin) ? imp[grow * ldi + cc[k]] : -1.0f;
      }
      int i0 = 0;
      for (int k = 1; k < 4; ++k)
        if (a[k] > a[i0]) i0 = k;
      int i1 = i0 == 0 ? 1 : 0;
      for (int k = i1 + 1; k < 4; ++k)
        if (k != i0 && a[k] > a[i1]) i1 = k;
      const int lo = i0 < i1 ? i0 : i1, hi = i0 < i1 ? i1 : i0;
      nib = (uint32_t)(lo | (hi << 2));
      if (cc[lo] >= 0 && cc[lo] < cin) v0 = w[grow * ldw + cc[lo]];
      if (cc[hi] >= 0 && cc[hi] < cin) v1 = w[grow * ldw + cc[hi]];
    }
    m |= (uint64_t)nib << (4 * g);
    packed[g] = v0 | (v1 << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(val_s + ((int64_t)blk * rows + r) * 32);
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  meta[(int64_t)blk * rows + r] = m;
}

// Dense-region gather: val_d[t][kb][r][k] = W[t*R + r][idx_d[t][32 kb + k]].
__global__ __launch_bounds__(256) void gather_dense_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                           const int32_t* __restrict__ idx_d, int cin, int rows,
                                                           int n_tiles, int n_dense_pad, uint16_t* __restrict__ val_d,
                                                           const int32_t* __restrict__ tiles) {
  const int nkb = n_dense_pad / 32;   // blocks per tile (the largest, with a tile table)
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tiles * nkb * rows) return;
  const int r = (int)(gid % rows);
  const int64_t tk = gid / rows;
  const int kb = (int)(tk % nkb);
  const int t = (int)(tk / nkb);
  const TileDesc td = tile_desc(tiles, t, 0, n_dense_pad, 0, 0);
  if (tiles && kb >= (td.n_dense + 31) / 32) return;
  const int blk = td.kd0 + kb;     // this block's index in the dense buffers
  const int64_t grow = (int64_t)t * rows + r;
  const int32_t* il = idx_d + (int64_t)blk * 32;
  uint32_t packed[16];
  for (int k = 0; k < 32; k += 2) {
    const int c0 = il[k], c1 = il[k + 1];
    const uint32_t v0 = (c0 >= 0 && c0 < cin) ? w[grow * ldw + c0] : 0u;
    const uint32_t v1 = (c1 >= 0 && c1 < cin) ? w[grow * ldw + c1] : 0u;
    packed[k / 2] = v0 | (v1 << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(val_d + ((int64_t)blk * rows + r) * 32);
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HINM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Cross-layer index translation: every index i >= 0 of the packed lists
// becomes map[i]; pads (-1) stay.  map has been checked to be a permutation.
__global__ __launch_bounds__(256) void translate_kernel(int32_t* __restrict__ idx, int64_t n,
                                                        const int32_t* __restrict__ map) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t v = idx[i];
  if (v >= 0) idx[i] = map[v];
}

// ---------------------------------------------------------------------------
// Boundary search on the device (FlexHiNM-GP notes, key design 1): the
// column ranking does not depend on v_s, so it is computed once; each grid
// point then only moves the two cuts, rebuilds the 2:4 groups in permuted
// order and sums the retained importance.
// ---------------------------------------------------------------------------

// rank[t][c] = position of column c under the order (-score, column).
__global__ __launch_bounds__(256) void rank_kernel(const double* __restrict__ s, int cin, int32_t* __restrict__ rank) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
  const double* st = s + (int64_t)t * cin;
  const double sc = c < cin ? st[c] : 0.0;
  int r = 0;
  for (int j = 0; j < cin; ++j) {
    const double sj = st[j];
    r += (sj > sc) | ((sj == sc) & (j < c));
  }
  if (c < cin) rank[(int64_t)t * cin + c] = r;
}

__global__ __launch_bounds__(256) void cut_kernel(const int32_t* __restrict__ rank, int64_t n, int n_dense, int n_24,
                                                  uint8_t* __restrict__ reg) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int r = rank[i];
  reg[i] = r < n_dense ? kDense : (r < n_dense + n_24 ? kTwoFour : kPruned);
}

// Fixed-order sum of 256 per-thread values (thread 0 holds the result).
__device__ inline double block_sum_256(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  return sh[0];
}

// R_dense of tile t: sum of the scores of its dense columns.  Thread k adds
// columns k, k+256, ... in ascending order, then a fixed tree: the same
// float64 value on every run.
__global__ __launch_bounds__(256) void rdense_kernel(const double* __restrict__ s, const int32_t* __restrict__ rank,
                                                     int cin, int n_dense, double* __restrict__ part) {
  __shared__ double sh[256];
  const int t = blockIdx.x;
  double acc = 0.0;
  for (int c = threadIdx.x; c < cin; c += 256)
    if (rank[(int64_t)t * cin + c] < n_dense) acc += s[(int64_t)t * cin + c];
  const double tot = block_sum_256(acc, sh);
  if (threadIdx.x == 0) part[t] = tot;
}

// R_24 of one row of tile t: over its 2:4 groups, the two largest
// importances of each group (the kept pair; ties do not change the sum),
// added in float64.  Thread k takes groups k, k+256, ...; fixed tree.
__global__ __launch_bounds__(256) void r24_kernel(const float* __restrict__ imp, int64_t ldi,
                                                  const int32_t* __restrict__ idx_s, int n_24_pad, int groups, int rows,
                                                  double* __restrict__ part) {
  __shared__ double sh[256];
  const int t = blockIdx.y, r = blockIdx.x;
  const float* row = imp + ((int64_t)t * rows + r) * ldi;
  const int32_t* list = idx_s + (int64_t)t * n_24_pad;
  double acc = 0.0;
  for (int q = threadIdx.x; q < groups; q += 256) {
    float a[4];
    for (int k = 0; k < 4; ++k) a[k] = row[list[4 * q + k]];
    // two largest of four
    float m1 = fmaxf(a[0], a[1]), n1 = fminf(a[0], a[1]);
    float m2 = fmaxf(a[2], a[3]), n2 = fminf(a[2], a[3]);
    const float top = fmaxf(m1, m2);
    const float second = fmaxf(fminf(m1, m2), fmaxf(n1, n2));
    acc += (double)top + (double)second;
  }
  const double tot = block_sum_256(acc, sh);
  if (threadIdx.x == 0) part[(int64_t)t * rows + r] = tot;
}

}  // namespace

// Shape of a pack: the uniform counts, or (with a tile table on the device)
// the largest per-tile pads, which size the launch grids.
struct PackShape {
  int T, cin, R;
  int n_dense, n_24, n_dense_pad, n_24_pad, groups;
  int64_t bytes_val_dense, bytes_idx_dense, bytes_val_24, bytes_meta_24, bytes_idx_24;
};

static int pack_core(const PackShape& p, const int32_t* tiles, const void* w_bf16, int64_t ldw,
                     const float* importance, int64_t ldi, const int32_t* perm, void* val_dense, int32_t* idx_dense,
                     void* val_24, uint64_t* meta_24, int32_t* idx_24, void* workspace, size_t workspace_bytes,
                     size_t need, void* stream_, uint32_t* packed_flags = nullptr) {
  if (!w_bf16 || !importance) return fail(HINM_EINVAL, "w and importance must be non-NULL");
  if (ldw < p.cin || ldi < p.cin)
    return fail(HINM_ESHAPE, "ldw=%lld and ldi=%lld must be >= cin=%d", (long long)ldw, (long long)ldi, p.cin);
  if (p.cin > (1 << 20)) return fail(HINM_ESHAPE, "cin=%d exceeds the 2^20 supported by the permutation check", p.cin);
  if (!hinm::aligned(w_bf16, 2) || !hinm::aligned(importance, 4) || (perm && !hinm::aligned(perm, 4)))
    return fail(HINM_EALIGN, "w must be 2-byte, importance and perm 4-byte aligned");
  struct Buf { const void* ptr; int64_t bytes; const char* name; } bufs[5] = {
      {val_dense, p.bytes_val_dense, "val_dense"}, {idx_dense, p.bytes_idx_dense, "idx_dense"},
      {val_24, p.bytes_val_24, "val_24"}, {meta_24, p.bytes_meta_24, "meta_24"},
      {idx_24, p.bytes_idx_24, "idx_24"}};
  for (const Buf& b : bufs) {
    if (b.bytes > 0 && !b.ptr) return fail(HINM_EINVAL, "%s is NULL but needs %lld bytes", b.name, (long long)b.bytes);
    if (b.ptr && !hinm::aligned(b.ptr, 16)) return fail(HINM_EALIGN, "%s is not 16-byte aligned", b.name);
  }
  if (!workspace || workspace_bytes < need)
    return fail(HINM_EWORKSPACE, "pack workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  int st = hinm::ensure_device();
  if (st) return st;

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const int T = p.T, cin = p.cin, R = p.R;
  char* ws = static_cast<char*>(workspace);
  int* flag = reinterpret_cast<int*>(ws);
  double* scores = reinterpret_cast<double*>(ws + 256);
  uint8_t* reg = reinterpret_cast<uint8_t*>(ws + 256 + (size_t)T * cin * 8);
  const uint16_t* w = static_cast<const uint16_t*>(w_bf16);

  // Stage 1: validate perm and importance, compute the scores; read the flag.
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(64), 0, stream, flag);
  if (perm)
    hipLaunchKernelGGL(check_perm_kernel, dim3(T), dim3(1024), ((cin + 31) / 32) * 4, stream, perm, cin, flag);
  hipLaunchKernelGGL(scores_kernel, dim3((cin + 255) / 256, T), dim3(256), 0, stream, importance, ldi, cin, R,
                     scores, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pack stage-1 launch");
  int hflag = 0;
  e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "pack stage-1");
  if (hflag & kFlagPerm) return fail(HINM_EPERM, "a perm row is not a permutation of 0..%d", cin - 1);
  if (hflag & kFlagImportance) return fail(HINM_EIMPORTANCE, "importance has a negative or non-finite entry");
  if (packed_flags) *packed_flags = (hflag & kFlagNotBlock64) ? 0u : (uint32_t)HINM_PACKED_WINDOWED;

  // Stage 2: regions, index lists, values and metadata.
  hipLaunchKernelGGL(regions_kernel, dim3((cin + 255) / 256, T), dim3(256), 0, stream, scores, cin, p.n_dense,
                     p.n_24, reg, tiles);
  hipLaunchKernelGGL(compact_kernel, dim3(T), dim3(1024), 0, stream, perm, reg, cin, p.n_dense_pad, p.n_24_pad,
                     idx_dense, idx_24, tiles);
  if (p.n_24_pad > 0) {
    const int64_t n = (int64_t)T * (p.n_24_pad / 64) * R;
    hipLaunchKernelGGL(encode24_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, w, ldw, importance,
                       ldi, idx_24, cin, R, T, p.groups, p.n_24_pad, static_cast<uint16_t*>(val_24), meta_24, tiles);
  }
  if (p.n_dense_pad > 0) {
    const int64_t n = (int64_t)T * (p.n_dense_pad / 32) * R;
    hipLaunchKernelGGL(gather_dense_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, w, ldw,
                       idx_dense, cin, R, T, p.n_dense_pad, static_cast<uint16_t*>(val_dense), tiles);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pack stage-2 launch");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "pack stage-2");
  return HINM_OK;
}

namespace hinm {

// The checks, scores, regions and index lists of a pack (its first stages)
// into caller buffers, for entry points that need the lists without the
// values.  ws is laid out as the pack workspace; synchronous.
int region_lists(const hinm_plan_t& p, const float* importance, int64_t ldi, const int32_t* perm, int32_t* idx_dense,
                 int32_t* idx_24, void* ws_, hipStream_t stream) {
  const int T = p.n_tiles, cin = p.cin, R = p.tile_rows;
  char* ws = static_cast<char*>(ws_);
  int* flag = reinterpret_cast<int*>(ws);
  double* scores = reinterpret_cast<double*>(ws + 256);
  uint8_t* reg = reinterpret_cast<uint8_t*>(ws + 256 + (size_t)T * cin * 8);
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(64), 0, stream, flag);
  if (perm)
    hipLaunchKernelGGL(check_perm_kernel, dim3(T), dim3(1024), ((cin + 31) / 32) * 4, stream, perm, cin, flag);
  hipLaunchKernelGGL(scores_kernel, dim3((cin + 255) / 256, T), dim3(256), 0, stream, importance, ldi, cin, R,
                     scores, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "region lists launch");
  int hflag = 0;
  e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "region lists");
  if (hflag & kFlagPerm) return fail(HINM_EPERM, "a perm row is not a permutation of 0..%d", cin - 1);
  if (hflag & kFlagImportance) return fail(HINM_EIMPORTANCE, "importance has a negative or non-finite entry");
  hipLaunchKernelGGL(regions_kernel, dim3((cin + 255) / 256, T), dim3(256), 0, stream, scores, cin, p.n_dense,
                     p.n_24, reg, nullptr);
  hipLaunchKernelGGL(compact_kernel, dim3(T), dim3(1024), 0, stream, perm, reg, cin, p.n_dense_pad, p.n_24_pad,
                     idx_dense, idx_24, nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "region lists launch");
  return HINM_OK;
}

}  // namespace hinm

extern "C" int hinm_pack(const hinm_plan_t* plan, const void* w_bf16, int64_t ldw, const float* importance,
                         int64_t ldi, const int32_t* perm, hinm_packed_t* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  hinm::clear_error();
  int st = hinm::check_plan(plan);
  if (st) return st;
  if (!out) return fail(HINM_EINVAL, "out must be non-NULL");
  const hinm_plan_t& p = *plan;
  const PackShape ps = {p.n_tiles, p.cin, p.tile_rows, p.n_dense, p.n_24, p.n_dense_pad, p.n_24_pad, p.groups,
                        p.bytes_val_dense, p.bytes_idx_dense, p.bytes_val_24, p.bytes_meta_24, p.bytes_idx_24};
  size_t need = 0;
  hinm_pack_workspace_bytes(plan, &need);
  out->plan = p;
  out->flags = 0;
  out->reserved = 0;
  return pack_core(ps, nullptr, w_bf16, ldw, importance, ldi, perm, out->val_dense, out->idx_dense, out->val_24,
                   out->meta_24, out->idx_24, workspace, workspace_bytes, need, stream, &out->flags);
}

extern "C" int hinm_pack_tiles(const hinm_tplan_t* plan, const void* w_bf16, int64_t ldw, const float* importance,
                               int64_t ldi, const int32_t* perm, hinm_tpacked_t* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  hinm::clear_error();
  int st = hinm::check_tplan(plan);
  if (st) return st;
  if (!out) return fail(HINM_EINVAL, "out must be non-NULL");
  if (!out->tiles) return fail(HINM_EINVAL, "out->tiles (the device tile table) is NULL");
  if (!hinm::aligned(out->tiles, 4)) return fail(HINM_EALIGN, "out->tiles is not 4-byte aligned");
  const hinm_tplan_t& p = *plan;
  const PackShape ps = {p.n_tiles, p.cin, p.tile_rows, 0, 0, p.max_n_dense_pad, p.max_n_24_pad, 0,
                        p.bytes_val_dense, p.bytes_idx_dense, p.bytes_val_24, p.bytes_meta_24, p.bytes_idx_24};
  size_t need = 0;
  hinm_pack_tiles_workspace_bytes(plan, &need);
  out->plan = p;
  return pack_core(ps, out->tiles, w_bf16, ldw, importance, ldi, perm, out->val_dense, out->idx_dense, out->val_24,
                   out->meta_24, out->idx_24, workspace, workspace_bytes, need, stream);
}

extern "C" int hinm_translate_indices(hinm_packed_t* packed, const int32_t* map, void* workspace,
                                      size_t workspace_bytes, void* stream_) {
  hinm::clear_error();
  if (!packed || !map) return fail(HINM_EINVAL, "packed and map must be non-NULL");
  int st = hinm::check_plan(&packed->plan);
  if (st) return st;
  const hinm_plan_t& p = packed->plan;
  if (!hinm::aligned(map, 4)) return fail(HINM_EALIGN, "map is not 4-byte aligned");
  if ((p.bytes_idx_dense > 0 && !packed->idx_dense) || (p.bytes_idx_24 > 0 && !packed->idx_24))
    return fail(HINM_EINVAL, "index lists are NULL");
  if (!workspace || workspace_bytes < 256)
    return fail(HINM_EWORKSPACE, "translate workspace of %zu bytes given, 256 needed", workspace_bytes);
  if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  st = hinm::ensure_device();
  if (st) return st;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  int* flag = static_cast<int*>(workspace);
  // 1. map must be a permutation of 0..cin-1 (nothing is written otherwise)
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(64), 0, stream, flag);
  hipLaunchKernelGGL(check_perm_kernel, dim3(1), dim3(1024), ((p.cin + 31) / 32) * 4, stream, map, p.cin, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "translate check launch");
  int hflag = 0;
  e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "translate check");
  if (hflag & kFlagPerm) return fail(HINM_EPERM, "map is not a permutation of 0..%d", p.cin - 1);
  // 2. rewrite both index lists in place
  const int64_t nd = (int64_t)p.n_tiles * p.n_dense_pad, ns = (int64_t)p.n_tiles * p.n_24_pad;
  if (nd > 0)
    hipLaunchKernelGGL(translate_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, stream, packed->idx_dense,
                       nd, map);
  if (ns > 0)
    hipLaunchKernelGGL(translate_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream, packed->idx_24,
                       ns, map);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "translate launch");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "translate");
  // a map that moves a channel out of its block of 64 breaks the lists' window order
  if (hflag & kFlagNotBlock64) packed->flags &= ~(uint32_t)HINM_PACKED_WINDOWED;
  return HINM_OK;
}

extern "C" int hinm_boundary_workspace_bytes(int64_t cout, int64_t cin, int32_t tile_rows, size_t* bytes) {
  hinm::clear_error();
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  hinm_plan_t p;
  int st = hinm_plan(cout, cin, tile_rows, 0.5, 0.5, &p);
  if (st) return st;
  const size_t T = (size_t)p.n_tiles, C = (size_t)p.cin, R = (size_t)p.tile_rows;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t list = up(T * (C + 64) * 4);
  *bytes = 256 + up(T * C * 8) + up(T * C * 4) + up(T * C) + 2 * list + up((T + T * R) * 8);
  return HINM_OK;
}

// Shared by the global and the per-tile search.  Global: one v_s, R_total
// summed over all tiles.  Per tile (v_tiles != NULL): tile t follows the same
// rule on its own R_t(v) = R_dense(t) + sum over its rows of R_24, and the
// grid goes on while any tile is still rising.
static int boundary_core(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double step,
                         const float* importance, int64_t ldi, const int32_t* perm, void* workspace,
                         size_t workspace_bytes, double* v_s_out, double* trace_v, double* trace_r, int32_t trace_cap,
                         int32_t* trace_len, double* v_tiles, int32_t* points_tiles, void* stream_) {
  if (!importance) return fail(HINM_EINVAL, "importance must be non-NULL");
  if (!(step > 0.0) || !std::isfinite(step)) return fail(HINM_EINVAL, "step=%g must be a positive finite number", step);
  if (trace_cap < 0 || (trace_cap > 0 && (!trace_v || !trace_r))) return fail(HINM_EINVAL, "bad trace arguments");
  hinm_plan_t p0;
  int st = hinm_plan(cout, cin, tile_rows, t_s, t_s, &p0);
  if (st) return st;
  if (ldi < cin) return fail(HINM_ESHAPE, "ldi=%lld < cin=%lld", (long long)ldi, (long long)cin);
  if (!hinm::aligned(importance, 4) || (perm && !hinm::aligned(perm, 4)))
    return fail(HINM_EALIGN, "importance and perm must be 4-byte aligned");
  size_t need = 0;
  hinm_boundary_workspace_bytes(cout, cin, tile_rows, &need);
  if (!workspace || workspace_bytes < need)
    return fail(HINM_EWORKSPACE, "boundary workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  st = hinm::ensure_device();
  if (st) return st;

  const int T = p0.n_tiles, C = p0.cin, R = p0.tile_rows;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  char* ws = static_cast<char*>(workspace);
  int* flag = reinterpret_cast<int*>(ws);
  size_t off = 256;
  double* scores = reinterpret_cast<double*>(ws + off);  off += up((size_t)T * C * 8);
  int32_t* rank = reinterpret_cast<int32_t*>(ws + off);  off += up((size_t)T * C * 4);
  uint8_t* reg = reinterpret_cast<uint8_t*>(ws + off);   off += up((size_t)T * C);
  int32_t* idx_d = reinterpret_cast<int32_t*>(ws + off); off += up((size_t)T * (C + 64) * 4);
  int32_t* idx_s = reinterpret_cast<int32_t*>(ws + off); off += up((size_t)T * (C + 64) * 4);
  double* part = reinterpret_cast<double*>(ws + off);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);

  // checks and scores (as hinm_pack), then the ranking, once
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(64), 0, stream, flag);
  if (perm)
    hipLaunchKernelGGL(check_perm_kernel, dim3(T), dim3(1024), ((C + 31) / 32) * 4, stream, perm, C, flag);
  hipLaunchKernelGGL(scores_kernel, dim3((C + 255) / 256, T), dim3(256), 0, stream, importance, ldi, C, R, scores, flag);
  hipLaunchKernelGGL(rank_kernel, dim3((C + 255) / 256, T), dim3(256), 0, stream, scores, C, rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "boundary set-up launch");
  int hflag = 0;
  e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "boundary set-up");
  if (hflag & kFlagPerm) return fail(HINM_EPERM, "a perm row is not a permutation of 0..%d", C - 1);
  if (hflag & kFlagImportance) return fail(HINM_EIMPORTANCE, "importance has a negative or non-finite entry");

  // grid v = t_s - step*k, k = 0, 1, ..., down to max(0, 2 t_s - 1); stop at the first strict decrease
  const bool per_tile = v_tiles != nullptr;
  const double lo = std::max(0.0, 2.0 * t_s - 1.0);
  std::vector<double> hpart((size_t)T + (size_t)T * R);
  std::vector<double> best_v(per_tile ? T : 1, t_s), best_r(per_tile ? T : 1, 0.0);
  std::vector<int> have(per_tile ? T : 1, 0), active(per_tile ? T : 1, 1), points(per_tile ? T : 1, 0);
  int n_trace = 0, n_active = per_tile ? T : 1;
  for (int k = 0; n_active > 0; ++k) {
    double v = t_s - step * k;
    if (v < lo - 1e-12) break;
    v = std::max(v, lo);
    hinm_plan_t pv;
    st = hinm_plan(cout, cin, tile_rows, t_s, v, &pv);
    if (st) return st;
    const int64_t n = (int64_t)T * C;
    hipLaunchKernelGGL(cut_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, rank, n, pv.n_dense,
                       pv.n_24, reg);
    hipLaunchKernelGGL(compact_kernel, dim3(T), dim3(1024), 0, stream, perm, reg, C, pv.n_dense_pad, pv.n_24_pad,
                       idx_d, idx_s, nullptr);
    hipLaunchKernelGGL(rdense_kernel, dim3(T), dim3(256), 0, stream, scores, rank, C, pv.n_dense, part);
    if (pv.groups > 0)
      hipLaunchKernelGGL(r24_kernel, dim3(R, T), dim3(256), 0, stream, importance, ldi, idx_s, pv.n_24_pad, pv.groups,
                         R, part + T);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "boundary launch");
    const size_t nbytes = ((size_t)T + (pv.groups > 0 ? (size_t)T * R : 0)) * sizeof(double);
    e = hipMemcpyAsync(hpart.data(), part, nbytes, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "boundary step");
    // totals in a fixed order: per tile its dense sum, then its rows' 2:4 sums
    std::vector<double> r_tile(T);
    for (int t = 0; t < T; ++t) {
      double r = hpart[t];
      if (pv.groups > 0)
        for (int i = 0; i < R; ++i) r += hpart[T + (size_t)t * R + i];
      r_tile[t] = r;
    }
    auto visit = [&](int u, double r) {
      ++points[u];
      if (have[u] && r < best_r[u]) {
        active[u] = 0;
        --n_active;
        return;
      }
      best_v[u] = v;
      best_r[u] = r;
      have[u] = 1;
    };
    if (per_tile) {
      for (int t = 0; t < T; ++t)
        if (active[t]) visit(t, r_tile[t]);
    } else {
      double r_tot = 0.0;
      for (int t = 0; t < T; ++t) r_tot += hpart[t];
      if (pv.groups > 0)
        for (size_t i = 0; i < (size_t)T * R; ++i) r_tot += hpart[T + i];
      if (n_trace < trace_cap) {
        trace_v[n_trace] = v;
        trace_r[n_trace] = r_tot;
      }
      ++n_trace;
      visit(0, r_tot);
    }
  }
  for (size_t u = 0; u < best_v.size(); ++u) {
    hinm_plan_t pb;
    st = hinm_plan(cout, cin, tile_rows, t_s, best_v[u], &pb);
    if (st) return st;
    const double vs = (double)pb.n_pruned / (double)cin;
    if (per_tile) {
      v_tiles[u] = vs;
      if (points_tiles) points_tiles[u] = points[u];
    } else {
      *v_s_out = vs;
    }
  }
  if (trace_len) *trace_len = n_trace;
  return HINM_OK;
}

extern "C" int hinm_boundary_search(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double step,
                                    const float* importance, int64_t ldi, const int32_t* perm, void* workspace,
                                    size_t workspace_bytes, double* v_s_out, double* trace_v, double* trace_r,
                                    int32_t trace_cap, int32_t* trace_len, void* stream) {
  hinm::clear_error();
  if (!v_s_out) return fail(HINM_EINVAL, "v_s_out must be non-NULL");
  return boundary_core(cout, cin, tile_rows, t_s, step, importance, ldi, perm, workspace, workspace_bytes, v_s_out,
                       trace_v, trace_r, trace_cap, trace_len, nullptr, nullptr, stream);
}

extern "C" int hinm_boundary_search_tiles(int64_t cout, int64_t cin, int32_t tile_rows, double t_s, double step,
                                          const float* importance, int64_t ldi, const int32_t* perm,
                                          void* workspace, size_t workspace_bytes, double* v_s_tiles,
                                          int32_t* points_tiles, void* stream) {
  hinm::clear_error();
  if (!v_s_tiles) return fail(HINM_EINVAL, "v_s_tiles must be non-NULL");
  return boundary_core(cout, cin, tile_rows, t_s, step, importance, ldi, perm, workspace, workspace_bytes, nullptr,
                       nullptr, nullptr, 0, nullptr, v_s_tiles, points_tiles, stream);
}
