// hinm_pack: vector scoring, region ranking, permuted index lists, 2:4 top-2
// selection with 2-bit metadata, and the dense-region value gather, for
// gfx950.  A one-time transform of a weight; written for exactness (bit
// identical to the definition) more than speed, but every kernel is a plain
// data-parallel pass with coalesced stores.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "hinm_internal.h"

using hinm::fail;

namespace {

constexpr uint8_t kPruned = 0, kTwoFour = 1, kDense = 2;
constexpr int kFlagPerm = 1, kFlagImportance = 2;

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
  bool bad = false;
  for (int j = threadIdx.x; j < cin; j += blockDim.x) {
    const int c = row[j];
    if (c < 0 || c >= cin) {
      bad = true;
      continue;
    }
    const uint32_t m = 1u << (c & 31);
    if (atomicOr(&seen[c >> 5], m) & m) bad = true;
  }
  if (bad) atomicOr(flag, kFlagPerm);
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
                                                      int n_24, uint8_t* __restrict__ reg) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
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
                                                       int32_t* __restrict__ idx_d, int32_t* __restrict__ idx_s) {
  __shared__ int wd[16], ws[16];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int32_t* od = idx_d + (int64_t)t * n_dense_pad;
  int32_t* os = idx_s + (int64_t)t * n_24_pad;
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
                                                       uint16_t* __restrict__ val_s, uint64_t* __restrict__ meta) {
  const int nkb = n_24_pad / 64;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tiles * nkb * rows) return;
  const int r = (int)(gid % rows);
  const int64_t tk = gid / rows;
  const int kb = (int)(tk % nkb);
  const int t = (int)(tk / nkb);
  const int64_t grow = (int64_t)t * rows + r;
  const int32_t* il = idx_s + (int64_t)t * n_24_pad + kb * 64;
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
  uint4* dst = reinterpret_cast<uint4*>(val_s + ((int64_t)(t * nkb + kb) * rows + r) * 32);
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  meta[(int64_t)(t * nkb + kb) * rows + r] = m;
}

// Dense-region gather: val_d[t][kb][r][k] = W[t*R + r][idx_d[t][32 kb + k]].
__global__ __launch_bounds__(256) void gather_dense_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                           const int32_t* __restrict__ idx_d, int cin, int rows,
                                                           int n_tiles, int n_dense_pad, uint16_t* __restrict__ val_d) {
  const int nkb = n_dense_pad / 32;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n_tiles * nkb * rows) return;
  const int r = (int)(gid % rows);
  const int64_t tk = gid / rows;
  const int kb = (int)(tk % nkb);
  const int t = (int)(tk / nkb);
  const int64_t grow = (int64_t)t * rows + r;
  const int32_t* il = idx_d + (int64_t)t * n_dense_pad + kb * 32;
  uint32_t packed[16];
  for (int k = 0; k < 32; k += 2) {
    const int c0 = il[k], c1 = il[k + 1];
    const uint32_t v0 = (c0 >= 0 && c0 < cin) ? w[grow * ldw + c0] : 0u;
    const uint32_t v1 = (c1 >= 0 && c1 < cin) ? w[grow * ldw + c1] : 0u;
    packed[k / 2] = v0 | (v1 << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(val_d + ((int64_t)(t * nkb + kb) * rows + r) * 32);
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

}  // namespace

extern "C" int hinm_pack(const hinm_plan_t* plan, const void* w_bf16, int64_t ldw, const float* importance,
                         int64_t ldi, const int32_t* perm, hinm_packed_t* out, void* workspace,
                         size_t workspace_bytes, void* stream_) {
  hinm::clear_error();
  int st = hinm::check_plan(plan);
  if (st) return st;
  const hinm_plan_t& p = *plan;
  if (!w_bf16 || !importance || !out) return fail(HINM_EINVAL, "w, importance and out must be non-NULL");
  if (ldw < p.cin || ldi < p.cin)
    return fail(HINM_ESHAPE, "ldw=%lld and ldi=%lld must be >= cin=%d", (long long)ldw, (long long)ldi, p.cin);
  if (p.cin > (1 << 20)) return fail(HINM_ESHAPE, "cin=%d exceeds the 2^20 supported by the permutation check", p.cin);
  if (!hinm::aligned(w_bf16, 2) || !hinm::aligned(importance, 4) || (perm && !hinm::aligned(perm, 4)))
    return fail(HINM_EALIGN, "w must be 2-byte, importance and perm 4-byte aligned");
  struct Buf { const void* ptr; int64_t bytes; const char* name; } bufs[5] = {
      {out->val_dense, p.bytes_val_dense, "val_dense"}, {out->idx_dense, p.bytes_idx_dense, "idx_dense"},
      {out->val_24, p.bytes_val_24, "val_24"}, {out->meta_24, p.bytes_meta_24, "meta_24"},
      {out->idx_24, p.bytes_idx_24, "idx_24"}};
  for (const Buf& b : bufs) {
    if (b.bytes > 0 && !b.ptr) return fail(HINM_EINVAL, "%s is NULL but needs %lld bytes", b.name, (long long)b.bytes);
    if (b.ptr && !hinm::aligned(b.ptr, 16)) return fail(HINM_EALIGN, "%s is not 16-byte aligned", b.name);
  }
  size_t need = 0;
  hinm_pack_workspace_bytes(plan, &need);
  if (!workspace || workspace_bytes < need)
    return fail(HINM_EWORKSPACE, "pack workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  st = hinm::ensure_device();
  if (st) return st;

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  out->plan = p;
  const int T = p.n_tiles, cin = p.cin, R = p.tile_rows;
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

  // Stage 2: regions, index lists, values and metadata.
  hipLaunchKernelGGL(regions_kernel, dim3((cin + 255) / 256, T), dim3(256), 0, stream, scores, cin, p.n_dense,
                     p.n_24, reg);
  hipLaunchKernelGGL(compact_kernel, dim3(T), dim3(1024), 0, stream, perm, reg, cin, p.n_dense_pad, p.n_24_pad,
                     out->idx_dense, out->idx_24);
  if (p.n_24_pad > 0) {
    const int64_t n = (int64_t)T * (p.n_24_pad / 64) * R;
    hipLaunchKernelGGL(encode24_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, w, ldw, importance,
                       ldi, out->idx_24, cin, R, T, p.groups, p.n_24_pad, static_cast<uint16_t*>(out->val_24),
                       out->meta_24);
  }
  if (p.n_dense_pad > 0) {
    const int64_t n = (int64_t)T * (p.n_dense_pad / 32) * R;
    hipLaunchKernelGGL(gather_dense_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, w, ldw,
                       out->idx_dense, cin, R, T, p.n_dense_pad, static_cast<uint16_t*>(out->val_dense));
  }
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pack stage-2 launch");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "pack stage-2");
  return HINM_OK;
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
  return HINM_OK;
}
