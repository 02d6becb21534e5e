// hinm_spmm: Y = (W (.) M) X for a packed HiNM weight on gfx950.
//
// One launch covers both region types of every tile (the FlexHiNM-GP notes,
// key design 4, use two CUDA streams and atomicAdd; here a workgroup runs the
// dense K-blocks on MFMA and the 2:4 K-blocks on the structured-sparse
// SMFMAC into the same fp32 accumulators, so no atomics are needed):
//   workgroup = (token block, tile x 64-row block, K split), 4 waves of 16 rows
//   per K-block: gather the block's X rows through the kept-vector indices
//   into LDS (transposed, k fastest), then
//     dense block (32 columns):  v_mfma_f32_16x16x32_bf16
//     2:4 block (64 positions):  v_smfmac_f32_16x16x64_bf16 with the packed
//                                values as the compressed A operand and the
//                                nibble metadata as its index operand
//   epilogue: fp32 -> bf16 (round to nearest even) into Y, or fp32 partial sums
//   into the workspace when the K dimension is split, followed by a
//   fixed-order reduction kernel (deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "hinm_internal.h"

using hinm::fail;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        // waves per workgroup, 16 rows each
constexpr int kRowsPerWg = 64;
constexpr int kLdsK = 72;        // LDS row pitch in bf16 (64 positions + 16 B pad)

struct SpmmArgs {
  const uint16_t* val_d;
  const int32_t* idx_d;
  const uint16_t* val_s;
  const uint64_t* meta;
  const int32_t* idx_s;
  const uint16_t* x;
  uint16_t* y;
  float* ws;
  int64_t ldx, ldy;
  int batch, batch_pad16;
  int cin, cout, rows;
  int nkb_d, nkb_s;          // K-blocks per tile in each region
  int n_rblocks, splits, n_kunits;
  int x_vec;                 // 1: 16-byte aligned X rows (ldx % 8 == 0)
};

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Copies the X rows of one K-block into LDS as xt[n][k] (k fastest): row
// idx[k] of X, tokens n0 .. n0+NT-1; -1 indices and tokens past the batch
// read as zero.
template <int NT, int K>
__device__ inline void gather_x(const SpmmArgs& a, const int32_t* __restrict__ idx, int n0, uint16_t* xt) {
  constexpr int kChunksPerRow = NT / 8;
  constexpr int kChunks = K * kChunksPerRow;
  for (int q = threadIdx.x; q < kChunks; q += kWaves * 64) {
    const int k = q / kChunksPerRow, u = q % kChunksPerRow;
    const int c = idx[k];
    const int nb = n0 + 8 * u;
    uint16_t v[8];
    if (c >= 0 && c < a.cin) {
      const uint16_t* src = a.x + (int64_t)c * a.ldx + nb;
      if (a.x_vec && nb + 8 <= a.batch) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src);
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = (uint16_t)(w[e] & 0xffffu);
          v[2 * e + 1] = (uint16_t)(w[e] >> 16);
        }
      } else {
        for (int e = 0; e < 8; ++e) v[e] = (nb + e < a.batch) ? src[e] : (uint16_t)0;
      }
    } else {
      for (int e = 0; e < 8; ++e) v[e] = 0;
    }
    for (int e = 0; e < 8; ++e) xt[(8 * u + e) * kLdsK + k] = v[e];
  }
}

template <int NT>
__global__ __launch_bounds__(kWaves * 64) void spmm_kernel(SpmmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xt[NT * kLdsK];
  constexpr int NB = NT / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * NT;
  const int t = blockIdx.y / a.n_rblocks, rb = blockIdx.y % a.n_rblocks;
  const int split = blockIdx.z;
  const int rrow = rb * kRowsPerWg + wave * 16;      // first tile row of this wave
  const bool active = rrow < a.rows;
  const int myrow = rrow + (lane & 15);
  const int kc = lane >> 4;                           // k chunk of this lane (0..3)

  // K units of this split: dense blocks first (1 unit each), then 2:4 blocks
  // (2 units each); a block belongs to the split holding its first unit.
  const int u_lo = (int)((int64_t)split * a.n_kunits / a.splits);
  const int u_hi = (int)((int64_t)(split + 1) * a.n_kunits / a.splits);

  f32x4 acc[NB];
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- dense region: 32-column blocks, MFMA 16x16x32 ----
  const int d_lo = min(u_lo, a.nkb_d), d_hi = min(u_hi, a.nkb_d);
  for (int kb = d_lo; kb < d_hi; ++kb) {
    gather_x<NT, 32>(a, a.idx_d + ((int64_t)t * a.nkb_d + kb) * 32, n0, xt);
    __syncthreads();
    if (active) {
      const uint16_t* ap = a.val_d + (((int64_t)t * a.nkb_d + kb) * a.rows + myrow) * 32 + 8 * kc;
      const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ap));
      for (int nb = 0; nb < NB; ++nb) {
        const uint16_t* bp = xt + (nb * 16 + (lane & 15)) * kLdsK + 8 * kc;
        const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bp));
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- 2:4 region: 64-position blocks, SMFMAC 16x16x64 ----
  // Lane (row, kc) holds the 8 kept values of groups 4kc..4kc+3 of its row
  // and their nibbles (metadata bits 16kc..16kc+15).  The B operand of lane
  // (token, kc) holds positions 8kc..8kc+7 and 32+8kc..32+8kc+7.
  for (int u = max(u_lo, a.nkb_d); u < u_hi; ++u) {
    if ((u - a.nkb_d) & 1) continue;                  // second unit of a 2:4 block
    const int kb = (u - a.nkb_d) >> 1;
    gather_x<NT, 64>(a, a.idx_s + ((int64_t)t * a.nkb_s + kb) * 64, n0, xt);
    __syncthreads();
    if (active) {
      const int64_t blk = ((int64_t)t * a.nkb_s + kb) * a.rows + myrow;
      const uint16_t* ap = a.val_s + blk * 32 + 8 * kc;
      const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ap));
      const int sidx = (int)((a.meta[blk] >> (16 * kc)) & 0xffffull);
      for (int nb = 0; nb < NB; ++nb) {
        const uint16_t* bp = xt + (nb * 16 + (lane & 15)) * kLdsK;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(bp + 8 * kc);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(bp + 32 + 8 * kc);
        const bf16x16 bv = __builtin_bit_cast(bf16x16, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, acc[nb], sidx, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!active) return;
  // Accumulator lane layout: acc[nb][i] is row 4*kc + i of the wave, token nb*16 + lane%16.
  const int64_t grow0 = (int64_t)t * a.rows + rrow + 4 * kc;
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + nb * 16 + (lane & 15);
    if (a.splits == 1) {
      if (n < a.batch)
        for (int i = 0; i < 4; ++i) a.y[(grow0 + i) * a.ldy + n] = bf16_rne(acc[nb][i]);
    } else if (n < a.batch_pad16) {
      float* dst = a.ws + ((int64_t)split * a.cout + grow0) * a.batch_pad16 + n;
      for (int i = 0; i < 4; ++i) dst[(int64_t)i * a.batch_pad16] = acc[nb][i];
    }
  }
}

// Sum of the split partials in split order, then bf16 into Y.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ ws, int splits, int cout, int batch,
                                                     int batch_pad16, uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)cout * batch) return;
  const int64_t row = i / batch;
  const int n = (int)(i % batch);
  const int64_t plane = (int64_t)cout * batch_pad16;
  const float* src = ws + row * batch_pad16 + n;
  float acc = 0.f;
  for (int s = 0; s < splits; ++s) acc += src[s * plane];
  y[row * ldy + n] = bf16_rne(acc);
}

}  // namespace

namespace hinm {

int ensure_device() {
  static int checked[64];  // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HINM_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(HINM_EDEVICE, "device ordinal %d out of range", dev);
  if (checked[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(HINM_EDEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    checked[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (checked[dev] == 2) return fail(HINM_EDEVICE, "device %d is %s, libhinm is built for gfx950", dev, prop.gcnArchName);
  }
  return checked[dev] == 1 ? HINM_OK : fail(HINM_EDEVICE, "device %d is not gfx950", dev);
}

}  // namespace hinm

extern "C" int hinm_spmm(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx, void* y_bf16,
                         int64_t ldy, void* workspace, size_t workspace_bytes, void* stream_) {
  hinm::clear_error();
  if (!packed) return fail(HINM_EINVAL, "packed is NULL");
  int st = hinm::check_plan(&packed->plan);
  if (st) return st;
  const hinm_plan_t& p = packed->plan;
  if (batch < 0) return fail(HINM_ESHAPE, "batch=%lld is negative", (long long)batch);
  if (batch > (1 << 24)) return fail(HINM_ESHAPE, "batch=%lld exceeds 2^24", (long long)batch);
  if (ldx < batch || ldy < batch)
    return fail(HINM_ESHAPE, "ldx=%lld and ldy=%lld must be >= batch=%lld", (long long)ldx, (long long)ldy,
                (long long)batch);
  if (batch == 0) return HINM_OK;
  if (!x_bf16 || !y_bf16) return fail(HINM_EINVAL, "x and y must be non-NULL");
  if (!hinm::aligned(x_bf16, 2) || !hinm::aligned(y_bf16, 2)) return fail(HINM_EALIGN, "x and y must be 2-byte aligned");
  struct Buf { const void* ptr; int64_t bytes; const char* name; } bufs[5] = {
      {packed->val_dense, p.bytes_val_dense, "val_dense"}, {packed->idx_dense, p.bytes_idx_dense, "idx_dense"},
      {packed->val_24, p.bytes_val_24, "val_24"}, {packed->meta_24, p.bytes_meta_24, "meta_24"},
      {packed->idx_24, p.bytes_idx_24, "idx_24"}};
  for (const Buf& b : bufs) {
    if (b.bytes > 0 && !b.ptr) return fail(HINM_EINVAL, "%s is NULL but holds %lld bytes", b.name, (long long)b.bytes);
    if (b.ptr && !hinm::aligned(b.ptr, 16)) return fail(HINM_EALIGN, "%s is not 16-byte aligned", b.name);
  }
  const hinm::SpmmShape sh = hinm::spmm_shape(&p, batch);
  if (sh.ws_bytes > 0) {
    if (!workspace || workspace_bytes < (size_t)sh.ws_bytes)
      return fail(HINM_EWORKSPACE, "spmm workspace of %zu bytes given, %lld needed", workspace_bytes,
                  (long long)sh.ws_bytes);
    if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  }
  st = hinm::ensure_device();
  if (st) return st;
  if ((int64_t)p.n_tiles * sh.n_rblocks > 65535) return fail(HINM_ESHAPE, "too many row blocks for one launch");

  SpmmArgs a;
  a.val_d = static_cast<const uint16_t*>(packed->val_dense);
  a.idx_d = packed->idx_dense;
  a.val_s = static_cast<const uint16_t*>(packed->val_24);
  a.meta = packed->meta_24;
  a.idx_s = packed->idx_24;
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.y = static_cast<uint16_t*>(y_bf16);
  a.ws = static_cast<float*>(workspace);
  a.ldx = ldx;
  a.ldy = ldy;
  a.batch = (int)batch;
  a.batch_pad16 = (int)((batch + 15) / 16 * 16);
  a.cin = p.cin;
  a.cout = p.cout;
  a.rows = p.tile_rows;
  a.nkb_d = p.n_dense_pad / HINM_KB_DENSE;
  a.nkb_s = p.n_24_pad / HINM_KB_24;
  a.n_rblocks = sh.n_rblocks;
  a.splits = sh.splits;
  a.n_kunits = sh.n_kunits;
  a.x_vec = hinm::aligned(x_bf16, 16) && (ldx % 8 == 0);

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const dim3 grid(sh.n_tblocks, p.n_tiles * sh.n_rblocks, sh.splits), block(kWaves * 64);
  switch (sh.nt) {
    case 16: hipLaunchKernelGGL(spmm_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(spmm_kernel<32>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(spmm_kernel<64>, grid, block, 0, stream, a); break;
  }
  if (sh.splits > 1) {
    const int64_t n = (int64_t)p.cout * batch;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.ws, sh.splits, p.cout,
                       (int)batch, a.batch_pad16, a.y, ldy);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HINM_EHIP, "spmm launch: %s", hipGetErrorString(e));
  return HINM_OK;
}
