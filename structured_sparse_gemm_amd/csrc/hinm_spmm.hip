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

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

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
  int y_vec;                 // 1: 16-byte aligned Y rows (ldy % 8 == 0)
  int x_lds;                 // 1: the batch > 64 kernel loads X rows straight into LDS (256-token blocks)
  int n_tiles;
  const int32_t* out_rows;   // NULL, or the Y row of each product row
  const int32_t* tiles;      // NULL (uniform counts), or [n_tiles][4]: first dense block, n_dense,
                             // first 2:4 block, n_24 of each tile
  int kd_total, ks_total;    // dense and 2:4 K-blocks over all tiles
  int part_rows;             // rows of a split reduction's partial-sum planes (all weights of a group)
  int tb_group;              // batch > 64 kernel: token blocks per group of its item order (>= 1)
  int stagger;               // batch > 64 kernel: tile t starts its K loops at block t * n / n_tiles
};

// Several packed weights multiplied by one X in one launch (hinm_spmm_group):
// the weights' tile row blocks are numbered one after another, and a
// workgroup (split decode) or work item (prefill) takes the fields of the
// weight its row block belongs to.
constexpr int kMaxSeg = 8;
struct Seg {
  const uint16_t* val_d;
  const int32_t* idx_d;
  const uint16_t* val_s;
  const uint64_t* meta;
  const int32_t* idx_s;
  uint16_t* y;
  int64_t ldy;
  int cout, n_tiles, nkb_d, nkb_s, kd_total, ks_total;
  int trb0;                  // first row block of this weight in the concatenation
  int row0;                  // first row of this weight in the partial-sum planes
};
struct Segs {
  int n;                     // 0 or 1: one weight, the fields of SpmmArgs
  Seg s[kMaxSeg];
};

// Weight g of a group: patches a's per-weight fields and returns the first
// row block and row of that weight.  select_seg finds the weight of
// concatenated row block gtrb by a scan of the table.
__device__ inline void seg_fields(const Segs& segs, int g, SpmmArgs& a, int& trb0, int& row0) {
  const Seg& S = segs.s[g];
  a.val_d = S.val_d;
  a.idx_d = S.idx_d;
  a.val_s = S.val_s;
  a.meta = S.meta;
  a.idx_s = S.idx_s;
  a.y = S.y;
  a.ldy = S.ldy;
  a.cout = S.cout;
  a.n_tiles = S.n_tiles;
  a.nkb_d = S.nkb_d;
  a.nkb_s = S.nkb_s;
  a.kd_total = S.kd_total;
  a.ks_total = S.ks_total;
  trb0 = S.trb0;
  row0 = S.row0;
}
__device__ inline void select_seg(const Segs& segs, int gtrb, SpmmArgs& a, int& trb0, int& row0) {
  trb0 = 0;
  row0 = 0;
  if (segs.n <= 1) return;
  int g = 0;
  for (int k = 1; k < segs.n; ++k) g = gtrb >= segs.s[k].trb0 ? k : g;
  seg_fields(segs, g, a, trb0, row0);
}

// Tile t's K-blocks: first dense block and count, first 2:4 block and count.
struct TileK {
  int kd0, nbd, ks0, nbs;
};
__device__ inline TileK tile_k(const SpmmArgs& a, int t) {
  if (a.tiles)
    return {a.tiles[4 * t], (a.tiles[4 * t + 1] + 31) / 32, a.tiles[4 * t + 2], (a.tiles[4 * t + 3] + 63) / 64};
  return {t * a.nkb_d, a.nkb_d, t * a.nkb_s, a.nkb_s};
}

// Y row that product row r goes to: r itself, or out_rows[r]; -1 for an
// out-of-range entry (the row is then not written).
__device__ inline int64_t y_row(const SpmmArgs& a, int64_t r) {
  if (!a.out_rows) return r;
  const int64_t d = a.out_rows[r];
  return (d >= 0 && d < a.cout) ? d : -1;
}

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Split-K hand-over: one workgroup of `splits` counts itself in on an
// agent-scope counter; true for the last to arrive.  The increment wraps (the
// hardware's atomic inc: old >= splits - 1 stores 0), so the counter is back
// at 0 after the last arrival without a separate store.
//
// Why the partial sums are visible to the last arriver without a cache
// writeback (gfx950 follows the gfx942 memory model of the LLVM AMDGPU
// back end): the partials are written and read only with agent-scope atomic
// stores and loads, which are issued with the sc1 bit and so are coherent
// across the XCDs' L2 caches (a store writes through to the device-coherent
// level, a load reads from it).  Each workgroup waits for its partial stores
// to be acknowledged (s_waitcnt vmcnt(0)) before its increment, and the last
// arriver issues its partial loads only after its increment has returned.
// A release / acquire pair would add an L2 writeback and invalidate, which
// are needed only for data written with ordinary stores; none is read here.
__device__ inline bool arrive(unsigned* ctr, int splits) {
  return __builtin_amdgcn_atomic_inc32(ctr, (unsigned)(splits - 1), __ATOMIC_RELAXED, "agent") ==
         (unsigned)(splits - 1);
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
        for (int i = 0; i < 4; ++i) {
          const int64_t yr = y_row(a, grow0 + i);
          if (yr >= 0) a.y[yr * a.ldy + n] = bf16_rne(acc[nb][i]);
        }
    } else if (n < a.batch_pad16) {
      float* dst = a.ws + ((int64_t)split * a.cout + grow0) * a.batch_pad16 + n;
      for (int i = 0; i < 4; ++i) dst[(int64_t)i * a.batch_pad16] = acc[nb][i];
    }
  }
}

// Sum of the split partials in split order, then bf16 into Y.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ ws, int splits, int cout, int batch,
                                                     int batch_pad16, uint16_t* __restrict__ y, int64_t ldy,
                                                     const int32_t* __restrict__ out_rows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)cout * batch) return;
  const int64_t row = i / batch;
  const int n = (int)(i % batch);
  const int64_t plane = (int64_t)cout * batch_pad16;
  const float* src = ws + row * batch_pad16 + n;
  float acc = 0.f;
  for (int s = 0; s < splits; ++s) acc += src[s * plane];
  const int64_t yr = out_rows ? (int64_t)out_rows[row] : row;
  if (yr >= 0 && yr < cout) y[yr * ldy + n] = bf16_rne(acc);
}

// ---------------------------------------------------------------------------
// Shared pieces of the decode and prefill kernels.
//
// X tiles sit in LDS row-major (one row per gathered X row, tokens
// contiguous), exactly as the gather reads them.  The MFMA B operand needs
// several K positions of one token per lane; ds_read_b64_tr_b16 supplies that
// transposition: within each 16-lane group, output lane j receives element
// j%4 of the 8-byte row segment addressed by lane 4q + j/4, for q = 0..3.
// So lane (i) of a group addresses LDS row "position(4r + i/4)" at token
// column base + 4*(i%4) to deliver slots 4r..4r+3 of its B operand.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline v4i16 tr_read(const uint16_t* lds_elem) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) char*)((__attribute__((address_space(3))) uint16_t*)lds_elem)));
}

// Loads 16 bytes (8 tokens) of X row c starting at token nb; zeros past the
// batch, for a -1 index, or when nb is past the batch.
__device__ inline u32x4 load_x_chunk(const SpmmArgs& a, int c, int nb) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (c < 0 || c >= a.cin || nb >= a.batch) return v;
  const uint16_t* src = a.x + (int64_t)c * a.ldx + nb;
  if (a.x_vec && nb + 8 <= a.batch) return *reinterpret_cast<const u32x4*>(src);
  uint32_t h[8];
  for (int e = 0; e < 8; ++e) h[e] = (nb + e < a.batch) ? (uint32_t)src[e] : 0u;
  v[0] = h[0] | (h[1] << 16);
  v[1] = h[2] | (h[3] << 16);
  v[2] = h[4] | (h[5] << 16);
  v[3] = h[6] | (h[7] << 16);
  return v;
}

// Loads 16 bytes (8 tokens) of X row c at token nb with no branches: the
// caller guarantees 16-byte aligned rows and nb + 8 <= batch; a pad index
// reads row 0 and the chunk is replaced by zeros.
__device__ inline u32x4 load_x_chunk_fast(const SpmmArgs& a, int c, int nb) {
  const bool ok = (c >= 0) & (c < a.cin);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.x + (int64_t)(ok ? c : 0) * a.ldx + nb);
  return ok ? v : u32x4{0u, 0u, 0u, 0u};
}

constexpr int kDecWaves = 8;

// ---------------------------------------------------------------------------
// Decode kernel, all loads up front (small batches).
// At decode sizes every compute unit's share of the packed weight is only a
// few latency-bandwidth products, so each wave issues the loads of up to CH
// of its K-blocks at once - packed values, metadata and index slices first,
// then the X rows those indices name - and only then multiplies them.  A
// block of either region occupies the same registers and issues the same
// loads (a dense block repeats its 32 indices into the second half), which
// keeps the code straight-line.  Workgroup = 16 rows of one tile x NTOK
// tokens, 8 waves over the tile's blocks round-robin; the 8 partial sums are
// added in wave order through LDS.
// ---------------------------------------------------------------------------
template <int NTOK, int CH, bool FAST>
__global__ __launch_bounds__(kDecWaves * 64) void decode3_kernel(SpmmArgs a) {
  constexpr int CPR = NTOK / 8;               // 16-byte chunks per X row
  constexpr int SLOT = 64 * NTOK;
  constexpr int NB = NTOK / 16;
  __shared__ __attribute__((aligned(16))) uint16_t xsh[kDecWaves * SLOT];
  __shared__ float red[kDecWaves * 16 * NTOK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrb = a.rows / 16;
  const int t = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int n0 = blockIdx.y * NTOK;
  const int row = rb * 16 + (lane & 15);
  const int kc = lane >> 4, i16 = lane & 15;
  const int nblk = a.nkb_d + a.nkb_s;
  const int cnt = wave < nblk ? (nblk - wave + kDecWaves - 1) / kDecWaves : 0;
  uint16_t* xs = xsh + wave * SLOT;

  f32x4 acc[NB];
  for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < cnt; c0 += CH) {
    u32x4 A[CH];
    uint64_t M[CH];
    int I[CH][CPR];
    u32x4 X[CH][CPR];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int b = wave + kDecWaves * min(c0 + j, cnt - 1);
      const bool dense = b < a.nkb_d;
      const int kb = dense ? b : b - a.nkb_d;
      const int64_t blk = ((int64_t)t * (dense ? a.nkb_d : a.nkb_s) + kb) * a.rows + row;
      const uint16_t* vp = (dense ? a.val_d : a.val_s) + blk * 32 + 8 * kc;
      A[j] = *reinterpret_cast<const u32x4*>(vp);
      M[j] = dense ? *reinterpret_cast<const uint64_t*>(vp) : a.meta[blk];
      const int32_t* il = dense ? a.idx_d + ((int64_t)t * a.nkb_d + kb) * 32 : a.idx_s + ((int64_t)t * a.nkb_s + kb) * 64;
      for (int k = 0; k < CPR; ++k) {
        const int pos = (lane + 64 * k) / CPR;
        I[j][k] = il[dense ? (pos & 31) : pos];
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      for (int k = 0; k < CPR; ++k) {
        const int nb = n0 + 8 * ((lane + 64 * k) % CPR);
        X[j][k] = FAST ? load_x_chunk_fast(a, I[j][k], nb) : load_x_chunk(a, I[j][k], nb);
      }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (c0 + j < cnt) {
        const int b = wave + kDecWaves * (c0 + j);
        for (int k = 0; k < CPR; ++k) *reinterpret_cast<u32x4*>(xs + 8 * (lane + 64 * k)) = X[j][k];
        const bf16x8 Av = __builtin_bit_cast(bf16x8, A[j]);
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* base = xs + 16 * nb + 4 * (i16 & 3);
          const v4i16 b0 = tr_read(base + (8 * kc + 0 + (i16 >> 2)) * NTOK);
          const v4i16 b1 = tr_read(base + (8 * kc + 4 + (i16 >> 2)) * NTOK);
          if (b < a.nkb_d) {
            const bf16x8 B = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, B, acc[nb], 0, 0, 0);
          } else {
            const v4i16 b2 = tr_read(base + (32 + 8 * kc + 0 + (i16 >> 2)) * NTOK);
            const v4i16 b3 = tr_read(base + (32 + 8 * kc + 4 + (i16 >> 2)) * NTOK);
            const bf16x16 B = __builtin_bit_cast(
                bf16x16, __builtin_shufflevector(__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                 __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2,
                                                 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
            acc[nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(Av, B, acc[nb],
                                                                (int)((M[j] >> (16 * kc)) & 0xffffull), 0, 0);
          }
        }
      }
    }
  }

  // fixed-order sum over the waves, bf16 out; acc[nb][e] is row 4*kc + e, token 16*nb + i16.
  for (int nb = 0; nb < NB; ++nb)
    for (int e = 0; e < 4; ++e) red[(wave * 16 + 4 * kc + e) * NTOK + 16 * nb + i16] = acc[nb][e];
  __syncthreads();
  for (int o = threadIdx.x; o < 16 * NTOK; o += kDecWaves * 64) {
    const int r = o / NTOK, n = o % NTOK;
    float sum = 0.f;
    for (int w = 0; w < kDecWaves; ++w) sum += red[w * 16 * NTOK + o];
    const int64_t yr = y_row(a, (int64_t)t * a.rows + rb * 16 + r);
    if (n0 + n < a.batch && yr >= 0) a.y[yr * a.ldy + n0 + n] = bf16_rne(sum);
  }
}

// Buffer resources (raw buffers, 32-bit offsets; an offset past the end
// reads zero).
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
constexpr uint32_t kOob = 0xFFFFFFF0u;     // offset past every buffer: loads return zeros

struct BufRes {
  __amdgpu_buffer_rsrc_t x, vd, vs, meta, id, is;
  uint32_t ldx_bytes;
};


// ---------------------------------------------------------------------------
// Decode kernel with split K and specialised waves (batch <= 64, tile_rows %
// 64 == 0).  Workgroup = 64 rows of one tile x NTOK tokens x one K range;
// waves 0-3 own 16 rows each, the others (2 at 16 tokens, 4 at 32 and 64)
// gather X.  The index -> X-row chain is the latency-critical part, so the
// gather waves issue it first and the row waves send only a few
// packed-value loads ahead of it; once the X loads are on their way (one
// barrier) the row waves keep a fixed number of blocks in flight ahead of
// their multiplies.  The two roles sit in different waves, so the X rows
// never wait behind the packed values in a wave's in-order load queue.  A K
// range longer than one LDS round is processed in rounds, each role issuing
// the next round's loads as soon as its registers are free.
//
// Every block, dense or 2:4, takes 64 LDS positions and one
// v_smfmac_f32_16x16x64_bf16: a dense block's 32 columns sit at positions
// 4q and 4q+1 of its groups (column 2q+e at position 4q+e; positions 4q+2
// and 4q+3 hold zeros) and use the fixed index pattern 0x4 (positions 0 and
// 1 of every group), which is exactly the dense product because the A
// operand of a dense block is its 32 values in order.  The multiply loop is
// then the same straight-line code for every block: blocks past the K range
// get zero values and zero X rows, and blocks alternate between two
// accumulators so consecutive SMFMACs do not wait on each other.
// ---------------------------------------------------------------------------
// LDS layout of the gathered X rows in the split decode kernel: position p
// holds its NB = NTOK/16 groups of 16 tokens as 32-byte granules, granule g
// at granule index xs_gran<NB>(p, g) (a bijection on every 64 positions).
// One ds_read_b64_tr_b16 of a B operand reads granule nb of the 16
// positions 8*kc + q + i (kc 0..3, i 0..3, q 0 or 4, plus 32 for the upper
// half); in the plain layout those land on half of the 64 banks (a quarter
// at NB = 4), so each half-wave took 2 to 4 passes.  The swizzle spreads
// each half-wave over all 64 banks.
template <int NB>
__device__ inline int xs_gran(int p, int g) {
  if constexpr (NB == 1) return p ^ (((p >> 3) & 1) << 2);
  else if constexpr (NB == 2) return 2 * p + (g ^ ((p >> 3) & 1));
  else return 4 * p + (g ^ (((p >> 1) & 1) | (((p >> 3) & 1) << 1)));
}

// Workgroup bid of a split decode -> its row block, K split and the number
// of splits of that row block: the first r1 row blocks have `splits`
// workgroups each, the others twice as many.
struct WgSplit {
  int gtrb, split, nsp;
};
__device__ inline WgSplit wg_split(int bid, int splits, int r1) {
  const int nlo = r1 * splits;
  if (bid < nlo) return {bid / splits, bid % splits, splits};
  const int q = bid - nlo, n2 = 2 * splits;
  return {r1 + q / n2, q % n2, n2};
}

// The split decode's body, shared by its one-weight and group kernels
// below.  k_* are the arguments its first loads depend on (index lists,
// their block totals, per-tile counts, the tile table) for one weight; a
// group (GROUP) takes them from weight k_seg of its segment table instead.
template <int NTOK, int MAXB, bool FAST, int NG, bool ONE, bool GROUP>
__device__ __attribute__((always_inline)) inline void decode5_body(
    const int32_t* __restrict__ k_idx_d, const int32_t* __restrict__ k_idx_s, const int32_t* __restrict__ k_tiles,
    int k_kd_total, int k_ks_total, int k_nkb_d, int k_nkb_s, int k_rows, int k_splits, int k_r1, int k_seg,
    const SpmmArgs& a0,
    const Segs* segs, int n_tb, float* __restrict__ part, unsigned* __restrict__ counters) {
  constexpr int CPR = NTOK / 8;                // 16-byte chunks per X row
  constexpr int MAXP = MAXB * 64;              // LDS positions per round
  constexpr int GT = 64 * NG;                  // gather threads (NG gather waves)
  static_assert(GT / CPR <= 64, "a gather step covers at most one block's positions per lane group");
  constexpr int MAXCH = MAXP * CPR / GT;       // X chunks per gather thread per round
  constexpr int NB = NTOK / 16;
  // Packed-value blocks in flight ahead of the multiplies, and how many of
  // them go out before the first X gathers: (4, 8) at 16 tokens, (2, 6) at
  // 32 and 64, where each gathered X row is a larger share of the load
  // queue (swept: 1.5-3.5% faster than (4, 8) at 48-64 tokens; wider
  // windows were slower).
  constexpr int DPF_ = NTOK == 16 ? 8 : 6;
  constexpr int DPF = MAXB < DPF_ ? MAXB : DPF_;
  constexpr int P0_ = NTOK == 16 ? 4 : 2;
  constexpr int P0 = DPF < P0_ ? DPF : P0_;
  __shared__ __attribute__((aligned(16))) uint16_t xs[MAXP * NTOK];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool gather = wave >= 4;
  const int kc = lane >> 4, i16 = lane & 15;
  const int nrb = k_rows / 64;
  const WgSplit ws = wg_split(blockIdx.x, k_splits, k_r1);
  const int split = ws.split;
  const int splits = ws.nsp;                     // K splits of this row block
  const int gtrb = ws.gtrb;                      // row block over all weights of a group
  SpmmArgs a = a0;
  int trb0 = 0, row0 = 0;                        // this weight's first row block and partial-sum row
  if constexpr (GROUP) seg_fields(*segs, k_seg, a, trb0, row0);
  const int trb = gtrb - trb0;                   // tile * nrb + row block
  const int t = trb / nrb, rb = trb % nrb;
  const int tb = blockIdx.y;
  const int n0 = tb * NTOK;
  const int row = rb * 64 + (wave & 3) * 16 + (lane & 15);   // tile row of this lane's A fragment
  TileK tk;
  if constexpr (GROUP) {
    tk = tile_k(a, t);
  } else if (k_tiles) {
    tk = {k_tiles[4 * t], (k_tiles[4 * t + 1] + 31) / 32, k_tiles[4 * t + 2], (k_tiles[4 * t + 3] + 63) / 64};
  } else {
    tk = {t * k_nkb_d, k_nkb_d, t * k_nkb_s, k_nkb_s};
  }
  const int nblk = tk.nbd + tk.nbs;
  // 32-bit: at most 64 splits of at most 2^19 blocks
  const int b_lo = split * nblk / splits, b_hi = (split + 1) * nblk / splits;

  // The index resources come first; each role makes the others it uses
  // inside its own branch, so that the gather waves' first loads wait for
  // nothing but the preloaded arguments.
  BufRes res;
  if constexpr (GROUP) {
    res.id = __builtin_amdgcn_make_buffer_rsrc((void*)a.idx_d, (short)0, (int)((uint32_t)a.kd_total * 32u * 4u), kBufferWord3);
    res.is = __builtin_amdgcn_make_buffer_rsrc((void*)a.idx_s, (short)0, (int)((uint32_t)a.ks_total * 64u * 4u), kBufferWord3);
  } else {
    res.id = __builtin_amdgcn_make_buffer_rsrc((void*)k_idx_d, (short)0, (int)((uint32_t)k_kd_total * 32u * 4u), kBufferWord3);
    res.is = __builtin_amdgcn_make_buffer_rsrc((void*)k_idx_s, (short)0, (int)((uint32_t)k_ks_total * 64u * 4u), kBufferWord3);
  }

  f32x4 acc[2][NB];
  for (int h = 0; h < 2; ++h)
    for (int j = 0; j < NB; ++j) acc[h][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Y rows of this thread's outputs, read now so that the write-out at the
  // end does not wait for them: rows grow0 + e (one split) or the rows of
  // the final reduction (several splits).
  constexpr int OPT = 64 * NTOK / 256;
  const int64_t grow0 = (int64_t)t * k_rows + rb * 64 + (wave & 3) * 16 + 4 * kc;
  const int64_t grow_base = (int64_t)t * k_rows + rb * 64;
  int64_t yrow[OPT > 4 ? OPT : 4];
  if (threadIdx.x < 256) {
    constexpr int NR = OPT > 4 ? OPT : 4;
    const int nr = splits == 1 ? 4 : OPT;
    for (int k = 0; k < NR; ++k) yrow[k] = splits == 1 ? grow0 + k : grow_base + (threadIdx.x + 256 * k) / NTOK;
    if (a.out_rows) {
      // all the row-map loads first, then one wait
      int32_t d[NR];
#pragma unroll
      for (int k = 0; k < NR; ++k) d[k] = a.out_rows[k < nr ? yrow[k] : yrow[0]];
#pragma unroll
      for (int k = 0; k < NR; ++k) yrow[k] = (d[k] >= 0 && d[k] < a.cout) ? d[k] : -1;
    }
  }

  // Rounds of up to MAXB blocks.  Each role issues the loads of round r + 1
  // as soon as it is done with the registers of round r - the gather waves
  // right after their LDS store, the row waves right after their multiplies
  // - so the next round's load latency hides behind this round's work.  Two
  // barriers a round: X rows are in LDS; the row waves are done with them.
  const int nrounds = (b_hi - b_lo + MAXB - 1) / MAXB;
  if (gather) {
    res.x = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)(uint32_t)(((int64_t)(a.cin - 1) * a.ldx + a.batch) * 2), kBufferWord3);
    res.ldx_bytes = (uint32_t)a.ldx * 2u;
    // Gather thread gt takes 16-byte chunk gt % CPR of LDS positions
    // gt / CPR + PPJ * j; position p is slot p % 64 of block p / 64, so the
    // block of step j is a compile-time constant and the dense / 2:4 choice
    // is uniform.  Buffer loads: an out-of-range offset reads zero.
    constexpr int PPJ = GT / CPR;
    const int gt = threadIdx.x - 256;
    const int pofs = gt / CPR;
    // Tokens of this lane's chunk inside the batch.  A ragged batch or rows
    // that are not 16-byte aligned still take one 16-byte load per chunk
    // (buffer loads serve 2-byte aligned addresses).  The tokens past the
    // batch - the next row's, or zeros past the buffer - reach only output
    // columns that are never written.  A chunk wholly past the batch gets a
    // column offset past every buffer, so it reads zeros and costs nothing.
    const int vt = FAST ? 8 : min(8, a.batch - (n0 + 8 * (gt % CPR)));
    const uint32_t xcol = vt > 0 ? (uint32_t)(n0 + 8 * (gt % CPR)) * 2u : 0x80000000u;
    // The buffer ends with the last token of the last X row, and its range
    // check zeroes every dword that crosses that end: with an odd number of
    // tokens left, the last row's partial chunk would lose its last token.
    // That chunk is loaded from one token earlier, so that its dwords end
    // with the buffer, and shifted back at the LDS store.  A tile's index
    // lists name every X row at most once, so a lane meets that row at most
    // once a round.
    const int fixrow = (!FAST && vt > 0 && vt < 8 && (vt & 1)) ? a.cin - 1 : -2;
    if (ONE && a.batch == 1) {
      // Batch 1 (its own instantiation; the run-time test keeps the general
      // gather below in it, which the compiler schedules better around this
      // one than it does alone): a 2-byte load of each gathered
      // element (always aligned, never past the buffer's end), the rest of
      // its 16-token granule zero.  16-byte loads would start 2 bytes past a
      // dword at every odd row of a contiguous X (1.4-1.6 us more for the
      // q/k/v and gate/up groups), and a quarter of the registers holds the
      // round.
      static_assert(!ONE || (NTOK == 16 && !FAST), "batch 1 runs the 16-token kernel");
      uint32_t x1[MAXCH];
      auto issue1 = [&](int r0) {
        const int r1 = min(r0 + MAXB, b_hi);
        const int nbr = r1 - r0;
        const int nd_r = max(0, min(r1, tk.nbd) - r0);
        const uint32_t dbase = (uint32_t)(tk.kd0 + r0) * 32u;
        const uint32_t sbase = (uint32_t)(tk.ks0 + max(0, r0 - tk.nbd)) * 64u;
        int cidx[MAXCH];
#pragma unroll
        for (int j = 0; j < MAXCH; ++j) {
          const int blk = (PPJ * j) >> 6;
          const int slot = pofs + ((PPJ * j) & 63);
          const bool dense = blk < nd_r;
          const uint32_t li = dense ? dbase + 32u * blk + 2u * (slot >> 2) + (slot & 1)
                                    : sbase + 64u * (blk - nd_r) + slot;
          const __amdgpu_buffer_rsrc_t r = dense ? res.id : res.is;
          const bool ok = blk < nbr && !(dense && (slot & 2));
          const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(r, ok ? li * 4u : kOob, 0, 0);
          cidx[j] = ok ? v : -1;
        }
#pragma unroll
        for (int j = 0; j < MAXCH; ++j) {
          const int ci = cidx[j];
          // the second 8-token chunk's lanes have an offset past the buffer (xcol)
          const uint32_t off = ci < 0 ? kOob : __umul24((uint32_t)ci, res.ldx_bytes) + xcol;
          x1[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(res.x, off, 0, 0);
        }
      };
      if (nrounds > 0) issue1(b_lo);
      __syncthreads();   // the first X gathers are on their way: let the packed values go
      for (int r = 0; r < nrounds; ++r) {
#pragma unroll
        for (int j = 0; j < MAXCH; ++j)
          *reinterpret_cast<u32x4*>(xs + xs_gran<NB>(pofs + PPJ * j, (gt % CPR) >> 1) * 16 + 8 * (gt & 1)) =
              u32x4{x1[j], 0u, 0u, 0u};
        if (r + 1 < nrounds) issue1(b_lo + (r + 1) * MAXB);
        __syncthreads();   // X rows are in LDS
        __syncthreads();   // the row waves are done with them
      }
    } else {
    u32x4 xr[MAXCH];
    int fix_j = -1;
    auto issue = [&](int r0) {
      const int r1 = min(r0 + MAXB, b_hi);
      const int nbr = r1 - r0;
      const int nd_r = max(0, min(r1, tk.nbd) - r0);   // dense blocks come first in the block order
      const uint32_t dbase = (uint32_t)(tk.kd0 + r0) * 32u;
      const uint32_t sbase = (uint32_t)(tk.ks0 + max(0, r0 - tk.nbd)) * 64u;
      int cidx[MAXCH];
#pragma unroll
      for (int j = 0; j < MAXCH; ++j) {
        const int blk = (PPJ * j) >> 6;
        const int slot = pofs + ((PPJ * j) & 63);
        const bool dense = blk < nd_r;
        const uint32_t li = dense ? dbase + 32u * blk + 2u * (slot >> 2) + (slot & 1)
                                  : sbase + 64u * (blk - nd_r) + slot;
        const __amdgpu_buffer_rsrc_t r = dense ? res.id : res.is;
        // rows past the K range and a dense block's positions 4q+2, 4q+3
        // (never selected by its index pattern) read as zeros
        const bool ok = blk < nbr && !(dense && (slot & 2));
        const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(r, ok ? li * 4u : kOob, 0, 0);
        cidx[j] = ok ? v : -1;
      }
      fix_j = -1;
#pragma unroll
      for (int j = 0; j < MAXCH; ++j) {
        const int ci = cidx[j];
        const uint32_t off = ci < 0 ? kOob : __umul24((uint32_t)ci, res.ldx_bytes) + xcol;
        if constexpr (FAST) {
          xr[j] = __builtin_amdgcn_raw_buffer_load_b128(res.x, off, 0, 0);
        } else {
          const bool fix = ci == fixrow;
          xr[j] = __builtin_amdgcn_raw_buffer_load_b128(res.x, fix ? off - 2u : off, 0, 0);
          fix_j = fix ? j : fix_j;
        }
      }
    };
    if (nrounds > 0) issue(b_lo);
    __syncthreads();   // the first X gathers are on their way: let the packed values go
    for (int r = 0; r < nrounds; ++r) {
      if (!FAST && __builtin_amdgcn_ballot_w64(fix_j >= 0) != 0) {
        // a wave that holds the last row's shifted chunk
#pragma unroll
        for (int j = 0; j < MAXCH; ++j) {
          const uint32_t d0 = xr[j][0], d1 = xr[j][1], d2 = xr[j][2], d3 = xr[j][3];
          const bool sh = j == fix_j;
          *reinterpret_cast<u32x4*>(xs + xs_gran<NB>(pofs + PPJ * j, (gt % CPR) >> 1) * 16 + 8 * (gt & 1)) =
              u32x4{sh ? __builtin_amdgcn_alignbyte(d1, d0, 2) : d0, sh ? __builtin_amdgcn_alignbyte(d2, d1, 2) : d1,
                    sh ? __builtin_amdgcn_alignbyte(d3, d2, 2) : d2, sh ? d3 >> 16 : d3};
        }
      } else {
#pragma unroll
        for (int j = 0; j < MAXCH; ++j)
          *reinterpret_cast<u32x4*>(xs + xs_gran<NB>(pofs + PPJ * j, (gt % CPR) >> 1) * 16 + 8 * (gt & 1)) = xr[j];
      }
      if (r + 1 < nrounds) issue(b_lo + (r + 1) * MAXB);
      __syncthreads();   // X rows are in LDS
      __syncthreads();   // the row waves are done with them
    }
    }
  } else {
    // Each role holds its own barriers (the condition is uniform per wave),
    // so the two roles keep disjoint register sets.
    res.vd = __builtin_amdgcn_make_buffer_rsrc((void*)a.val_d, (short)0, (int)((uint32_t)a.kd_total * a.rows * 64u), kBufferWord3);
    res.vs = __builtin_amdgcn_make_buffer_rsrc((void*)a.val_s, (short)0, (int)((uint32_t)a.ks_total * a.rows * 64u), kBufferWord3);
    res.meta = __builtin_amdgcn_make_buffer_rsrc((void*)a.meta, (short)0, (int)((uint32_t)a.ks_total * a.rows * 8u), kBufferWord3);
    u32x4 av[MAXB];
    uint64_t mv[MAXB];
    // Loads of block r0 + j into slot j; a block past this split's range
    // reads zeros (its X rows are zeros too).
    auto issue_blk = [&](int r0, int j) {
      const int b = r0 + j;
      const bool dense = b < tk.nbd;
      const uint32_t brow = dense ? (uint32_t)((tk.kd0 + b) * a.rows + row)
                                  : (uint32_t)((tk.ks0 + (b - tk.nbd)) * a.rows + row);
      av[j] = __builtin_amdgcn_raw_buffer_load_b128(dense ? res.vd : res.vs, b < b_hi ? brow * 64u + 16u * kc : kOob,
                                                    0, 0);
      mv[j] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(res.meta, dense || b >= b_hi ? kOob
                                                                                                       : brow * 8u, 0, 0));
    };
    // This lane's transpose-read offsets within a block: positions
    // 8*kc + i16/4 + {0, 4, 32, 36}, token group nb, tokens 4*(i16 % 4)...
    int ro[4][NB];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        ro[k][nb] = xs_gran<NB>(8 * kc + (i16 >> 2) + 4 * (k & 1) + 32 * (k >> 1), nb) * 16 + 4 * (i16 & 3);
    // DPF blocks in flight ahead of the multiplies: a wave that queued all
    // of a round's loads at once would stall in issue, behind the memory
    // system's back-pressure, before it could multiply the first block.
    // Only P0 of them go out before the first X gathers: the index slices
    // those gathers wait for are tiny next to the packed values and would
    // otherwise queue behind them.
#pragma unroll
    for (int j = 0; j < P0; ++j) issue_blk(b_lo, j);
    __syncthreads();   // wait until the first X gathers are issued
#pragma unroll
    for (int j = P0; j < DPF; ++j) issue_blk(b_lo, j);
    for (int r = 0; r < nrounds; ++r) {
      const int r0 = b_lo + r * MAXB;
      const int nd_r = max(0, min(min(r0 + MAXB, b_hi), tk.nbd) - r0);
      // Nothing that reads the packed values may move above the barrier:
      // waiting for them there would hold back the whole workgroup.
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();   // X rows are in LDS
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < MAXB; ++j) {
        if (j + DPF < MAXB) issue_blk(r0, j + DPF);
        const bf16x8 A = __builtin_bit_cast(bf16x8, av[j]);
        const int sidx = j < nd_r ? 0x4444 : (int)((mv[j] >> (16 * kc)) & 0xffffull);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* base = xs + (64 * j) * NTOK;   // the swizzle maps blocks of 64 positions onto themselves
          const v4i16 b0 = tr_read(base + ro[0][nb]);
          const v4i16 b1 = tr_read(base + ro[1][nb]);
          const v4i16 b2 = tr_read(base + ro[2][nb]);
          const v4i16 b3 = tr_read(base + ro[3][nb]);
          const bf16x16 B = __builtin_bit_cast(
              bf16x16, __builtin_shufflevector(__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                               __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2,
                                               3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
          acc[j & 1][nb] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(A, B, acc[j & 1][nb], sidx, 0, 0);
        }
      }
      // the next round's first blocks (zeros after the last round)
#pragma unroll
      for (int j = 0; j < DPF; ++j) issue_blk(r0 + MAXB, j);
      __syncthreads();   // the next round overwrites xs
    }
  }
  for (int j = 0; j < NB; ++j) acc[0][j] += acc[1][j];

  // acc[nb][e]: tile row rb*64 + wave*16 + 4*kc + e, token 16*nb + i16.
  if (splits == 1) {
    if (!gather)
      for (int nb = 0; nb < NB; ++nb) {
        const int n = n0 + 16 * nb + i16;
        if (n < a.batch)
          for (int e = 0; e < 4; ++e)
            if (yrow[e] >= 0) a.y[yrow[e] * a.ldy + n] = bf16_rne(acc[0][nb][e]);
      }
    return;
  }
  // Partial sums: part[split][tb][rows of all weights][NTOK].  Partials and the arrival
  // counter go through agent-scope (device-coherent) stores, loads and
  // atomics, and each workgroup waits for its stores to complete before it
  // counts itself in, so nothing needs a whole-cache writeback or
  // invalidate.  The last workgroup of a (tile row block, token block) to
  // arrive adds the partials in split order and puts the counter back to 0.
  float* my = part + (((int64_t)split * n_tb + tb) * a.part_rows + row0) * NTOK;
  if (!gather)
    for (int nb = 0; nb < NB; ++nb)
      for (int e = 0; e < 4; ++e)
        __hip_atomic_store(my + (grow0 + e) * NTOK + 16 * nb + i16, acc[0][nb][e], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* ctr = counters + (int64_t)gtrb * n_tb + tb;
  if (threadIdx.x == 0) s_last = arrive(ctr, splits);
  __syncthreads();
  if (!s_last || threadIdx.x >= 256) return;
  const int64_t plane = (int64_t)n_tb * a.part_rows * NTOK;
  const float* p0 = part + ((int64_t)tb * a.part_rows + row0 + grow_base) * NTOK;
  float sum[OPT];
  for (int k = 0; k < OPT; ++k) sum[k] = 0.f;
  for (int sp0 = 0; sp0 < splits; sp0 += 8) {
    // up to 8 splits' loads in flight at once; none for splits past the last
    float v[8][OPT];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sp0 + u < splits) {
#pragma unroll
        for (int k = 0; k < OPT; ++k)
          v[u][k] = __hip_atomic_load(p0 + (sp0 + u) * plane + threadIdx.x + 256 * k, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      } else {
#pragma unroll
        for (int k = 0; k < OPT; ++k) v[u][k] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < OPT; ++k) sum[k] = (sp0 + u < splits) ? sum[k] + v[u][k] : sum[k];
  }
  for (int k = 0; k < OPT; ++k) {
    const int o = threadIdx.x + 256 * k;
    const int n = o % NTOK;
    if (n0 + n < a.batch && yrow[k] >= 0) a.y[yrow[k] * a.ldy + n0 + n] = bf16_rne(sum[k]);
  }
}

// The rest of a one-weight split decode's arguments: only fields its body
// reads, so that no argument-buffer load brings in a word the kernel does
// not use (the compiler reuses such a word's register at once, and must
// then wait for the load in flight before the first index loads).
struct DecArgs {
  const uint16_t* val_d;
  const uint16_t* val_s;
  const uint64_t* meta;
  const uint16_t* x;
  uint16_t* y;
  const int32_t* out_rows;
  int64_t ldy;
  int ldx;                   // below 2^23 on this path
  int batch, cin, cout, part_rows, n_tb;
};

// One weight.  The leading arguments are plain scalars, preloaded into SGPRs
// at wave launch, so the index loads go out without waiting for the
// argument buffer.
template <int NTOK, int MAXB, bool FAST, int NG, bool ONE = false>
__global__ __launch_bounds__(256 + 64 * NG) void decode5_kernel(const int32_t* __restrict__ k_idx_d,
                                                                const int32_t* __restrict__ k_idx_s,
                                                                const int32_t* __restrict__ k_tiles, int k_kd_total,
                                                                int k_ks_total, int k_nkb_d, int k_nkb_s, int k_rows,
                                                                int splits, int k_r1, DecArgs d,
                                                                float* __restrict__ part,
                                                                unsigned* __restrict__ counters) {
  SpmmArgs a0{};
  a0.val_d = d.val_d;
  a0.val_s = d.val_s;
  a0.meta = d.meta;
  a0.x = d.x;
  a0.y = d.y;
  a0.out_rows = d.out_rows;
  a0.ldx = d.ldx;
  a0.ldy = d.ldy;
  a0.batch = d.batch;
  a0.cin = d.cin;
  a0.cout = d.cout;
  a0.part_rows = d.part_rows;
  a0.rows = k_rows;
  a0.kd_total = k_kd_total;
  a0.ks_total = k_ks_total;
  decode5_body<NTOK, MAXB, FAST, NG, ONE, false>(k_idx_d, k_idx_s, k_tiles, k_kd_total, k_ks_total, k_nkb_d, k_nkb_s,
                                                 k_rows, splits, k_r1, 0, a0, nullptr, d.n_tb, part, counters);
}

// A group of up to 8 weights.  b1..b7 are the first concatenated row blocks
// of weights 1..7 (INT_MAX past the last weight), preloaded like the
// one-weight kernel's leading arguments, so a workgroup finds its weight
// without reading the segment table and then reads that weight's fields in
// one round trip.
template <int NTOK, int MAXB, bool FAST, int NG, bool ONE = false>
__global__ __launch_bounds__(256 + 64 * NG) void decode5_group_kernel(int k_rows, int splits, int k_r1, int b1, int b2,
                                                                      int b3, int b4, int b5, int b6, int b7,
                                                                      SpmmArgs a0, Segs segs, int n_tb,
                                                                      float* __restrict__ part,
                                                                      unsigned* __restrict__ counters) {
  static_assert(kMaxSeg == 8, "seven boundaries");
  const int gtrb = wg_split(blockIdx.x, splits, k_r1).gtrb;
  const int g = (gtrb >= b1) + (gtrb >= b2) + (gtrb >= b3) + (gtrb >= b4) + (gtrb >= b5) + (gtrb >= b6) +
                (gtrb >= b7);
  decode5_body<NTOK, MAXB, FAST, NG, ONE, true>(nullptr, nullptr, nullptr, 0, 0, 0, 0, k_rows, splits, k_r1, g, a0, &segs,
                                                n_tb, part, counters);
}

// ---------------------------------------------------------------------------
// Prefill kernel, software-pipelined (large batches, tile_rows % 64 == 0).
// Workgroup = 64 rows of one tile x NT tokens, 4 waves of 64 rows x NT/4
// tokens.  K-blocks stream through a double-buffered LDS tile of gathered X
// rows; while block b is multiplied, the X rows and packed values of block
// b+1 are in flight into registers and the index slice of block b+2 is being
// fetched.  Loads go through buffer resources with 32-bit offsets: a gathered
// row costs one 24-bit multiply-add, and pad indices get an out-of-range
// offset so the hardware returns zeros.  All loads are unconditional (a dense
// block repeats its 32 rows into the unused half of the tile) and the loop is
// unrolled twice over two register sets, so the code is straight-line.
// Dense blocks: v_mfma_f32_32x32x16_bf16; 2:4 blocks:
// v_smfmac_f32_32x32x32_bf16; B operands via ds_read_b64_tr_b16 from rows
// whose pitch is 64 bytes mod 256, which keeps each pair of 16-lane groups
// of a transpose read on disjoint banks.  Workgroups are ordered so each XCD
// sweeps one token block across all tiles.  Y leaves through LDS in 16-byte
// row chunks.
// ---------------------------------------------------------------------------
template <int NT>
struct PrefillCfg {
  static constexpr int PITCH = NT + 32;       // bf16 per LDS row: 64 bytes mod 256
  static constexpr int TW = NT / 4;           // tokens per wave
  static constexpr int NTB = TW / 32;         // 32-token MFMA blocks per wave
  static constexpr int CPR = NT / 8;          // 16-byte chunks per gathered row
  static constexpr int PG = 256 / CPR;        // position groups per workgroup
  static constexpr int DA = 4;                // packed-value prefetch depth (blocks)
  // The block loops are unrolled four times over compile-time register sets
  // and step k uses packed-value set k % DA, so DA must divide 4 (a depth of
  // 3 or 6 would pair blocks with the wrong values).
  static_assert(4 % DA == 0, "packed-value prefetch depth must divide the unroll of 4");
};

// This thread's share of one block's packed values (16 bytes) and 2:4
// metadata (4 bytes, threads 0..127) on the way to LDS.
struct PrefillA {
  u32x4 v;
  uint32_t m;
};


// One region's K-blocks [0, nb) (DENSE: 32-column blocks, else 2:4 blocks of
// 64 positions), pipelined.  Keeping the two regions in separate loops keeps
// the accumulators in fixed registers.
//
// Every byte a workgroup needs is fetched once per workgroup:
//   - X: thread (position group, chunk) gathers PPT rows x 16 bytes; the 64
//     positions of a 2:4 block give PPT = 64 / PG, the 32 of a dense block
//     PPT / 2.
//   - indices: each wave loads the WP indices of its own positions, one per
//     lane, and hands them to its lane groups with v_readlane and selects.
//   - packed values: one 16-byte load per thread covers the 64 rows x 64
//     bytes of a block; they are written into the 64-byte padding at the end
//     of each X row of the LDS tile (row r's chunk c at chunk c ^ (r/4 % 4),
//     so 16 consecutive rows of one chunk fall on distinct banks).
//   - 2:4 metadata: 512 bytes per block, one dword per thread of waves 0-1,
//     into a small LDS array.
template <int NT, bool FAST, bool DENSE>
__device__ inline void prefill_phase(const SpmmArgs& a, const BufRes& res, uint16_t* xs0, uint16_t* xs1,
                                     uint32_t* ms0, uint32_t* ms1, int kbase, int nb, int rot, int rb, int n0,
                                     f32x16 (&acc)[2][PrefillCfg<NT>::NTB]) {
  using C = PrefillCfg<NT>;
  constexpr int KPOS = DENSE ? 32 : 64;       // positions per block
  constexpr int PPT = KPOS / C::PG;           // gathered rows per thread
  constexpr int WP = KPOS / 4;                // positions per wave
  if (nb == 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok_w = wave * C::TW;
  const int g = lane >> 4, i = lane & 15;
  const int kcb = g >> 1;                       // B-operand K chunk (0..1)
  const int colb = tok_w + 16 * (g & 1) + 4 * (i & 3);
  const int kca = lane >> 5;                    // A-operand K chunk (0..1)
  const int cnk = threadIdx.x % C::CPR;
  const int pbase = (threadIdx.x / C::CPR) * PPT;          // first of this thread's PPT positions
  constexpr int G = 64 / C::CPR;              // position groups per wave
  const int grp = lane / C::CPR;
  // Without FAST (unaligned X rows or the batch's last token block): one
  // 16-byte load per chunk all the same (buffer loads take 2-byte-aligned
  // offsets); a chunk wholly past the batch reads zeros, tokens past the
  // batch inside a chunk reach only unwritten output columns, and the last X
  // row's partial chunk with an odd token count is loaded one token early
  // (the buffer's range check zeroes every dword crossing its end) and
  // shifted back at the LDS store.
  const int vt = FAST ? 8 : min(8, a.batch - (n0 + 8 * cnk));
  const uint32_t xcol = vt > 0 ? (uint32_t)(n0 + 8 * cnk) * 2u : 0x80000000u;
  const int fixrow = (!FAST && vt > 0 && vt < 8 && (vt & 1)) ? a.cin - 1 : -2;
  const __amdgpu_buffer_rsrc_t rid = DENSE ? res.id : res.is;
  const __amdgpu_buffer_rsrc_t rv = DENSE ? res.vd : res.vs;
  const uint32_t vrow = (uint32_t)rb * 64u;
  const int arow = threadIdx.x >> 2;                       // value row this thread stores
  const int acol = C::PITCH * arow + NT + 8 * ((threadIdx.x & 3) ^ ((arow >> 2) & 3));

  // Indices: each lane of a wave loads one of the wave's WP indices; lane
  // group q then takes positions q*PPT .. q*PPT+PPT-1 of them through
  // v_readlane (uniform values) and per-group selects.
  const uint32_t ipos = (uint32_t)(wave * WP + (lane % WP));
  auto load_idx = [&](int b) -> int {
    b = min(b, nb - 1);
    b = b + rot < nb ? b + rot : b + rot - nb;     // the block order starts at block rot
    const uint32_t off = ((uint32_t)(kbase + b) * KPOS + ipos) * 4u;
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rid, off, 0, 0);
  };
  auto spread_idx = [&](int iw, int (&ci)[PPT]) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      int c = __builtin_amdgcn_readlane(iw, j);
#pragma unroll
      for (int q = 1; q < G; ++q) {
        const int m = -(int)(grp == q);
        c = (c & ~m) | (__builtin_amdgcn_readlane(iw, q * PPT + j) & m);
      }
      ci[j] = c;
    }
  };
  int fixm[2] = {0, 0};                       // per register set: loads j that were shifted
  auto load_x = [&](const int (&ci)[PPT], u32x4 (&st)[PPT], int& fm) {
    fm = 0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const uint32_t off = ci[j] < 0 ? kOob : __umul24((uint32_t)ci[j], res.ldx_bytes) + xcol;
      if constexpr (FAST) {
        st[j] = __builtin_amdgcn_raw_buffer_load_b128(res.x, off, 0, 0);
      } else {
        const bool fix = ci[j] == fixrow;
        st[j] = __builtin_amdgcn_raw_buffer_load_b128(res.x, fix ? off - 2u : off, 0, 0);
        fm |= fix ? 1 << j : 0;
      }
    }
  };
  auto load_a = [&](int b, PrefillA& st) {
    b = min(b, nb - 1);
    b = b + rot < nb ? b + rot : b + rot - nb;
    const uint32_t blk = (uint32_t)(kbase + b) * (uint32_t)a.rows + vrow;
    st.v = __builtin_amdgcn_raw_buffer_load_b128(rv, blk * 64u + 16u * threadIdx.x, 0, 0);
    if constexpr (!DENSE)
      st.m = __builtin_amdgcn_raw_buffer_load_b32(res.meta, threadIdx.x < 128 ? blk * 8u + 4u * threadIdx.x : kOob,
                                                  0, 0);
  };
  auto store = [&](uint16_t* xs, uint32_t* ms, const u32x4 (&x)[PPT], int fm, const PrefillA& st) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      u32x4 v = x[j];
      if constexpr (!FAST) {                      // shift the last X row's partial chunk (selects, no branch)
        const bool sh = (fm >> j) & 1;
        const uint32_t d0 = x[j][0], d1 = x[j][1], d2 = x[j][2], d3 = x[j][3];
        v = u32x4{sh ? __builtin_amdgcn_alignbyte(d1, d0, 2) : d0, sh ? __builtin_amdgcn_alignbyte(d2, d1, 2) : d1,
                  sh ? __builtin_amdgcn_alignbyte(d3, d2, 2) : d2, sh ? d3 >> 16 : d3};
      }
      *reinterpret_cast<u32x4*>(xs + (pbase + j) * C::PITCH + 8 * cnk) = v;
    }
    *reinterpret_cast<u32x4*>(xs + acol) = st.v;
    if constexpr (!DENSE)
      if (threadIdx.x < 128) ms[threadIdx.x] = st.m;
  };
  auto compute = [&](const uint16_t* xb, const uint32_t* ms) {
    u32x4 av[4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 32 * r + (lane & 31);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        av[2 * r + s] = *reinterpret_cast<const u32x4*>(xb + row * C::PITCH + NT + 8 * ((2 * s + kca) ^ ((row >> 2) & 3)));
    }
    if constexpr (DENSE) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {               // two K steps of 16 columns
#pragma unroll
        for (int j = 0; j < C::NTB; ++j) {
          const uint16_t* base = xb + colb + 32 * j;
          const v4i16 b0 = tr_read(base + (16 * s + 8 * kcb + 0 + (i >> 2)) * C::PITCH);
          const v4i16 b1 = tr_read(base + (16 * s + 8 * kcb + 4 + (i >> 2)) * C::PITCH);
          const bf16x8 B = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int r = 0; r < 2; ++r)
            acc[r][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[2 * r + s]), B,
                                                                acc[r][j], 0, 0, 0);
        }
      }
    } else {
      const uint64_t* mt = reinterpret_cast<const uint64_t*>(ms);
      const uint64_t mv[2] = {mt[lane & 31], mt[32 + (lane & 31)]};
#pragma unroll
      for (int s = 0; s < 2; ++s) {               // two K steps of 32 positions
        int sidx[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) sidx[r] = (int)((mv[r] >> (32 * s + 16 * kca)) & 0xffffull);
#pragma unroll
        for (int j = 0; j < C::NTB; ++j) {
          const uint16_t* base = xb + colb + 32 * j;
          const int p0 = 32 * s + 8 * kcb + (i >> 2);
          const v4i16 b0 = tr_read(base + (p0 + 0) * C::PITCH);
          const v4i16 b1 = tr_read(base + (p0 + 4) * C::PITCH);
          const v4i16 b2 = tr_read(base + (p0 + 16) * C::PITCH);
          const v4i16 b3 = tr_read(base + (p0 + 20) * C::PITCH);
          const bf16x16 B = __builtin_bit_cast(
              bf16x16, __builtin_shufflevector(__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                               __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3,
                                               4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
#pragma unroll
          for (int r = 0; r < 2; ++r)
            acc[r][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, av[2 * r + s]), B,
                                                                  acc[r][j], sidx[r], 0, 0);
        }
      }
    }
  };

  __syncthreads();                   // the LDS tiles may still be read by the previous phase
  // Register sets: packed values of DA blocks (A[b % DA]), X rows of 2 blocks
  // (X[b % 2]) and the indices of one block.  At block bb: issue the X
  // gathers of bb+2 (their indices arrived during bb-1), then the indices of
  // bb+3 and the values of bb+DA; compute bb from LDS tile bb % 2; write X and
  // values of bb+1 into the other tile.  An X gather has about two block
  // times to arrive, a value load DA block times.
  constexpr int DA = C::DA;
  PrefillA A[DA];
  u32x4 X[2][PPT];
  int Iw[2];                          // index words of blocks bb+3 and bb+4
  int CI[PPT];                        // this thread's indices of block bb+2
  uint16_t* const tile[2] = {xs0, xs1};
  uint32_t* const mtile[2] = {ms0, ms1};
  Iw[0] = load_idx(0);
  Iw[1] = load_idx(1);
  spread_idx(Iw[0], CI);
  load_x(CI, X[0], fixm[0]);
  spread_idx(Iw[1], CI);
  load_x(CI, X[1], fixm[1]);
  Iw[0] = load_idx(2);
  Iw[1] = load_idx(3);
#pragma unroll
  for (int d = 0; d < DA; ++d) load_a(d, A[d]);
  spread_idx(Iw[0], CI);
  store(tile[0], mtile[0], X[0], fixm[0], A[0]);
  __syncthreads();
  auto step = [&](auto kc, int bb) {
    constexpr int k = decltype(kc)::value;
    load_x(CI, X[k % 2], fixm[k % 2]); // X(bb+2)
    Iw[k % 2] = load_idx(bb + 4);
    load_a(bb + DA, A[k % DA]);
    compute(tile[k % 2], mtile[k % 2]);
    store(tile[(k + 1) % 2], mtile[(k + 1) % 2], X[(k + 1) % 2], fixm[(k + 1) % 2], A[(k + 1) % DA]);
    spread_idx(Iw[(k + 1) % 2], CI);  // indices of bb+3
    __syncthreads();
  };
  int b = 0;
  for (; b + 4 <= nb; b += 4) {
    step(std::integral_constant<int, 0>{}, b);
    step(std::integral_constant<int, 1>{}, b + 1);
    step(std::integral_constant<int, 2>{}, b + 2);
    step(std::integral_constant<int, 3>{}, b + 3);
  }
  if (b < nb) step(std::integral_constant<int, 0>{}, b);
  if (b + 1 < nb) step(std::integral_constant<int, 1>{}, b + 1);
  if (b + 2 < nb) step(std::integral_constant<int, 2>{}, b + 2);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// s_waitcnt with only the vector-memory count: vmcnt(n), nothing else.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A buffer load whose 16 bytes per lane go straight to LDS: lane l's bytes
// land at lds + 16 l (an offset past the buffer writes zeros).  The sc0 bit
// (cache policy 1) makes the load miss in the CU's L1 and read from L2: a
// gathered X row is used once per workgroup, so L1 allocation buys nothing
// (0.5-1% faster on every batch-1024/2048 shape measured).
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_u8*)lds, 16, off, 0, 0, 1);
}

__device__ inline v4i16 tr_read_b(const uint8_t* lds) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u8*)lds);
}

// prefill_phase with the X rows loaded straight into LDS (buffer loads into
// LDS take 2-byte-aligned addresses, so any X layout).  The gathered rows
// never pass through VGPRs: each wave issues
// its share of block b + 1's rows into the other tile at the start of step
// b, multiplies block b, stores the packed values of b + 1 (loaded DA blocks
// earlier through VGPRs), waits for its own row loads and meets the other
// waves at the barrier.
//
// Tile layout (bytes): X rows, 64 positions x 2 NT bytes, the 16-byte chunk c
// of position p at chunk c ^ 4 (p % 4) (a 32-lane half of a transpose read
// then covers every bank once); packed values at 128 NT, 64 rows x 64 bytes,
// chunk q of row r at q ^ (r / 4 % 4).  X load j of a wave brings 64 / CPR
// consecutive positions starting at wave * RPW + j * 64 / CPR, lane l taking
// chunk l % CPR of position + l / CPR.
//
// TAIL (1 or 2: the token block ends past the batch): chunks wholly past the
// batch read zeros (no traffic); tokens past the batch inside a chunk reach
// only output columns that are never written.  The buffer ends with the last
// token of the last X row and its range check zeroes every dword that
// crosses that end, so with an odd batch (TAIL 2) the last row's partial
// chunk with an odd token count is loaded one token early and shifted back
// in LDS once it has landed (a tile names each X row at most once).  The
// shift is a branch, which is kept out of the other instantiations.
template <int NT, bool DENSE, int TAIL>
__device__ inline void prefill_phase_lds(const SpmmArgs& a, const BufRes& res, uint16_t* xs0, uint16_t* xs1,
                                         uint32_t* ms0, uint32_t* ms1, int kbase, int nb, int rot, int rb, int n0,
                                         f32x16 (&acc)[2][PrefillCfg<NT>::NTB]) {
  using C = PrefillCfg<NT>;
  constexpr int KPOS = DENSE ? 32 : 64;       // positions per block
  constexpr int RPW = KPOS / 4;               // positions per wave
  constexpr int XROW = 2 * NT;                // bytes per X row in LDS
  constexpr int CPR = NT / 8;                 // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;               // positions per X load
  constexpr int NJ = RPW / RPL;               // X loads per wave per block
  constexpr int AOFS = 64 * XROW;             // packed values
  constexpr int PA = DENSE ? 2 : 3;           // loads a step issues after its X loads
  static_assert(AOFS + 64 * 64 <= 64 * C::PITCH * 2, "tile size");
  if (nb == 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok_w = wave * C::TW;
  const int g = lane >> 4, i = lane & 15;
  const int kcb = g >> 1;                     // B-operand K chunk (0..1)
  const int kca = lane >> 5;                  // A-operand K chunk (0..1)
  const int q = lane / CPR, sl = lane % CPR;
  const __amdgpu_buffer_rsrc_t rid = DENSE ? res.id : res.is;
  const __amdgpu_buffer_rsrc_t rv = DENSE ? res.vd : res.vs;
  const uint32_t vrow = (uint32_t)rb * 64u;
  const uint32_t xcol = (uint32_t)n0 * 2u;
  uint32_t xch[NJ];                           // this lane's source chunk of X load j, in bytes
#pragma unroll
  for (int j = 0; j < NJ; ++j) xch[j] = 16u * (uint32_t)(sl ^ (4 * ((j * RPL + q) & 3)));
  const int arow = threadIdx.x >> 2;          // packed-value row this thread stores
  const int aofs = AOFS + arow * 64 + 16 * ((threadIdx.x & 3) ^ ((arow >> 2) & 3));

  // Indices: lane l < RPW of the wave loads the index of position
  // wave * RPW + l; X load j of lane l needs the one of position
  // j * RPL + l / CPR, taken with v_readlane and selects.
  const uint32_t ipos = (uint32_t)(wave * RPW + (lane % RPW));
  auto load_idx = [&](int b) -> int {
    b = min(b, nb - 1);
    b = b + rot < nb ? b + rot : b + rot - nb;     // the block order starts at block rot
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rid, ((uint32_t)(kbase + b) * KPOS + ipos) * 4u, 0, 0);
  };
  auto spread_idx = [&](int iw, int (&ci)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      int c = __builtin_amdgcn_readlane(iw, j * RPL);
#pragma unroll
      for (int u = 1; u < RPL; ++u) {
        const int m = -(int)(q == u);
        c = (c & ~m) | (__builtin_amdgcn_readlane(iw, j * RPL + u) & m);
      }
      ci[j] = c;
    }
  };
  int fixm = 0;                               // TAIL: loads j of the last issue that were shifted
  auto load_x = [&](const int (&ci)[NJ], uint16_t* xs) {
    fixm = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint32_t off = ci[j] < 0 ? kOob : __umul24((uint32_t)ci[j], res.ldx_bytes) + xcol + xch[j];
      if constexpr (TAIL != 0) {
        const int vt = a.batch - (n0 + (int)(xch[j] >> 1));   // tokens of the chunk inside the batch
        off = vt <= 0 ? kOob : off;
        if constexpr (TAIL == 2) {
          const bool fix = ci[j] == a.cin - 1 && vt > 0 && vt < 8 && (vt & 1);
          off = fix ? off - 2u : off;
          fixm |= fix ? 1 << j : 0;
        }
      }
      load_lds16(res.x, reinterpret_cast<uint8_t*>(xs) + (wave * RPW + j * RPL) * XROW, off);
    }
  };
  // TAIL, after this wave's loads have landed: shift the marked chunks back by one token
  auto fix_x = [&](uint16_t* xs) {
    if constexpr (TAIL == 2) {
      if (__builtin_amdgcn_ballot_w64(fixm != 0) != 0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (fixm & (1 << j)) {
            u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(xs) + (wave * RPW + j * RPL) * XROW + 16 * lane);
            const u32x4 d = *p;
            *p = u32x4{__builtin_amdgcn_alignbyte(d[1], d[0], 2), __builtin_amdgcn_alignbyte(d[2], d[1], 2),
                       __builtin_amdgcn_alignbyte(d[3], d[2], 2), d[3] >> 16};
          }
        }
      }
    }
  };
  auto load_a = [&](int b, PrefillA& st) {
    b = min(b, nb - 1);
    b = b + rot < nb ? b + rot : b + rot - nb;
    const uint32_t blk = (uint32_t)(kbase + b) * (uint32_t)a.rows + vrow;
    st.v = __builtin_amdgcn_raw_buffer_load_b128(rv, blk * 64u + 16u * threadIdx.x, 0, 0);
    if constexpr (!DENSE)
      st.m = __builtin_amdgcn_raw_buffer_load_b32(res.meta, threadIdx.x < 128 ? blk * 8u + 4u * threadIdx.x : kOob,
                                                  0, 0);
  };
  auto store_a = [&](uint16_t* xs, uint32_t* ms, const PrefillA& st) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(xs) + aofs) = st.v;
    if constexpr (!DENSE)
      if (threadIdx.x < 128) ms[threadIdx.x] = st.m;
  };
  // B operand: lane (g, i) reads 4 tokens of position p (p % 4 == i / 4) at
  // token tok_w + 16 (g % 2) + 4 (i % 4) + 32 j.
  const uint32_t cb0 = (uint32_t)(tok_w / 8 + 2 * (g & 1) + ((i >> 1) & 1));
  const uint32_t bsw = (uint32_t)(4 * ((i >> 2) & 3));
  auto compute = [&](const uint16_t* xt, const uint32_t* ms) {
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(xt);
    u32x4 av[4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 32 * r + (lane & 31);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        av[2 * r + s] = *reinterpret_cast<const u32x4*>(xb + AOFS + row * 64 + 16 * ((2 * s + kca) ^ ((row >> 2) & 3)));
    }
    if constexpr (DENSE) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {               // two K steps of 16 columns
#pragma unroll
        for (int j = 0; j < C::NTB; ++j) {
          const uint8_t* base = xb + 16u * ((cb0 + 4u * j) ^ bsw) + 8u * (i & 1) + (16 * s + 8 * kcb + (i >> 2)) * XROW;
          const v4i16 b0 = tr_read_b(base);
          const v4i16 b1 = tr_read_b(base + 4 * XROW);
          const bf16x8 B = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int r = 0; r < 2; ++r)
            acc[r][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[2 * r + s]), B,
                                                                acc[r][j], 0, 0, 0);
        }
      }
    } else {
      const uint64_t* mt = reinterpret_cast<const uint64_t*>(ms);
      const uint64_t mv[2] = {mt[lane & 31], mt[32 + (lane & 31)]};
#pragma unroll
      for (int s = 0; s < 2; ++s) {               // two K steps of 32 positions
        int sidx[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) sidx[r] = (int)((mv[r] >> (32 * s + 16 * kca)) & 0xffffull);
#pragma unroll
        for (int j = 0; j < C::NTB; ++j) {
          const uint8_t* base = xb + 16u * ((cb0 + 4u * j) ^ bsw) + 8u * (i & 1) + (32 * s + 8 * kcb + (i >> 2)) * XROW;
          const v4i16 b0 = tr_read_b(base);
          const v4i16 b1 = tr_read_b(base + 4 * XROW);
          const v4i16 b2 = tr_read_b(base + 16 * XROW);
          const v4i16 b3 = tr_read_b(base + 20 * XROW);
          const bf16x16 B = __builtin_bit_cast(
              bf16x16, __builtin_shufflevector(__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7),
                                               __builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3,
                                               4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15));
#pragma unroll
          for (int r = 0; r < 2; ++r)
            acc[r][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8, av[2 * r + s]), B,
                                                                  acc[r][j], sidx[r], 0, 0);
        }
      }
    }
  };

  __syncthreads();                   // the LDS tiles may still be read by the previous phase
  // Register sets: packed values of DA blocks (A[b % DA]) and the index
  // words of blocks bb+2 and bb+3.  At block bb: issue the X rows of bb+1
  // into the other tile, the indices of bb+3 and the values of bb+DA;
  // multiply bb; store the values of bb+1; spread the indices of bb+2; wait
  // for this wave's rows of bb+1; barrier.
  constexpr int DA = C::DA;
  PrefillA A[DA];
  int Iw[2];
  int CI[NJ];
  uint16_t* const tile[2] = {xs0, xs1};
  uint32_t* const mtile[2] = {ms0, ms1};
  Iw[0] = load_idx(0);
  Iw[1] = load_idx(1);
#pragma unroll
  for (int d = 0; d < DA; ++d) load_a(d, A[d]);
  spread_idx(Iw[0], CI);
  load_x(CI, tile[0]);
  spread_idx(Iw[1], CI);
  Iw[0] = load_idx(2);
  store_a(tile[0], mtile[0], A[0]);
  wait_vm<1>();                      // the X rows of block 0 (only the index load of block 2 is younger)
  fix_x(tile[0]);
  __syncthreads();
  auto step = [&](auto kc, int bb) {
    constexpr int k = decltype(kc)::value;
    // Raised priority while the wave issues its loads, so that on a SIMD
    // shared with the other workgroup the gathers go out ahead of that
    // workgroup's MFMA and LDS work and more lines stay in flight.
    __builtin_amdgcn_s_setprio(2);
    if (bb + 1 < nb) load_x(CI, tile[(k + 1) % 2]);   // X(bb+1)
    else fixm = 0;
    Iw[(k + 1) % 2] = load_idx(bb + 3);
    load_a(bb + DA, A[k % DA]);
    __builtin_amdgcn_s_setprio(0);
    compute(tile[k % 2], mtile[k % 2]);
    store_a(tile[(k + 1) % 2], mtile[(k + 1) % 2], A[(k + 1) % DA]);
    spread_idx(Iw[k % 2], CI);        // indices of bb+2
    wait_vm<PA>();                    // this wave's X rows of bb+1 are in LDS
    fix_x(tile[(k + 1) % 2]);
    __syncthreads();
  };
  int b = 0;
  for (; b + 4 <= nb; b += 4) {
    step(std::integral_constant<int, 0>{}, b);
    step(std::integral_constant<int, 1>{}, b + 1);
    step(std::integral_constant<int, 2>{}, b + 2);
    step(std::integral_constant<int, 3>{}, b + 3);
  }
  if (b < nb) step(std::integral_constant<int, 0>{}, b);
  if (b + 1 < nb) step(std::integral_constant<int, 1>{}, b + 1);
  if (b + 2 < nb) step(std::integral_constant<int, 2>{}, b + 2);
}

// FAST: 16-byte aligned X rows and a token block inside the batch; TAIL: the
// token block ends past the batch (1: even batch, 2: odd batch).
// Share `split` of an item's K range split `splits` ways: the first dense and
// 2:4 block and the counts.  The blocks stay in order, dense first.  Cut in
// two, the range is cut by cost: a 2:4 block gathers 64 X rows against a
// dense block's 32, so a dense block counts one unit and a 2:4 block two (a
// cut inside a 2:4 block goes to its start, the same rule for both halves,
// so the halves partition the blocks).  Cut in four, it is cut by block
// count: the cost cut was measured slower there (down_proj 4096x11008 at
// batch 128 / 256 / 512: 21.7 / 30.7 / 42.3 -> 24.1 / 31.8 / 43.2 us, four
// balanced splits finishing and handing over their partial sums together),
// while in two it was faster (batch 800 / 1024: 61.6 / 60.1 -> 60.3 / 58.8;
// up_proj 11008x4096 at batch 256, halves: 30.2 -> 29.1).
struct KShare {
  int kd, nd, ks, ns;
  int rd, rs;       // first block of the dense and 2:4 loops (the order wraps around)
};
__device__ inline KShare k_share(const TileK& tk, int split, int splits) {
  const int w = splits == 2 ? 2 : 1;                 // units of a 2:4 block
  const int64_t units = tk.nbd + w * (int64_t)tk.nbs;
  const int lo = (int)((int64_t)split * units / splits), hi = (int)((int64_t)(split + 1) * units / splits);
  const int d_lo = min(lo, tk.nbd), d_hi = min(hi, tk.nbd);
  const int s_lo = (max(lo, tk.nbd) - tk.nbd) / w, s_hi = (max(hi, tk.nbd) - tk.nbd) / w;
  return {tk.kd0 + d_lo, d_hi - d_lo, tk.ks0 + s_lo, s_hi - s_lo, 0, 0};
}

// X straight into LDS; TAIL: the token block ends past the batch (1: even
// batch, 2: odd batch).
template <int NT, int TAIL>
__device__ inline void prefill_body_lds(const SpmmArgs& a, const BufRes& res, uint16_t* xs0, uint16_t* xs1,
                                        uint32_t* ms0, uint32_t* ms1, const KShare& ks, int rb, int n0,
                                        f32x16 (&acc)[2][PrefillCfg<NT>::NTB]) {
  prefill_phase_lds<NT, true, TAIL>(a, res, xs0, xs1, ms0, ms1, ks.kd, ks.nd, ks.rd, rb, n0, acc);
  prefill_phase_lds<NT, false, TAIL>(a, res, xs0, xs1, ms0, ms1, ks.ks, ks.ns, ks.rs, rb, n0, acc);
}

// X through registers; FAST: 16-byte aligned X rows and a token block inside
// the batch.
template <int NT, bool FAST>
__device__ inline void prefill_body_staged(const SpmmArgs& a, const BufRes& res, uint16_t* xs0, uint16_t* xs1,
                                           uint32_t* ms0, uint32_t* ms1, const KShare& ks, int rb, int n0,
                                           f32x16 (&acc)[2][PrefillCfg<NT>::NTB]) {
  prefill_phase<NT, FAST, true>(a, res, xs0, xs1, ms0, ms1, ks.kd, ks.nd, ks.rd, rb, n0, acc);
  prefill_phase<NT, FAST, false>(a, res, xs0, xs1, ms0, ms1, ks.ks, ks.ns, ks.rs, rb, n0, acc);
}

// Persistent launch: gridDim.x = 8 * per_xcd workgroups, workgroup L runs on
// XCD L % 8 (round-robin dispatch).  The (token block, tile row block) items,
// token-block major, are cut into 8 contiguous ranges, one per XCD; the XCD's
// workgroups take its range in order, so each XCD works through its token
// blocks one after another and keeps the current X slice in its L2.
__device__ inline BufRes make_res(const SpmmArgs& a) {
  BufRes res;
  const uint32_t xbytes = (uint32_t)(((int64_t)(a.cin - 1) * a.ldx + a.batch) * 2);
  res.x = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)xbytes, kBufferWord3);
  res.vd = __builtin_amdgcn_make_buffer_rsrc((void*)a.val_d, (short)0, (int)((uint32_t)a.kd_total * a.rows * 64u), kBufferWord3);
  res.vs = __builtin_amdgcn_make_buffer_rsrc((void*)a.val_s, (short)0, (int)((uint32_t)a.ks_total * a.rows * 64u), kBufferWord3);
  res.meta = __builtin_amdgcn_make_buffer_rsrc((void*)a.meta, (short)0, (int)((uint32_t)a.ks_total * a.rows * 8u), kBufferWord3);
  res.id = __builtin_amdgcn_make_buffer_rsrc((void*)a.idx_d, (short)0, (int)((uint32_t)a.kd_total * 32u * 4u), kBufferWord3);
  res.is = __builtin_amdgcn_make_buffer_rsrc((void*)a.idx_s, (short)0, (int)((uint32_t)a.ks_total * 64u * 4u), kBufferWord3);
  res.ldx_bytes = (uint32_t)a.ldx * 2u;
  return res;
}

template <int NT, bool SPLIT, bool MIX = false>
__global__ __launch_bounds__(256, 2) void prefill_kernel(SpmmArgs a0, Segs segs, int n_tb) {
  static_assert(!MIX || SPLIT, "two split counts are a K split");
  using C = PrefillCfg<NT>;
  __shared__ __attribute__((aligned(16))) uint16_t xs_a[64 * C::PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t xs_b[64 * C::PITCH];
  __shared__ __attribute__((aligned(16))) uint32_t ms_a[128];
  __shared__ __attribute__((aligned(16))) uint32_t ms_b[128];
  uint16_t* const xs[2] = {xs_a, xs_b};   // separate LDS objects: loads into one tile never
  uint32_t* const ms[2] = {ms_a, ms_b};   // hold up reads of the other
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrb = a0.rows / 64;
  const int n_tr = a0.n_tiles * nrb;              // row blocks over all weights of a group
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd = gridDim.x / 8;
  const int tok_w = wave * C::TW;
  const SpmmArgs& a = a0;                         // fields shared by every weight (per-tile order below)

  // Per-tile counts: every tile runs the same number of K-block steps (its
  // kept entries per row are fixed by t_s), but a 2:4 block gathers 64 X rows
  // against a dense block's 32, so a tile costs n_dense_blocks + 2 n_24_blocks.
  // When workgroups take more than one item each, every token block takes the
  // tiles largest cost first (ties by tile), alternating direction from one
  // token block to the next, so a slot that meets a costly tile in one token
  // block meets a cheap one in the next.  With one item per workgroup the
  // order cannot change the finish time and is skipped; tiles past the
  // order's LDS room keep their natural order.  The costs are staged in the
  // second X buffer, which no item has used yet.
  // With fewer items than the grid holds, each item's K range is split over
  // `splits` workgroups (consecutive item numbers, so on one XCD); the
  // partial sums meet through the workspace as in the split decode.
  const int splits = SPLIT ? a.splits : 1;
  const int n_items = n_tb * n_tr;
  const int items = n_items * splits;
  __shared__ int s_last;
  constexpr int kMaxOrdered = 1024;
  __shared__ int16_t order[kMaxOrdered];
  const bool ordered = a.tiles != nullptr && a.n_tiles <= kMaxOrdered && items > (int)gridDim.x;
  if (ordered) {
    int16_t* cost = reinterpret_cast<int16_t*>(xs[1]);
    for (int t = threadIdx.x; t < a.n_tiles; t += 256) {
      const TileK k = tile_k(a, t);
      cost[t] = (int16_t)(k.nbd + 2 * k.nbs);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < a.n_tiles; t += 256) {
      const int c = cost[t];
      int r = 0;
      for (int u = 0; u < a.n_tiles; ++u) {
        const int cu = cost[u];
        r += (cu > c) | ((cu == c) & (u < t));
      }
      order[r] = (int16_t)t;
    }
    __syncthreads();
  }

  // Pieces of this XCD: with one split count, pieces (item, split) of the
  // XCD's contiguous range; with two (MIX), the XCD's items in order,
  // the first wx whole and the rest in two halves, wx chosen so that the XCD
  // has one piece per workgroup: the whole items take the first slots of
  // their compute units and halves the second ones.  Partial sums are kept
  // for the halved items only, numbered over all XCDs (m_h0: those of the
  // XCDs before this one; n_half: all of them).  Its own instantiation
  // (MIX), so that the one-count split keeps its code.
  constexpr bool mix = MIX;
  int i_lo, i_hi, m_lo = 0, m_wx = 0, m_h0 = 0, n_half = 0;
  if constexpr (mix) {
    for (int x = 0; x < 8; ++x) {
      const int lo = (int)((int64_t)x * n_items / 8), nx = (int)((int64_t)(x + 1) * n_items / 8) - lo;
      const int wx = min(nx, max(0, 2 * nx - per_xcd));
      if (x < xcd) m_h0 += nx - wx;
      if (x == xcd) {
        m_lo = lo;
        m_wx = wx;
        i_lo = 0;
        i_hi = wx + 2 * (nx - wx);
      }
      n_half += nx - wx;
    }
  } else {
    i_lo = (int)((int64_t)xcd * items / 8);
    i_hi = (int)((int64_t)(xcd + 1) * items / 8);
  }
  for (int it = i_lo + slot; it < i_hi; it += per_xcd) {
    {
      int split = SPLIT ? it % splits : 0, item = SPLIT ? it / splits : it, nsp = splits;
      int pidx = item, pstride = n_items;          // partial sums: plane split, entry pidx of pstride
      if constexpr (mix) {
        const bool whole = it < m_wx;
        item = m_lo + (whole ? it : m_wx + (it - m_wx) / 2);
        split = whole ? 0 : (it - m_wx) % 2;
        nsp = whole ? 1 : 2;
        pidx = m_h0 + (whole ? 0 : (it - m_wx) / 2);
        pstride = n_half;
      }
      // items in groups of a.tb_group token blocks, row-block major inside a
      // group (one token block per group: token-block major)
      int tb, gtrb;
      {
        const int G = a.tb_group, full = n_tb / G * G;
        if (item < full * n_tr) {
          const int rem = item % (n_tr * G);
          gtrb = rem / G;
          tb = item / (n_tr * G) * G + rem % G;
        } else {
          const int r2 = item - full * n_tr, gt = n_tb - full;
          gtrb = r2 / gt;
          tb = full + r2 % gt;
        }
      }
      SpmmArgs a = a0;
      int trb0, row0;
      select_seg(segs, gtrb, a, trb0, row0);
      const BufRes res = make_res(a);
      const int trb = gtrb - trb0;
      const int n0 = tb * NT;
      int t = trb / nrb;
      const int rb = trb % nrb;
      if (ordered) t = order[(tb & 1) ? a.n_tiles - 1 - t : t];
      f32x16 acc[2][C::NTB];
      for (int r = 0; r < 2; ++r)
        for (int j = 0; j < C::NTB; ++j)
          for (int e = 0; e < 16; ++e) acc[r][j][e] = 0.f;

      const TileK tk = tile_k(a, t);
      KShare ks = SPLIT ? k_share(tk, split, nsp) : KShare{tk.kd0, tk.nbd, tk.ks0, tk.nbs, 0, 0};
      if (a.stagger) {
        // Items start their K loops at staggered blocks: tile t at t/n_tiles
        // of its range, so that tiles whose index lists walk X in the same
        // order do not read the same rows at the same time, plus (3 tb mod
        // 8)/8 for token block tb, so that the XCDs, which work on different
        // token blocks at once, reach a tile's packed values at different
        // times (the first read comes from HBM, the later ones from the
        // last-level cache).  The order depends on (tile, token block) only,
        // so every schedule of the items gives the same bits.
        const int64_t tq = (3 * tb) & 7;
        ks.rd = ks.nd ? (int)(((int64_t)t * ks.nd / a.n_tiles + tq * ks.nd / 8) % ks.nd) : 0;
        ks.rs = ks.ns ? (int)(((int64_t)t * ks.ns / a.n_tiles + tq * ks.ns / 8) % ks.ns) : 0;
      }
      const bool tail = n0 + NT > a.batch;
      bool direct = false;
      if constexpr (NT == 256) direct = a.x_lds;
      if (direct) {
        if constexpr (NT == 256) {
          if (!tail) prefill_body_lds<NT, 0>(a, res, xs[0], xs[1], ms[0], ms[1], ks, rb, n0, acc);
          else if (a.batch & 1) prefill_body_lds<NT, 2>(a, res, xs[0], xs[1], ms[0], ms[1], ks, rb, n0, acc);
          else prefill_body_lds<NT, 1>(a, res, xs[0], xs[1], ms[0], ms[1], ks, rb, n0, acc);
        }
      } else if (a.x_vec && !tail) {
        prefill_body_staged<NT, true>(a, res, xs[0], xs[1], ms[0], ms[1], ks, rb, n0, acc);
      } else {
        prefill_body_staged<NT, false>(a, res, xs[0], xs[1], ms[0], ms[1], ks, rb, n0, acc);
      }
      __syncthreads();

      if (SPLIT && (!MIX || nsp > 1)) {
        // Partials part[split][item][NACC][thread] (the accumulators' own
        // register order, lanes adjacent) through agent-scope
        // (device-coherent) stores and loads; each workgroup waits for its
        // stores before it counts itself in, and the last to arrive adds the
        // partials in split order and puts the counter back to 0.
        constexpr int NACC = 2 * C::NTB * 16;
        unsigned* ctr = reinterpret_cast<unsigned*>(reinterpret_cast<char*>(a.ws) - hinm::kWsCounterBytes) + item;
        float* my = a.ws + ((int64_t)split * pstride + pidx) * 256 * NACC + threadIdx.x;
        for (int r = 0; r < 2; ++r)
          for (int j = 0; j < C::NTB; ++j)
            for (int e = 0; e < 16; ++e)
              __hip_atomic_store(my + ((r * C::NTB + j) * 16 + e) * 256, acc[r][j][e], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) s_last = arrive(ctr, nsp);
        __syncthreads();
        if (!s_last) continue;
        // per accumulator: up to SV splits' partials in flight at once,
        // added in split order from zero
        constexpr int SV = 4;
        const int64_t sstride = (int64_t)pstride * 256 * NACC;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int j = 0; j < C::NTB; ++j) {
            const float* pg = a.ws + (int64_t)pidx * 256 * NACC + (r * C::NTB + j) * 16 * 256 + threadIdx.x;
            float sum[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) sum[e] = 0.f;
            for (int sp0 = 0; sp0 < nsp; sp0 += SV) {
              float v[SV][16];
#pragma unroll
              for (int u = 0; u < SV; ++u) {
                if (sp0 + u < nsp) {
#pragma unroll
                  for (int e = 0; e < 16; ++e)
                    v[u][e] = __hip_atomic_load(pg + (sp0 + u) * sstride + e * 256, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                } else {
#pragma unroll
                  for (int e = 0; e < 16; ++e) v[u][e] = 0.f;
                }
              }
#pragma unroll
              for (int u = 0; u < SV; ++u)
#pragma unroll
                for (int e = 0; e < 16; ++e) sum[e] = (sp0 + u < nsp) ? sum[e] + v[u][e] : sum[e];
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[r][j][e] = sum[e];
          }
      }

      // epilogue: acc[r][j][e] is row 32r + 8(e/4) + 4(lane/32) + e%4, token tok_w + 32j + lane%32.
      uint16_t* ys = xs[0];
      for (int r = 0; r < 2; ++r)
        for (int j = 0; j < C::NTB; ++j)
          for (int e = 0; e < 16; ++e)
            ys[(32 * r + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * C::PITCH + tok_w + 32 * j + (lane & 31)] =
                bf16_rne(acc[r][j][e]);
      __syncthreads();
      for (int q = threadIdx.x; q < 64 * C::CPR; q += 256) {
        const int r = q / C::CPR, c = q % C::CPR;
        const int n = n0 + 8 * c;
        if (n >= a.batch) continue;
        const int64_t yr = y_row(a, (int64_t)t * a.rows + rb * 64 + r);
        if (yr < 0) continue;
        uint16_t* dst = a.y + yr * a.ldy + n;
        const uint16_t* src = ys + r * C::PITCH + 8 * c;
        if (a.y_vec && n + 8 <= a.batch) {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        } else {
          for (int e = 0; e < 8 && n + e < a.batch; ++e) dst[e] = src[e];
        }
      }
      __syncthreads();   // ys aliases the X tile of the next item
    }
  }
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

static bool segs_y_vec(const Segs& sg) {
  for (int g = 0; g < sg.n; ++g)
    if (!hinm::aligned(sg.s[g].y, 16) || sg.s[g].ldy % 8 != 0) return false;
  return true;
}

// The packed buffers of either layout: the uniform one (tiles == NULL, block
// counts from the plan) or the per-tile one (a device tile table).
struct PackedView {
  const void* val_dense;
  const int32_t* idx_dense;
  const void* val_24;
  const uint64_t* meta_24;
  const int32_t* idx_24;
  const int32_t* tiles;
  int kd_total, ks_total;
  uint32_t flags;       // HINM_PACKED_* (every weight of a group)
};

// `p` has been validated by the caller (for the per-tile layout it carries
// the largest per-tile pads and the buffer totals).
// The prefill and split decode kernels address X and the packed buffers with
// 32-bit buffer offsets and gather with a 24-bit multiply (row index and row
// pitch in bytes both below 2^24).
static bool fits32(const hinm_plan_t& p, int64_t ldx, int64_t batch) {
  const int64_t lim = (int64_t)1 << 31, lim24 = (int64_t)1 << 24;
  const int64_t xbytes = ((int64_t)(p.cin - 1) * ldx + batch) * 2;
  return xbytes < lim && ldx * 2 < lim24 && p.cin <= lim24 && p.bytes_val_dense < lim && p.bytes_val_24 < lim &&
         p.bytes_idx_dense < lim && p.bytes_idx_24 < lim && p.bytes_meta_24 < lim;
}

// segs: NULL, or the weights of a group (then p is their combined shape: cout
// and n_tiles summed, pads and buffer sizes the largest; packed_v, y_bf16 and
// ldy are the first weight's); only the split decode and prefill kernels
// take a group, and the caller checks that one of them runs.
static int spmm_impl(const hinm_plan_t& p, const PackedView& packed_v, const void* x_bf16, int64_t batch,
                     int64_t ldx, void* y_bf16, int64_t ldy, const int32_t* out_rows, void* workspace,
                     size_t workspace_bytes, void* stream_, const Segs* segs = nullptr) {
  const PackedView* packed = &packed_v;
  int st = HINM_OK;
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
  if (!segs)   // a group's weights are checked one by one by its entry point
    for (const Buf& b : bufs) {
      if (b.bytes > 0 && !b.ptr) return fail(HINM_EINVAL, "%s is NULL but holds %lld bytes", b.name, (long long)b.bytes);
      if (b.ptr && !hinm::aligned(b.ptr, 16)) return fail(HINM_EALIGN, "%s is not 16-byte aligned", b.name);
    }
  hinm::SpmmShape sh = hinm::spmm_shape(&p, batch);
  if (sh.ws_bytes > 0) {
    if (!workspace || workspace_bytes < (size_t)sh.ws_bytes)
      return fail(HINM_EWORKSPACE, "spmm workspace of %zu bytes given, %lld needed", workspace_bytes,
                  (long long)sh.ws_bytes);
    if (!hinm::aligned(workspace, 256)) return fail(HINM_EALIGN, "workspace is not 256-byte aligned");
  }
  st = hinm::ensure_device();
  if (st) return st;
  if (sh.path == hinm::kPathGeneric && (int64_t)p.n_tiles * sh.n_rblocks > 65535)
    return fail(HINM_ESHAPE, "too many row blocks for one launch");
  if (sh.path == hinm::kPathDecode && sh.n_tblocks > 65535) return fail(HINM_ESHAPE, "batch too large");

  SpmmArgs a;
  a.val_d = static_cast<const uint16_t*>(packed->val_dense);
  a.idx_d = packed->idx_dense;
  a.val_s = static_cast<const uint16_t*>(packed->val_24);
  a.meta = packed->meta_24;
  a.idx_s = packed->idx_24;
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.y = static_cast<uint16_t*>(y_bf16);
  a.ws = sh.ws_bytes > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + sh.ws_counter_bytes) : nullptr;
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
  // At 256-token blocks X rows go straight into LDS, whatever their
  // alignment (the register-staged gather stays selectable for comparison);
  // at 128-token blocks the register-staged gather measured faster.
  a.x_lds = hinm::option(HINM_OPT_PREFILL_PATH) == 0;
  a.y_vec = hinm::aligned(y_bf16, 16) && (ldy % 8 == 0);
  a.n_tiles = p.n_tiles;
  a.out_rows = out_rows;
  a.tiles = packed->tiles;
  a.kd_total = packed->kd_total;
  a.ks_total = packed->ks_total;
  a.part_rows = p.cout;
  a.tb_group = hinm::option(HINM_OPT_PREFILL_TB_GROUP) > 0 ? (int)hinm::option(HINM_OPT_PREFILL_TB_GROUP)
                                                            : ((packed->flags & HINM_PACKED_WINDOWED) ? 2 : 1);
  a.stagger = hinm::option(HINM_OPT_PREFILL_STAGGER) == 0;
  Segs one;
  one.n = 0;
  if (segs) a.y_vec = a.y_vec && segs_y_vec(*segs);
  const Segs& sg = segs ? *segs : one;

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  // The prefill and split decode kernels address X and the packed buffers
  // with 32-bit buffer offsets and gather with a 24-bit multiply (row index
  // and row pitch in bytes both below 2^24); beyond those ranges kernels
  // with 64-bit addressing take over (the generic kernel without a K split,
  // or the 16-row decode kernel; neither needs a workspace).
  const bool f32 = fits32(p, ldx, batch);
  if (sh.path == hinm::kPathDecodeSplit && !f32) {
    sh.path = hinm::kPathDecode;
    sh.splits = 1;
    a.splits = 1;
  }
  if (packed->tiles && !((sh.path == hinm::kPathPrefill || sh.path == hinm::kPathDecodeSplit) && f32))
    return fail(HINM_ESHAPE, "the per-tile layout needs tile_rows %% 64 == 0 and buffers below 2^31 bytes");
  if (segs && !((sh.path == hinm::kPathPrefill || sh.path == hinm::kPathDecodeSplit) && f32))
    return fail(HINM_ESHAPE, "internal: a group of weights needs the split decode or prefill kernel");
  if (sh.path == hinm::kPathPrefill) {
    if (!f32) {
      sh.path = hinm::kPathGeneric;
      sh.nt = 64;
      sh.n_tblocks = (int)((batch + 63) / 64);
      sh.splits = 1;
      a.splits = 1;
      sh.split_mix = false;
    }
  }
  if (sh.path == hinm::kPathDecodeSplit) {
    const bool fast = a.x_vec && (batch % sh.nt == 0);
    unsigned* counters = static_cast<unsigned*>(workspace);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + sh.ws_counter_bytes);
    // 16 tokens: 24 blocks a round (48 KB of LDS), 2 gather waves; 32 and
    // 64 tokens: 96 KB rounds (24 / 12 blocks) with 4 gather waves.
    // the first split_rows row blocks take sh.splits workgroups, the rest twice as many
    const int64_t nrb_all = (int64_t)p.n_tiles * (p.tile_rows / 64);
    const dim3 grid((unsigned)(sh.split_rows * sh.splits + (nrb_all - sh.split_rows) * 2 * sh.splits), sh.n_tblocks),
        b6(384), b8(512);
    // the arguments the first loads depend on, preloaded into SGPRs (a group
    // takes them from its segment table, and preloads its weight boundaries)
    const int32_t* kid = a.idx_d;
    const int32_t* kis = a.idx_s;
    const int32_t* ktl = a.tiles;
    const int kdt = a.kd_total, kst = a.ks_total, knd = a.nkb_d, kns = a.nkb_s, krw = a.rows, ksp = sh.splits;
    const int kr1 = (int)sh.split_rows;
    // a group's weight boundaries in concatenated row blocks, INT_MAX past the last weight
    int gb[kMaxSeg];
    for (int g = 0; g < kMaxSeg; ++g) gb[g] = segs && g < sg.n ? sg.s[g].trb0 : INT_MAX;
    const DecArgs da{a.val_d, a.val_s, a.meta, a.x, a.y, a.out_rows, a.ldy, (int)a.ldx, a.batch, a.cin, a.cout,
                     a.part_rows, sh.n_tblocks};
#define HINM_DECODE5(NT_, MB_, F_, NG_, ONE_, BLK_)                                                                   \
  do {                                                                                                              \
    if (segs)                                                                                                       \
      hipLaunchKernelGGL((decode5_group_kernel<NT_, MB_, F_, NG_, ONE_>), grid, BLK_, 0, stream, krw, ksp, kr1,      \
                         gb[1], gb[2], gb[3], gb[4], gb[5], gb[6], gb[7], a, sg, sh.n_tblocks, part, counters);     \
    else                                                                                                            \
      hipLaunchKernelGGL((decode5_kernel<NT_, MB_, F_, NG_, ONE_>), grid, BLK_, 0, stream, kid, kis, ktl, kdt, kst, \
                         knd, kns, krw, ksp, kr1, da, part, counters);                                             \
  } while (0)
    // 32 and 64 tokens: 96 KB rounds and four gather waves (one workgroup
    // per compute unit); at 32 tokens, when a launch has more workgroups
    // than compute units, 48 KB rounds and two gather waves instead (130
    // VGPRs), so that two workgroups share a unit and all of them run at
    // once.
    const int key = batch == 1 ? 1 : sh.nt * 2 + (fast ? 1 : 0) + (sh.nt > 16 && sh.two_per_cu ? 1000 : 0);
    switch (key) {
      case 1: HINM_DECODE5(16, 24, false, 2, true, b6); break;
      case 33: HINM_DECODE5(16, 24, true, 2, false, b6); break;
      case 32: HINM_DECODE5(16, 24, false, 2, false, b6); break;
      case 65: HINM_DECODE5(32, 24, true, 4, false, b8); break;
      case 64: HINM_DECODE5(32, 24, false, 4, false, b8); break;
      case 1065: HINM_DECODE5(32, 12, true, 2, false, b6); break;
      case 1064: HINM_DECODE5(32, 12, false, 2, false, b6); break;
      case 129: HINM_DECODE5(64, 12, true, 4, false, b8); break;
      default: HINM_DECODE5(64, 12, false, 4, false, b8); break;
    }
#undef HINM_DECODE5
  } else if (sh.path == hinm::kPathDecode) {
    const dim3 grid(p.n_tiles * (p.tile_rows / 16), sh.n_tblocks), block(kDecWaves * 64);
    const bool fast = a.x_vec && (batch % sh.nt == 0);
    if (sh.nt == 16) {
      if (fast) hipLaunchKernelGGL((decode3_kernel<16, 12, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode3_kernel<16, 12, false>), grid, block, 0, stream, a);
    } else if (sh.nt == 32) {
      if (fast) hipLaunchKernelGGL((decode3_kernel<32, 6, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode3_kernel<32, 6, false>), grid, block, 0, stream, a);
    } else {
      if (fast) hipLaunchKernelGGL((decode3_kernel<64, 3, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode3_kernel<64, 3, false>), grid, block, 0, stream, a);
    }
  } else if (sh.path == hinm::kPathPrefill) {
    // persistent grid: 8 XCDs x (32 CUs x 2 workgroups), never more than the work items.
    const int items = p.n_tiles * (p.tile_rows / 64) * sh.n_tblocks * sh.splits;
    const int per_xcd = hinm::option(HINM_OPT_PREFILL_PER_XCD) > 0 ? (int)hinm::option(HINM_OPT_PREFILL_PER_XCD) : 64;
    const int nwg = 8 * std::min(per_xcd, (items + 7) / 8);
    // the K-split epilogue is a separate instantiation, so the unsplit
    // kernel keeps its registers
    if (sh.nt == 256) {
      if (sh.splits > 1) hipLaunchKernelGGL((prefill_kernel<256, true>), dim3(nwg), dim3(256), 0, stream, a, sg, sh.n_tblocks);
      else hipLaunchKernelGGL((prefill_kernel<256, false>), dim3(nwg), dim3(256), 0, stream, a, sg, sh.n_tblocks);
    } else {
      if (sh.split_mix) hipLaunchKernelGGL((prefill_kernel<128, true, true>), dim3(nwg), dim3(256), 0, stream, a, sg, sh.n_tblocks);
      else if (sh.splits > 1) hipLaunchKernelGGL((prefill_kernel<128, true>), dim3(nwg), dim3(256), 0, stream, a, sg, sh.n_tblocks);
      else hipLaunchKernelGGL((prefill_kernel<128, false>), dim3(nwg), dim3(256), 0, stream, a, sg, sh.n_tblocks);
    }
  } else {
    const dim3 grid(sh.n_tblocks, p.n_tiles * sh.n_rblocks, sh.splits), block(kWaves * 64);
    switch (sh.nt) {
      case 16: hipLaunchKernelGGL(spmm_kernel<16>, grid, block, 0, stream, a); break;
      case 32: hipLaunchKernelGGL(spmm_kernel<32>, grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL(spmm_kernel<64>, grid, block, 0, stream, a); break;
    }
    if (sh.splits > 1) {
      const int64_t n = (int64_t)p.cout * batch;
      hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.ws, sh.splits,
                         p.cout, (int)batch, a.batch_pad16, a.y, ldy, a.out_rows);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HINM_EHIP, "spmm launch: %s", hipGetErrorString(e));
  return HINM_OK;
}

static PackedView uniform_view(const hinm_packed_t& k) {
  const hinm_plan_t& p = k.plan;
  return {k.val_dense, k.idx_dense, k.val_24, k.meta_24, k.idx_24, nullptr,
          p.n_tiles * (p.n_dense_pad / HINM_KB_DENSE), p.n_tiles * (p.n_24_pad / HINM_KB_24), k.flags};
}

extern "C" int hinm_spmm(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx, void* y_bf16,
                         int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  hinm::clear_error();
  if (!packed) return fail(HINM_EINVAL, "packed is NULL");
  int st = hinm::check_plan(&packed->plan);
  if (st) return st;
  return spmm_impl(packed->plan, uniform_view(*packed), x_bf16, batch, ldx, y_bf16, ldy, nullptr, workspace,
                   workspace_bytes, stream);
}

extern "C" int hinm_spmm_tiles(const hinm_tpacked_t* packed, const void* x_bf16, int64_t batch, int64_t ldx,
                               void* y_bf16, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  hinm::clear_error();
  if (!packed) return fail(HINM_EINVAL, "packed is NULL");
  int st = hinm::check_tplan(&packed->plan);
  if (st) return st;
  if (!packed->tiles) return fail(HINM_EINVAL, "the tile table is NULL");
  if (!hinm::aligned(packed->tiles, 4)) return fail(HINM_EALIGN, "the tile table is not 4-byte aligned");
  const hinm_tplan_t& p = packed->plan;
  const PackedView v = {packed->val_dense, packed->idx_dense, packed->val_24, packed->meta_24, packed->idx_24,
                        packed->tiles, p.dense_blocks, p.blocks_24, 0u};
  return spmm_impl(hinm::shape_plan(p), v, x_bf16, batch, ldx, y_bf16, ldy, nullptr, workspace, workspace_bytes,
                   stream);
}

extern "C" int hinm_spmm_rows(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx,
                              void* y_bf16, int64_t ldy, const int32_t* out_rows, void* workspace,
                              size_t workspace_bytes, void* stream) {
  hinm::clear_error();
  if (!packed) return fail(HINM_EINVAL, "packed is NULL");
  int st = hinm::check_plan(&packed->plan);
  if (st) return st;
  if (!out_rows) return fail(HINM_EINVAL, "out_rows is NULL");
  if (!hinm::aligned(out_rows, 4)) return fail(HINM_EALIGN, "out_rows is not 4-byte aligned");
  return spmm_impl(packed->plan, uniform_view(*packed), x_bf16, batch, ldx, y_bf16, ldy, out_rows, workspace,
                   workspace_bytes, stream);
}

// A group of packed weights for hinm_spmm_group: checked one by one, with
// their combined shape (cout and n_tiles summed, pads and buffer sizes the
// largest), which decides the launch shape of the one launch.
static int group_shape(int n, const hinm_packed_t* const* packed, hinm_plan_t* comb) {
  if (n < 1 || n > kMaxSeg) return fail(HINM_EINVAL, "n=%d weights; 1 to %d are supported", n, kMaxSeg);
  if (!packed) return fail(HINM_EINVAL, "packed is NULL");
  int64_t cout = 0, tiles = 0;
  for (int g = 0; g < n; ++g) {
    if (!packed[g]) return fail(HINM_EINVAL, "packed[%d] is NULL", g);
    const hinm_plan_t& q = packed[g]->plan;
    int st = hinm::check_plan(&q);
    if (st) return st;
    if (q.cin != packed[0]->plan.cin || q.tile_rows != packed[0]->plan.tile_rows)
      return fail(HINM_ESHAPE, "packed[%d] has cin=%d, tile_rows=%d; a group needs those of packed[0] (%d, %d)", g, q.cin,
                  q.tile_rows, packed[0]->plan.cin, packed[0]->plan.tile_rows);
    const hinm_packed_t& k = *packed[g];
    struct Buf { const void* ptr; int64_t bytes; const char* name; } bufs[5] = {
        {k.val_dense, q.bytes_val_dense, "val_dense"}, {k.idx_dense, q.bytes_idx_dense, "idx_dense"},
        {k.val_24, q.bytes_val_24, "val_24"}, {k.meta_24, q.bytes_meta_24, "meta_24"}, {k.idx_24, q.bytes_idx_24, "idx_24"}};
    for (const Buf& b : bufs) {
      if (b.bytes > 0 && !b.ptr) return fail(HINM_EINVAL, "packed[%d]: %s is NULL but holds %lld bytes", g, b.name, (long long)b.bytes);
      if (b.ptr && !hinm::aligned(b.ptr, 16)) return fail(HINM_EALIGN, "packed[%d]: %s is not 16-byte aligned", g, b.name);
    }
    cout += q.cout;
    tiles += q.n_tiles;
  }
  if (cout > INT32_MAX) return fail(HINM_ESHAPE, "the group's rows exceed 2^31");
  hinm_plan_t c = packed[0]->plan;
  for (int g = 1; g < n; ++g) {
    const hinm_plan_t& q = packed[g]->plan;
    c.n_dense_pad = std::max(c.n_dense_pad, q.n_dense_pad);
    c.n_24_pad = std::max(c.n_24_pad, q.n_24_pad);
    c.bytes_val_dense = std::max(c.bytes_val_dense, q.bytes_val_dense);
    c.bytes_idx_dense = std::max(c.bytes_idx_dense, q.bytes_idx_dense);
    c.bytes_val_24 = std::max(c.bytes_val_24, q.bytes_val_24);
    c.bytes_meta_24 = std::max(c.bytes_meta_24, q.bytes_meta_24);
    c.bytes_idx_24 = std::max(c.bytes_idx_24, q.bytes_idx_24);
  }
  c.cout = (int32_t)cout;
  c.n_tiles = (int32_t)tiles;
  *comb = c;
  return HINM_OK;
}

// One launch for the whole group when the split decode or the prefill kernel
// runs it; otherwise one launch per weight.
static bool group_together(int n, const hinm_plan_t& comb, int64_t batch, int64_t ldx) {
  if (n < 2 || comb.tile_rows % 64 != 0) return false;
  const hinm::SpmmShape sh = hinm::spmm_shape(&comb, batch);
  return (sh.path == hinm::kPathPrefill || sh.path == hinm::kPathDecodeSplit) && fits32(comb, ldx, batch);
}

extern "C" int hinm_spmm_group_workspace_bytes(int n, const hinm_packed_t* const* packed, int64_t batch,
                                               size_t* bytes) {
  hinm::clear_error();
  hinm_plan_t comb;
  int st = group_shape(n, packed, &comb);
  if (st) return st;
  if (!bytes) return fail(HINM_EINVAL, "bytes is NULL");
  if (batch < 0) return fail(HINM_ESHAPE, "batch=%lld is negative", (long long)batch);
  // enough for either way of running it (one launch, or one per weight)
  int64_t need = 0;
  if (batch > 0) {
    need = n > 1 && comb.tile_rows % 64 == 0 ? hinm::spmm_shape(&comb, batch).ws_bytes : 0;
    for (int g = 0; g < n; ++g) need = std::max(need, hinm::spmm_shape(&packed[g]->plan, batch).ws_bytes);
  }
  *bytes = (size_t)need;
  return HINM_OK;
}

extern "C" int hinm_spmm_group(int n, const hinm_packed_t* const* packed, const void* x_bf16, int64_t batch,
                               int64_t ldx, void* const* y_bf16, const int64_t* ldy, void* workspace,
                               size_t workspace_bytes, void* stream) {
  hinm::clear_error();
  hinm_plan_t comb;
  int st = group_shape(n, packed, &comb);
  if (st) return st;
  if (!y_bf16 || !ldy) return fail(HINM_EINVAL, "y and ldy must be non-NULL");
  for (int g = 0; g < n; ++g) {
    if (ldy[g] < batch) return fail(HINM_ESHAPE, "ldy[%d]=%lld is below batch=%lld", g, (long long)ldy[g], (long long)batch);
    if (batch > 0 && (!y_bf16[g] || !hinm::aligned(y_bf16[g], 2)))
      return fail(y_bf16[g] ? HINM_EALIGN : HINM_EINVAL, "y[%d] must be non-NULL and 2-byte aligned", g);
  }
  if (!group_together(n, comb, batch, ldx)) {
    for (int g = 0; g < n; ++g) {
      st = spmm_impl(packed[g]->plan, uniform_view(*packed[g]), x_bf16, batch, ldx, y_bf16[g], ldy[g], nullptr,
                     workspace, workspace_bytes, stream);
      if (st) return st;
    }
    return HINM_OK;
  }
  Segs sg;
  sg.n = n;
  int trb = 0, row = 0;
  for (int g = 0; g < n; ++g) {
    const hinm_packed_t& k = *packed[g];
    const hinm_plan_t& q = k.plan;
    Seg& S = sg.s[g];
    S.val_d = static_cast<const uint16_t*>(k.val_dense);
    S.idx_d = k.idx_dense;
    S.val_s = static_cast<const uint16_t*>(k.val_24);
    S.meta = k.meta_24;
    S.idx_s = k.idx_24;
    S.y = static_cast<uint16_t*>(y_bf16[g]);
    S.ldy = ldy[g];
    S.cout = q.cout;
    S.n_tiles = q.n_tiles;
    S.nkb_d = q.n_dense_pad / HINM_KB_DENSE;
    S.nkb_s = q.n_24_pad / HINM_KB_24;
    S.kd_total = q.n_tiles * S.nkb_d;
    S.ks_total = q.n_tiles * S.nkb_s;
    S.trb0 = trb;
    S.row0 = row;
    trb += q.n_tiles * (q.tile_rows / 64);
    row += q.cout;
  }
  PackedView v0 = uniform_view(*packed[0]);
  for (int g = 1; g < n; ++g) v0.flags &= packed[g]->flags;
  return spmm_impl(comb, v0, x_bf16, batch, ldx, y_bf16[0], ldy[0], nullptr, workspace, workspace_bytes, stream, &sg);
}

// ---------------------------------------------------------------------------
// Allocation-free product: the scratch of the split reduction (arrival
// counters, then partial sums) lives in this file-scope device array, one
// copy per device, instead of in a caller workspace.  In host code the name
// `scratch` is only a stand-in; kernels get the device address taken with
// hipGetSymbolAddress.
// ---------------------------------------------------------------------------
static_assert(hinm::kWsCounterBytes == 65536, "the scratch size counts 64 KiB of arrival counters");
static __device__ __align__(256) unsigned char scratch[HINM_NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void zero_words_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once set up

// The device address of the current device's scratch array.  The first call
// on a device takes the address (with that device current) and clears the
// arrival counters with a fill kernel on `stream`; every product leaves them
// at zero again.
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HINM_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HINM_EDEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(HINM_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    constexpr int n = (int)(hinm::kWsCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<unsigned*>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HINM_EHIP, "clearing the scratch counters: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HINM_OK;
}

}  // namespace

extern "C" int hinm_spmm_noalloc(const hinm_packed_t* packed, const void* x_bf16, int64_t batch, int64_t ldx,
                                 void* y_bf16, int64_t ldy, void* stream) {
  hinm::clear_error();
  if (!packed) return fail(HINM_EINVAL, "packed is NULL");
  int st = hinm::check_plan(&packed->plan);
  if (st) return st;
  if (batch <= 0)   // spmm_impl's own checks (negative batch, no-op at 0)
    return spmm_impl(packed->plan, uniform_view(*packed), x_bf16, batch, ldx, y_bf16, ldy, nullptr, nullptr, 0,
                     stream);
  const hinm::SpmmShape sh = hinm::spmm_shape(&packed->plan, batch);
  if (sh.ws_bytes > (int64_t)HINM_NOALLOC_SCRATCH_BYTES)
    return fail(HINM_EWORKSPACE,
                "this product needs %lld bytes of scratch, more than the %lld the allocation-free entry point "
                "holds; call hinm_spmm with a workspace",
                (long long)sh.ws_bytes, (long long)HINM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (sh.ws_bytes > 0) {
    st = hinm::ensure_device();
    if (st) return st;
    st = scratch_address(reinterpret_cast<hipStream_t>(stream), &ws);
    if (st) return st;
  }
  return spmm_impl(packed->plan, uniform_view(*packed), x_bf16, batch, ldx, y_bf16, ldy, nullptr, ws,
                   sh.ws_bytes > 0 ? (size_t)HINM_NOALLOC_SCRATCH_BYTES : 0, stream);
}
