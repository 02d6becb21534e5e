// Probe of the gfx950 structured-sparse MFMA (SMFMAC) operand layouts that the
// packed HiNM format is built on (test infrastructure, not part of libhinm).
//
// The 2:4 region keeps two of every four consecutive input positions (the 2:4
// structured-sparsity article, section 3: exactly two per group, two bits of
// position per kept element); the packed format stores, per row and group g,
// the kept values in position order and the nibble i0 | i1 << 2 at bits 4g of
// a 64-bit word.  One wave loads a block in that logical form into the lane
// layout the product kernels use and runs one SMFMAC:
//   16x16x64: lane l = 16 kc + i holds row i's compressed values 8kc..8kc+7,
//             index bits 16kc..16kc+15 of the row's word, and of column i the
//             positions 8kc..8kc+7 and 32+8kc..32+8kc+7; result row 4kc + e.
//   32x32x32: lane l = 32 kc + i holds row i's compressed values 8kc..8kc+7,
//             index bits 16kc..16kc+15, and of column i the positions
//             8kc..8kc+7 and 16+8kc..16+8kc+7; result row 8(e/4) + 4kc + e%4.
// If that layout were wrong, the result would differ from the plain 2:4
// product computed on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ inline __bf16 as_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

// A [16][32] compressed bf16 bits, meta [16], B [64][16] bf16 bits, D [16][16] fp32.
__global__ __launch_bounds__(64) void probe16_kernel(const uint16_t* A, const uint64_t* meta, const uint16_t* B,
                                                     float* D) {
  const int l = threadIdx.x, kc = l >> 4, i = l & 15;
  bf16x8_t a;
  bf16x16_t b;
  for (int e = 0; e < 8; ++e) {
    a[e] = as_bf16(A[i * 32 + 8 * kc + e]);
    b[e] = as_bf16(B[(8 * kc + e) * 16 + i]);
    b[8 + e] = as_bf16(B[(32 + 8 * kc + e) * 16 + i]);
  }
  const int idx = (int)((meta[i] >> (16 * kc)) & 0xffffull);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, acc, idx, 0, 0);
  for (int e = 0; e < 4; ++e) D[(4 * kc + e) * 16 + i] = acc[e];
}

// A [32][16] compressed bf16 bits, meta [32] (low 32 bits used), B [32][32], D [32][32].
__global__ __launch_bounds__(64) void probe32_kernel(const uint16_t* A, const uint64_t* meta, const uint16_t* B,
                                                     float* D) {
  const int l = threadIdx.x, kc = l >> 5, i = l & 31;
  bf16x8_t a;
  bf16x16_t b;
  for (int e = 0; e < 8; ++e) {
    a[e] = as_bf16(A[i * 16 + 8 * kc + e]);
    b[e] = as_bf16(B[(8 * kc + e) * 32 + i]);
    b[8 + e] = as_bf16(B[(16 + 8 * kc + e) * 32 + i]);
  }
  const int idx = (int)((meta[i] >> (16 * kc)) & 0xffffull);
  f32x16_t acc;
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  acc = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, acc, idx, 0, 0);
  for (int e = 0; e < 16; ++e) D[(8 * (e >> 2) + 4 * kc + (e & 3)) * 32 + i] = acc[e];
}

// Runs one probe (shape 16 or 32) on device buffers and waits for it; returns
// the HIP error code (0 on success).
extern "C" int smfmac_probe(int shape, const void* A, const void* meta, const void* B, void* D) {
  if (shape == 16)
    hipLaunchKernelGGL(probe16_kernel, dim3(1), dim3(64), 0, 0, (const uint16_t*)A, (const uint64_t*)meta,
                       (const uint16_t*)B, (float*)D);
  else if (shape == 32)
    hipLaunchKernelGGL(probe32_kernel, dim3(1), dim3(64), 0, 0, (const uint16_t*)A, (const uint64_t*)meta,
                       (const uint16_t*)B, (float*)D);
  else
    return (int)hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  return (int)hipDeviceSynchronize();
}
