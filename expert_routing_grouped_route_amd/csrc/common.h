// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Rows per M-tile of the grouped GEMMs; the dispatch scan builds the
// per-expert M-tile prefix table in units of this.
constexpr int kBM = 256;
// Assignments handled per block of the dispatch count/rank kernels (minimum).
constexpr int kDispatchChunk = 256;
// Tokens per block of the router.
constexpr int kRouteTokens = 16;
// Top-k upper limit.
constexpr int kMaxK = 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}

__device__ __forceinline__ u32x4 ld_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores.  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with the 8 K-elements of group
// (l / 16); D comes back with column (l % 16), rows 4*(l/16) + 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16) * B(16x32) + C.  Lane l supplies row (l % 32) of A and column
// (l % 32) of B, each with the 8 K-elements of group (l / 32); D comes back
// with column (l % 32), value v at row 8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_times(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// silu(g) * u with the hardware reciprocal (1 ulp) in place of an IEEE
// division, for products that are rounded to bf16 next.  For large negative g
// the reciprocal of +inf is 0, so the result is a signed zero, as with the
// division.
__device__ __forceinline__ float silu_times_rcp(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 in one 32-bit word (lo in bits 0..15), rounded
// to nearest, ties to even, by the gfx950 packed convert (checked against the
// integer sequence u + 0x7FFF + ((u >> 16) & 1) on all 2^32 non-NaN inputs).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace moe
