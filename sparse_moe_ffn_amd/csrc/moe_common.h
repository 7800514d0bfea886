// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// bfloat16 is carried as its 16 raw bits.
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Two floats to packed bfloat16 (lo in the low half), round to nearest even,
// on the conversion instruction of gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }
// SiLU on the hardware exp2 and reciprocal (about 1e-7 relative error), for
// results that are rounded to bfloat16 anyway.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

// D = A(16x32) * B(32x16) + C on the matrix cores.  Lane l supplies row l%16
// of A and column l%16 of B, each over the 8 k-values of block l/16; lane l
// receives C rows 4*(l/16) .. +3 of column l%16.
__device__ __forceinline__ floatx4 mfma16x16x32(const uint4& a, const uint4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave-wide reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Map a linear workgroup id so that consecutive logical ids run on the same
// XCD.  Workgroups are dispatched round-robin over the 8 XCDs, so id b runs
// on XCD b % 8; the logical id returned keeps each XCD on one contiguous
// range of the logical order (neighbours share the XCD's L2).
__device__ __forceinline__ int xcd_swizzle(int b, int n) {
  constexpr int kXcd = 8;
  const int per = n / kXcd;          // full rounds
  const int full = per * kXcd;
  if (b >= full) return b;           // ragged last round keeps its order
  return (b % kXcd) * per + b / kXcd;
}

}  // namespace moe
