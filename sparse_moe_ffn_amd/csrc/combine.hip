// Combine kernel: out[n] = sum_{j=0..k-1} y[n*k + j] (+ shared_y[n]).
//
// "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert", 逐步图 step 4
// and 易错点: a token's contributions from its k slots are added, never
// assigned.  Here every (token, slot) row of y was written exactly once by
// the down product, and each output element is summed by one thread in the
// fixed slot order (float32, rounded once), so the result does not depend on
// scheduling and no value atomics are used.
//
// bf16: a thread handles 8 consecutive columns (16-byte loads of each of the
// k rows; the k rows of a token are adjacent, so a workgroup streams one
// contiguous block of k*H values).  The loads of up to 8 slots are issued
// before any of them is added, so a token costs one memory latency instead
// of k; y is read once, so its loads are non-temporal.  fp32: one column
// per thread.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_bf16_kernel(
    const uint16_t* __restrict__ y, const uint16_t* __restrict__ ys, uint16_t* __restrict__ out,
    int H, int k) {
  const int n = blockIdx.x;
  const int h0 = (blockIdx.y * kCombineThreads + threadIdx.x) * 8;
  if (h0 >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const uint16_t* src = y + (int64_t)n * k * H + h0;
  constexpr int kBatch = 8;
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    u32x4_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (j0 + u < k) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + (int64_t)(j0 + u) * H));
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (j0 + u < k) {                                    // slot order
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(v[u][i] & 0xffffu));
          acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(v[u][i] >> 16));
        }
      }
    }
  }
  if (ys) {
    const uint4 v = *reinterpret_cast<const uint4*>(ys + (int64_t)n * H + h0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
      acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + (int64_t)n * H + h0) = o;
}

__global__ __launch_bounds__(kCombineThreads) void combine_f32_kernel(
    const float* __restrict__ y, const float* __restrict__ ys, float* __restrict__ out, int H, int k) {
  const int n = blockIdx.x;
  const int h = blockIdx.y * kCombineThreads + threadIdx.x;
  if (h >= H) return;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) acc += y[((int64_t)n * k + j) * H + h];
  if (ys) acc += ys[(int64_t)n * H + h];
  out[(int64_t)n * H + h] = acc;
}

hipError_t launch_combine(const void* y, const void* shared_y, void* out, int64_t N, int64_t H,
                          int64_t top_k, int32_t dtype, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (dtype == MOE_BF16) {
    const dim3 grid((unsigned)N, (unsigned)((H / 8 + kCombineThreads - 1) / kCombineThreads));
    hipLaunchKernelGGL(combine_bf16_kernel, grid, dim3(kCombineThreads), 0, s, (const uint16_t*)y,
                       (const uint16_t*)shared_y, (uint16_t*)out, (int)H, (int)top_k);
  } else {
    const dim3 grid((unsigned)N, (unsigned)((H + kCombineThreads - 1) / kCombineThreads));
    hipLaunchKernelGGL(combine_f32_kernel, grid, dim3(kCombineThreads), 0, s, (const float*)y,
                       (const float*)shared_y, (float*)out, (int)H, (int)top_k);
  }
  return hipGetLastError();
}

}  // namespace moe
