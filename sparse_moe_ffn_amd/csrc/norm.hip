// Residual add + RMSNorm in front of the MoE block:
//
//   r[n]      = x[n] + residual_in[n]      (float32 sum, rounded once to dtype)
//   normed[n] = r[n] / sqrt(mean_h r[n,h]^2 + eps) * weight
//
// The nano-vLLM Qwen3 notes (lshu.cn/news/442807), Qwen3DecoderLayer and
// question 4: the norm before the MLP takes the residual stream, adds the
// incoming activations to it, keeps the sum as the new residual and hands
// its normalisation to the MLP, both in one kernel; with no residual yet the
// input is the residual.  "Step 19: Real Model — Qwen3ForCausalLM", section
// "RMSNorm：去掉均值中心化": no mean subtraction, no bias.
//
// One workgroup per token.  A thread owns 8-element chunks of the row
// (16-byte loads in bf16), keeps the rounded sums in registers, adds its
// squares sequentially, and the row total is a fixed-order reduction (wave
// shuffles, then the 4 wave partials in wave order), so a token's result
// does not depend on the batch.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 8;   // chunks of 8 per thread: hidden <= 16384

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
    v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Store 8 values rounded to the element type and leave in v what was stored.
__device__ __forceinline__ void store8(uint16_t* p, float* v) {
  const uint4 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  *reinterpret_cast<uint4*>(p) = u;
  load8(reinterpret_cast<const uint16_t*>(&u), v);
}
__device__ __forceinline__ void store8(float* p, float* v) {
  *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<float4*>(p + 4) = float4{v[4], v[5], v[6], v[7]};
}

template <typename T>
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_kernel(
    const T* x, const T* residual_in, T* residual_out, const T* __restrict__ weight,
    T* __restrict__ normed, int H, float eps) {
  const int64_t row = (int64_t)blockIdx.x * H;
  const int nch = H / 8;
  float v[kNormMaxChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kNormMaxChunks; ++q) {
    const int c = threadIdx.x + q * kNormThreads;
    if (c >= nch) break;
    const int64_t off = row + c * 8;
    load8(x + off, v[q]);
    if (residual_in) {
      float b[8];
      load8(residual_in + off, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[q][i] += b[i];
    }
    store8(residual_out + off, v[q]);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[q][i] * v[q][i];
  }
  ss = wave_sum(ss);
  __shared__ float part[kNormThreads / kWave];
  if (lane_id() == 0) part[threadIdx.x / kWave] = ss;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) total += part[w];
  const float inv = 1.0f / sqrtf(total / (float)H + eps);
#pragma unroll
  for (int q = 0; q < kNormMaxChunks; ++q) {
    const int c = threadIdx.x + q * kNormThreads;
    if (c >= nch) break;
    float w[8];
    load8(weight + c * 8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[q][i] = v[q][i] * inv * w[i];
    store8(normed + row + c * 8, v[q]);
  }
}

int64_t add_rmsnorm_max_hidden() { return (int64_t)kNormThreads * kNormMaxChunks * 8; }

hipError_t launch_add_rmsnorm(const void* x, const void* residual_in, void* residual_out, const void* weight,
                              void* normed, int64_t N, int64_t H, float eps, int32_t dtype, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(add_rmsnorm_kernel<uint16_t>, dim3((unsigned)N), dim3(kNormThreads), 0, s,
                       (const uint16_t*)x, (const uint16_t*)residual_in, (uint16_t*)residual_out,
                       (const uint16_t*)weight, (uint16_t*)normed, (int)H, eps);
  else
    hipLaunchKernelGGL(add_rmsnorm_kernel<float>, dim3((unsigned)N), dim3(kNormThreads), 0, s,
                       (const float*)x, (const float*)residual_in, (float*)residual_out,
                       (const float*)weight, (float*)normed, (int)H, eps);
  return hipGetLastError();
}

}  // namespace moe
