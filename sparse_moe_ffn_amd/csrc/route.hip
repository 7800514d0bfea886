// Router kernel: logits = x . router_w^T (float32 accumulation), softmax over
// all E experts in float32, top-k with equal probabilities going to the lower
// expert id, optional renormalisation, and the shared-expert gate
// sigmoid(x . g) as one extra logit column.
//
// Follows "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert",
// 题面速览 (routing block) and "Nano-vLLM 代码笔记 (八)",
// Qwen3MoeSparseMoeBlock forward.
//
// One workgroup routes 16 tokens.  bf16: the [16 x (E+1)] logit tile is a
// matrix-core product (16x16x32 bf16 MFMA, float32 accumulation) with H split
// over 8 waves; fp32: plain FMA dot products.  The tile goes to LDS, then
// each wave routes its tokens: two probabilities per lane for E = 128,
// wave-wide max / sum, and k rounds of a (value, id) wave argmax.
#include <float.h>
#include <limits.h>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRouteTok = 16;
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouteMaxCols = ((kMaxExperts + 1 + 15) / 16) * 16;            // 528
constexpr int kRoutePer = kMaxExperts / kWave;                                 // 8
constexpr int kLogitLd = kRouteMaxCols + 1;
constexpr int kRouteBf16Waves = 8;
constexpr int kRouteBf16Threads = kRouteBf16Waves * kWave;

// Softmax, top-k and renormalisation of one token, by one whole wave.
__device__ void route_token(const float* __restrict__ logit, int E, int k, int norm,
                            int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = lane_id();
  float v[kRoutePer];
  float m = -FLT_MAX;
#pragma unroll
  for (int i = 0; i < kRoutePer; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? logit[e] : -FLT_MAX;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kRoutePer; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? expf(v[i] - m) : 0.0f;
    s += v[i];
  }
  s = wave_sum(s);
#pragma unroll
  for (int i = 0; i < kRoutePer; ++i) {
    float pr = v[i] / s;
    // A NaN (from NaN inputs) ranks below every probability but above the
    // taken marker, so k valid ids are always produced.
    v[i] = (pr == pr) ? pr : -1.0f;
  }
  int my_id = 0;
  float my_v = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bv = -3.0f;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < kRoutePer; ++i) {
      const int e = lane + kWave * i;
      if (e < E && v[i] > bv) { bv = v[i]; be = e; }     // ascending e: lowest id on ties
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
#pragma unroll
    for (int i = 0; i < kRoutePer; ++i)
      if (be == lane + kWave * i) v[i] = -2.0f;            // taken
    if (lane == r) { my_id = be; my_v = bv; }
  }
  float w = my_v;
  if (norm) {
    float t = 0.0f;
    for (int r = 0; r < k; ++r) t += __shfl(my_v, r, kWave);   // slot order
    w = my_v / t;
  }
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = w;
  }
}

__device__ void route_tile_from_lds(const float (*logits)[kLogitLd], int t0, int N, int E, int k, int norm,
                                    int has_shared, int32_t* ids, float* w, float* shared_scale) {
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int t = wave; t < kRouteTok; t += nwaves) {
    const int n = t0 + t;
    if (n >= N) break;
    route_token(logits[t], E, k, norm, ids + (int64_t)n * k, w + (int64_t)n * k);
    if (has_shared && lane_id() == 0) shared_scale[n] = sigmoid_f32(logits[t][E]);
  }
}

// bf16 logits: the 16 x (E [+1]) tile is a matrix-core product, computed in
// groups of up to 144 columns.  The K dimension is dealt round-robin to the
// 8 waves (32 columns of H per step), every wave covers all columns of the
// group, and the 8 partial tiles are summed through LDS in wave order, so
// each logit is reduced in a fixed order that does not depend on the batch.
constexpr int kRouteSub = 9;                 // 16-column sub-tiles per group

__global__ __launch_bounds__(kRouteBf16Threads) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ router_w,
    const uint16_t* __restrict__ shared_gate, int N, int H, int E, int k, int norm,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ shared_scale) {
  __shared__ float logits[kRouteTok][kLogitLd];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kRouteTok;
  const int cols = E + (shared_gate ? 1 : 0);
  const int nsub = (cols + 15) / 16;

  const int arow = min(t0 + (lane & 15), N - 1);
  const uint16_t* a_src = x + (int64_t)arow * H + (lane >> 4) * 8;
  const uint4 zero = {0u, 0u, 0u, 0u};
  for (int s0 = 0; s0 < nsub; s0 += kRouteSub) {
    const int gsub = min(kRouteSub, nsub - s0);
    const uint16_t* b_src[kRouteSub];
    floatx4 acc[kRouteSub];
#pragma unroll
    for (int i = 0; i < kRouteSub; ++i) {
      const int c = (s0 + i) * 16 + (lane & 15);
      const uint16_t* src = nullptr;
      if (c < E) src = router_w + (int64_t)c * H;
      else if (c == E && shared_gate) src = shared_gate;
      b_src[i] = src ? src + (lane >> 4) * 8 : nullptr;
      acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = wave * 32; k0 < H; k0 += kRouteBf16Waves * 32) {
      const uint4 a = *reinterpret_cast<const uint4*>(a_src + k0);
      uint4 b[kRouteSub];
#pragma unroll
      for (int i = 0; i < kRouteSub; ++i)
        if (i < gsub) b[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : zero;
#pragma unroll
      for (int i = 0; i < kRouteSub; ++i)
        if (i < gsub) acc[i] = mfma16x16x32(a, b[i], acc[i]);
    }
    for (int wv = 0; wv < kRouteBf16Waves; ++wv) {
      if (wave == wv) {
#pragma unroll
        for (int i = 0; i < kRouteSub; ++i) {
          if (i < gsub) {
            const int c = (s0 + i) * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float& dst = logits[(lane >> 4) * 4 + r][c];
              dst = (wv == 0) ? acc[i][r] : dst + acc[i][r];
            }
          }
        }
      }
      __syncthreads();
    }
  }
  route_tile_from_lds(logits, t0, N, E, k, norm, shared_gate != nullptr, ids, w, shared_scale);
}

__global__ __launch_bounds__(kRouteThreads) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ router_w,
    const float* __restrict__ shared_gate, int N, int H, int E, int k, int norm,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ shared_scale) {
  __shared__ float logits[kRouteTok][kLogitLd];
  const int t0 = blockIdx.x * kRouteTok;
  const int cols = E + (shared_gate ? 1 : 0);
  for (int q = threadIdx.x; q < kRouteTok * cols; q += kRouteThreads) {
    const int t = q / cols, c = q % cols;
    const int n = min(t0 + t, N - 1);
    const float* xr = x + (int64_t)n * H;
    const float* wr = (c < E) ? router_w + (int64_t)c * H : shared_gate;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
    logits[t][c] = acc;
  }
  __syncthreads();
  route_tile_from_lds(logits, t0, N, E, k, norm, shared_gate != nullptr, ids, w, shared_scale);
}

hipError_t launch_route(const moe_problem& p, const void* x, const void* router_w,
                        const void* shared_gate, int32_t* ids, float* w, float* shared_scale,
                        hipStream_t s) {
  const int N = (int)p.num_tokens, H = (int)p.hidden, E = (int)p.num_experts, k = (int)p.top_k;
  const dim3 grid((N + kRouteTok - 1) / kRouteTok);
  if (p.dtype == MOE_BF16) {
    hipLaunchKernelGGL(route_bf16_kernel, grid, dim3(kRouteBf16Threads), 0, s,
                       (const uint16_t*)x, (const uint16_t*)router_w, (const uint16_t*)shared_gate,
                       N, H, E, k, (int)p.norm_topk_prob, ids, w, shared_scale);
  } else {
    hipLaunchKernelGGL(route_f32_kernel, grid, dim3(kRouteThreads), 0, s,
                       (const float*)x, (const float*)router_w, (const float*)shared_gate,
                       N, H, E, k, (int)p.norm_topk_prob, ids, w, shared_scale);
  }
  return hipGetLastError();
}

}  // namespace moe
