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

#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRouteTok = 16;
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouteMaxCols = ((kMaxExperts + 1 + 15) / 16) * 16;            // 528
constexpr int kLogitLd = kRouteMaxCols + 4;     // rows stay 16-byte aligned
constexpr int kRouteBf16Waves = 8;
constexpr int kRouteBf16Threads = kRouteBf16Waves * kWave;
constexpr int kRouteSelWaves = kRouteThreads / kWave > kRouteBf16Waves ? kRouteThreads / kWave : kRouteBf16Waves;

// Softmax, top-k and renormalisation of one token, by one whole wave.  The
// token's logits sit in an LDS row every lane can read (same-address reads
// are broadcasts); lane l owns experts l, l+64, ... (PER per lane).
//   1. every lane scans the row for the maximum;
//   2. each lane turns its own entries into z = exp(l - max), in place;
//   3. every lane sums the row in expert order (float32, one fixed order);
//   4. each lane divides its entries by the sum: p = z / sum;
//   5. radix select: the k-th largest probability T is found bit by bit from
//      the top (p >= 0, so the float bits order like the values); each step
//      counts the entries >= a candidate with one ballot per owned slot;
//   6. the kept set is every p > T plus, among p == T, the lowest expert ids
//      (ballot prefixes in expert order) until k are kept;
//   7. the k kept (p, id) are compacted into LDS in expert order and each
//      takes slot = #{kept with larger p} + #{kept with equal p, lower id}:
//      descending probability, equal probabilities to the lower expert id;
//   8. with renormalisation the k probabilities are summed in slot order and
//      each is divided by that sum.
// NaN probabilities (only from NaN inputs) are treated as 0.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

__device__ __forceinline__ int popc64(unsigned long long v) { return __popcll(v); }

template <int PER>
__device__ __forceinline__ void route_token(float* __restrict__ row, float* __restrict__ sel_v,
                                            int* __restrict__ sel_e, float* __restrict__ sel_o, int E,
                                            int k, int norm,
                                            int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = lane_id();
  const int Ep = (E + 31) & ~31;
  // 1. maximum
  float m = -FLT_MAX;
  for (int e0 = 0; e0 < Ep; e0 += 32) {
    float4 q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = *reinterpret_cast<const float4*>(row + e0 + 4 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float qq[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) m = (e0 + 4 * j + c < E) ? fmaxf(m, qq[c]) : m;
    }
  }
  // 2. exponentials of the owned entries
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    if (e < E) row[e] = expf(row[e] - m);
  }
  wave_lds_fence();
  // 3. sum in expert order
  float s = 0.0f;
  for (int e0 = 0; e0 < Ep; e0 += 32) {
    float4 q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = *reinterpret_cast<const float4*>(row + e0 + 4 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float qq[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (e0 + 4 * j + c < E) s += qq[c];
    }
  }
  // 4. probabilities, as order-preserving bit patterns
  float v[PER];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const float pr = (e < E) ? row[e] / s : 0.0f;
    v[i] = (pr == pr) ? pr : 0.0f;
    key[i] = (e < E) ? __float_as_uint(v[i]) : 0u;
  }
  // 5. radix select of the k-th largest key (entries past E hold key 0 and
  //    are never counted: they are excluded from every ballot)
  unsigned long long valid[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) valid[i] = __ballot(lane + kWave * i < E);
  uint32_t T = 0;
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt += popc64(__ballot(key[i] >= cand) & valid[i]);
    if (cnt >= k) T = cand;
  }
  // 6. kept set: above T, then the lowest ids among those equal to T
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) n_gt += popc64(__ballot(key[i] > T) & valid[i]);
  int need_eq = k - n_gt;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  bool keep[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const unsigned long long eq = __ballot(key[i] == T) & valid[i];
    const int before = popc64(eq & below);                 // equal entries with a lower id in this slot
    keep[i] = (lane + kWave * i < E) && (key[i] > T || (key[i] == T && before < need_eq));
    need_eq -= popc64(eq);                                 // slot i covers ids [64i, 64i + 64)
  }
  // 7. compact the kept entries in expert order, then order them
  int base = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const unsigned long long kb = __ballot(keep[i]);
    if (keep[i]) {
      const int pos = base + popc64(kb & below);
      sel_v[pos] = v[i];
      sel_e[pos] = lane + kWave * i;
    }
    base += popc64(kb);
  }
  wave_lds_fence();
  float mv = 0.0f;
  int slot = 0;
  if (lane < k) {
    mv = sel_v[lane];
    const int me = sel_e[lane];
    for (int j = 0; j < k; ++j) {
      const float ov = sel_v[j];
      slot += (ov > mv) || (ov == mv && sel_e[j] < me);
    }
    ids_out[slot] = me;
    sel_o[slot] = mv;
  }
  wave_lds_fence();
  if (lane < k) {
    // 8. renormalisation: the kept probabilities summed in slot order
    float t = 0.0f;
    if (norm)
      for (int j = 0; j < k; ++j) t += sel_o[j];
    w_out[slot] = norm ? mv / t : mv;
  }
  wave_lds_fence();
}

template <int PER>
__device__ __forceinline__ void route_tile_from_lds(float (*logits)[kLogitLd], float (*sel_v)[kMaxTopK],
                                                    int (*sel_e)[kMaxTopK], float (*sel_o)[kMaxTopK], int t0,
                                                    int N, int E,
                                    int k, int norm, int has_shared, int32_t* ids, float* w,
                                    float* shared_scale) {
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int t = wave; t < kRouteTok; t += nwaves) {
    const int n = t0 + t;
    if (n >= N) break;
    if (has_shared && lane_id() == 0) shared_scale[n] = sigmoid_f32(logits[t][E]);
    route_token<PER>(logits[t], sel_v[wave], sel_e[wave], sel_o[wave], E, k, norm, ids + (int64_t)n * k,
                     w + (int64_t)n * k);
  }
}

// bf16 logits: the 16 x (E [+1]) tile is a matrix-core product, computed in
// groups of up to 144 columns.  The K dimension is dealt round-robin to the
// 8 waves (32 columns of H per step), every wave covers all columns of the
// group, and the 8 partial tiles are summed in wave order, so each logit is
// reduced in a fixed order that does not depend on the batch.
constexpr int kRouteSub = 9;                 // 16-column sub-tiles per group
constexpr int kRouteUnroll = 4;              // K steps in flight per wave (E <= 256)

template <int PER>
__global__ __launch_bounds__(kRouteBf16Threads) void route_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ router_w,
    const uint16_t* __restrict__ shared_gate, int N, int H, int E, int k, int norm,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ shared_scale) {
  __shared__ __attribute__((aligned(16))) float logits[kRouteTok][kLogitLd];
  __shared__ float part[kRouteBf16Waves][kRouteTok][kRouteSub * 16];
  __shared__ float sel_v[kRouteSelWaves][kMaxTopK];
  __shared__ int sel_e[kRouteSelWaves][kMaxTopK];
  __shared__ float sel_o[kRouteSelWaves][kMaxTopK];
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
    constexpr int kUnroll = (PER >= 8) ? 2 : kRouteUnroll;   // fewer registers next to wide rows
    // Up to kUnroll of this wave's K steps are loaded before any is
    // used, so their memory latencies overlap.
    constexpr int kStride = kRouteBf16Waves * 32;
    for (int k0 = wave * 32; k0 < H; k0 += kUnroll * kStride) {
      uint4 a[kUnroll];
      uint4 b[kUnroll][kRouteSub];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kk = k0 + u * kStride;
        if (kk < H) {
          a[u] = *reinterpret_cast<const uint4*>(a_src + kk);
#pragma unroll
          for (int i = 0; i < kRouteSub; ++i)
            if (i < gsub) b[u][i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + kk) : zero;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (k0 + u * kStride < H) {
#pragma unroll
          for (int i = 0; i < kRouteSub; ++i)
            if (i < gsub) acc[i] = mfma16x16x32(a[u], b[u][i], acc[i]);
        }
      }
    }
    // Every wave stores its partial tile; after one barrier each thread sums
    // the 8 partials of its elements in wave order into the logit tile.
#pragma unroll
    for (int i = 0; i < kRouteSub; ++i) {
      if (i < gsub) {
        const int c = i * 16 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][(lane >> 4) * 4 + r][c] = acc[i][r];
      }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kRouteTok * gsub * 16; q += kRouteBf16Threads) {
      const int row = q / (gsub * 16), c = q % (gsub * 16);
      float sum = part[0][row][c];
#pragma unroll
      for (int wv = 1; wv < kRouteBf16Waves; ++wv) sum += part[wv][row][c];
      logits[row][s0 * 16 + c] = sum;
    }
    __syncthreads();
  }
  route_tile_from_lds<PER>(logits, sel_v, sel_e, sel_o, t0, N, E, k, norm, shared_gate != nullptr, ids, w,
                           shared_scale);
}

template <int PER>
__global__ __launch_bounds__(kRouteThreads) void route_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ router_w,
    const float* __restrict__ shared_gate, int N, int H, int E, int k, int norm,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ shared_scale) {
  __shared__ __attribute__((aligned(16))) float logits[kRouteTok][kLogitLd];
  __shared__ float sel_v[kRouteSelWaves][kMaxTopK];
  __shared__ int sel_e[kRouteSelWaves][kMaxTopK];
  __shared__ float sel_o[kRouteSelWaves][kMaxTopK];
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
  route_tile_from_lds<PER>(logits, sel_v, sel_e, sel_o, t0, N, E, k, norm, shared_gate != nullptr, ids, w,
                           shared_scale);
}

hipError_t launch_route(const moe_problem& p, const void* x, const void* router_w,
                        const void* shared_gate, int32_t* ids, float* w, float* shared_scale,
                        hipStream_t s) {
  const int N = (int)p.num_tokens, H = (int)p.hidden, E = (int)p.num_experts, k = (int)p.top_k;
  const dim3 grid((N + kRouteTok - 1) / kRouteTok);
  const int nw = (int)p.norm_topk_prob;
  auto go = [&](auto per) {
    constexpr int PER = decltype(per)::value;
    if (p.dtype == MOE_BF16)
      hipLaunchKernelGGL(route_bf16_kernel<PER>, grid, dim3(kRouteBf16Threads), 0, s, (const uint16_t*)x,
                         (const uint16_t*)router_w, (const uint16_t*)shared_gate, N, H, E, k, nw, ids, w,
                         shared_scale);
    else
      hipLaunchKernelGGL(route_f32_kernel<PER>, grid, dim3(kRouteThreads), 0, s, (const float*)x,
                         (const float*)router_w, (const float*)shared_gate, N, H, E, k, nw, ids, w,
                         shared_scale);
  };
  if (E <= 64) go(std::integral_constant<int, 1>{});
  else if (E <= 128) go(std::integral_constant<int, 2>{});
  else if (E <= 256) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

}  // namespace moe
