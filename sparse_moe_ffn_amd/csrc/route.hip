// Router: logits = x . router_w^T (float32 accumulation), softmax over all E
// experts in float32, top-k with equal probabilities going to the lower
// expert id, optional renormalisation, and the shared-expert gate
// sigmoid(x . g) as one extra logit column.
//
// Follows "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert",
// 题面速览 (routing block) and the nano-vLLM Qwen3-30B-A3B notes
// (lshu.cn/news/442807), qwen3_moe.py, Qwen3MoeSparseMoeBlock forward.
//
// Two kernels:
//   logits: a (token tile) x (H slice) grid.  Each workgroup multiplies its
//     tokens by router rows over one of kSlices slices of H (16x16x32 bf16
//     MFMA, float32 accumulation; fp32: plain FMA) and writes a partial
//     logit tile.  Spreading H over workgroups spreads the router weight
//     reads over many CUs, which is what matters for small batches; there a
//     workgroup is a single wave for 16 tokens and three 16-column
//     sub-tiles, so a 64-token batch runs on 96 CUs.  Large batches take
//     64-token tiles and every column, so the router rows are re-read less.
//   select: one wave per token.  The kSlices partials are summed in slice
//     order (the same order for every batch size, so a token's routing does
//     not depend on the batch), then softmax, top-k and renormalisation run
//     in registers (route_token below).
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRouteTok = 16;                 // tokens per logits workgroup
constexpr int kSlices = 8;                    // H slices (fixed for every N)
constexpr int kLogitsThreads = 256;           // 4 waves
constexpr int kLogitsWaves = kLogitsThreads / kWave;
constexpr int kMaxSubPerWave = 9;             // 16-column sub-tiles per wave: 4*9*16 >= 512+1
constexpr int kSmallSub = 3;                  // 16-column sub-tiles of a small-batch logits wave
constexpr int kLargeTiles = 4;                // 16-token tiles of a large-batch logits workgroup
constexpr int kLargeBatch = 1024;             // tokens from which the large-batch tiling is used
                                              // (whole forward, H=2048, E=128, top-8: 512 / 640 / 768
                                              // tokens 220.5 / 229.3 / 241.6 us against 223.2 / 230.8 /
                                              // 242.6 with it from 512; from 2048, 1536 tokens lost 2 us)
constexpr int kXcds = 8;                      // XCDs of the GPU; workgroups are dealt to them in turn
constexpr int kSelectWaves = 4;               // tokens per select workgroup
constexpr int kRoundsMaxK = 8;                // top-k by argmax rounds up to this k, radix select above

// Columns of the partial tiles: E router rows, the shared gate, padding to 16.
__host__ __device__ constexpr int route_cols(int E, bool shared) { return ((E + (shared ? 1 : 0) + 15) / 16) * 16; }

// ------------------------------------------------------------- wave reductions
// Butterfly/broadcast DPP steps; the result ends in lane 63 and is read back
// from there, so every lane gets the same value and the combination order is
// fixed by the instruction sequence.
template <typename Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, float identity, Op op) {
  const int id = __float_as_int(identity);
  auto step = [&](auto ctrl, auto row_mask) {
    const int o = __builtin_amdgcn_update_dpp(id, __float_as_int(v), decltype(ctrl)::value,
                                              decltype(row_mask)::value, 0xF, false);
    v = op(v, __int_as_float(o));
  };
  step(std::integral_constant<int, 0xB1>{}, std::integral_constant<int, 0xF>{});    // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{}, std::integral_constant<int, 0xF>{});    // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{}, std::integral_constant<int, 0xF>{});   // row_half_mirror
  step(std::integral_constant<int, 0x140>{}, std::integral_constant<int, 0xF>{});   // row_mirror: row totals
  step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});   // row_bcast15 into rows 1, 3
  step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});   // row_bcast31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int popc64(unsigned long long v) { return __popcll(v); }

// ------------------------------------------------------------- select
// Softmax, top-k and renormalisation of one token by one wave.  Lane l holds
// logits of experts l, l+64, ... (PER per lane).
//   1. m = max over all E; z = exp(l - m); S = sum of z (wave reductions);
//      p = z / S;
//   2. radix select: the k-th largest probability T is found bit by bit from
//      the top (p >= 0, so the float bits order like the values); each step
//      counts the entries >= a candidate with one ballot per owned slot;
//   3. the kept set is every p > T plus, among p == T, the lowest expert ids
//      (ballot prefixes in expert order) until k are kept;
//   4. the k kept (p, id) are compacted into LDS in expert order and each
//      takes slot = #{kept with larger p} + #{kept with equal p, lower id}:
//      descending probability, equal probabilities to the lower expert id;
//   5. with renormalisation the k probabilities are summed in slot order and
//      each is divided by that sum.
// NaN probabilities (only from NaN inputs) are treated as 0.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <int PER>
__device__ __forceinline__ void route_token(const float (&lg)[PER], int E, int k, int norm,
                                            float* __restrict__ sel_v, int* __restrict__ sel_e,
                                            float* __restrict__ sel_o, int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out) {
  const int lane = lane_id();
  float m = -FLT_MAX;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + kWave * i < E) m = fmaxf(m, lg[i]);
  m = wave_reduce_dpp(m, -FLT_MAX, [](float a, float b) { return fmaxf(a, b); });
  float z[PER];
  float zs = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    z[i] = (lane + kWave * i < E) ? expf(lg[i] - m) : 0.0f;
    zs += z[i];
  }
  const float s = wave_reduce_dpp(zs, 0.0f, [](float a, float b) { return a + b; });
  float v[PER];
  uint32_t key[PER];
  unsigned long long valid[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool in = lane + kWave * i < E;
    const float pr = in ? z[i] / s : 0.0f;
    v[i] = (pr == pr) ? pr : 0.0f;
    key[i] = in ? __float_as_uint(v[i]) : 0u;
    valid[i] = __ballot(in);
  }
  uint32_t T = 0;
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt += popc64(__ballot(key[i] >= cand) & valid[i]);
    if (cnt >= k) T = cand;
  }
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
    keep[i] = ((valid[i] >> lane) & 1ull) && (key[i] > T || (key[i] == T && before < need_eq));
    need_eq -= popc64(eq);                                 // slot i covers ids [64i, 64i + 64)
  }
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
    float t = 0.0f;
    if (norm)
      for (int j = 0; j < k; ++j) t += sel_o[j];          // slot order
    w_out[slot] = norm ? mv / t : mv;
  }
  wave_lds_fence();
}

// The same selection as route_token for small k, as k rounds of a wave-wide
// argmax: each round takes the largest remaining probability, the lowest
// expert id among equal ones (the lowest block of 64 ids with a match, then
// its lowest lane), and removes it.  Rounds come out in descending order with
// ties to the lower id, so slot j is round j; the renormalising sum adds the
// rounds in order, as route_token adds the slots.  Same ids, weights and
// slot order, in fewer dependent steps than the radix select when k is small.
template <int PER>
__device__ __forceinline__ void route_token_rounds(const float (&lg)[PER], int E, int k, int norm,
                                                   int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = lane_id();
  float m = -FLT_MAX;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (lane + kWave * i < E) m = fmaxf(m, lg[i]);
  m = wave_reduce_dpp(m, -FLT_MAX, [](float a, float b) { return fmaxf(a, b); });
  float z[PER];
  float zs = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    z[i] = (lane + kWave * i < E) ? expf(lg[i] - m) : 0.0f;
    zs += z[i];
  }
  const float s = wave_reduce_dpp(zs, 0.0f, [](float a, float b) { return a + b; });
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool in = lane + kWave * i < E;
    const float pr = in ? z[i] / s : 0.0f;
    v[i] = in ? ((pr == pr) ? pr : 0.0f) : -1.0f;     // -1: no expert here
  }
  int my_id = 0;
  float my_v = 0.0f, t = 0.0f;
  for (int j = 0; j < k; ++j) {
    float lm = v[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) lm = fmaxf(lm, v[i]);
    const float M = wave_reduce_dpp(lm, -FLT_MAX, [](float a, float b) { return fmaxf(a, b); });
    int id = 0;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {               // the lowest block with a match wins
      const unsigned long long b = __ballot(v[i] == M);
      if (b) id = kWave * i + (int)__builtin_ctzll(b);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + kWave * i == id) v[i] = -1.0f;
    if (lane == j) {
      my_id = id;
      my_v = M;
    }
    t += M;                                            // slot order
  }
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = norm ? my_v / t : my_v;
  }
}

// One wave per token, kSelectWaves tokens per workgroup.  After the
// large-batch logits kernel (by_tile set), workgroup b takes its tokens from
// a tile that was written on its own XCD (b % 8): tile b % 8 + 8 g, g =
// (b / 8) / kSelectPerTile, so the partials are read from that XCD's L2.
constexpr int kSelectPerTile = kRouteTok * kLargeTiles / kSelectWaves;   // select workgroups per large tile

template <int PER>
__global__ __launch_bounds__(kSelectWaves * kWave) void route_select_kernel(
    const float* __restrict__ partial, int N, int E, int k, int norm, int has_shared, int cols, int by_tile,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ shared_scale) {
  __shared__ float sel_v[kSelectWaves][kMaxTopK];
  __shared__ int sel_e[kSelectWaves][kMaxTopK];
  __shared__ float sel_o[kSelectWaves][kMaxTopK];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  int first = blockIdx.x * kSelectWaves;
  if (by_tile) {
    const int b = blockIdx.x, q = b / kXcds;
    const int tile = b % kXcds + kXcds * (q / kSelectPerTile);
    first = tile * kRouteTok * kLargeTiles + (q % kSelectPerTile) * kSelectWaves;
  }
  const int n = first + wave;
  if (n >= N) return;                                      // whole wave leaves together
  const int64_t slice = (int64_t)N * cols;
  const float* src = partial + (int64_t)n * cols;
  float lg[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    float acc = 0.0f;
    if (e < E) {
      float part[kSlices];
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) part[sl] = src[sl * slice + e];
#pragma unroll
      for (int sl = 0; sl < kSlices; ++sl) acc += part[sl];   // slice order
    }
    lg[i] = acc;
  }
  if (has_shared && lane == 0) {
    float acc = 0.0f;
    for (int sl = 0; sl < kSlices; ++sl) acc += src[sl * slice + E];
    shared_scale[n] = sigmoid_f32(acc);
  }
  if (k <= kRoundsMaxK)
    route_token_rounds<PER>(lg, E, k, norm, ids + (int64_t)n * k, w + (int64_t)n * k);
  else
    route_token<PER>(lg, E, k, norm, sel_v[wave], sel_e[wave], sel_o[wave], ids + (int64_t)n * k,
                     w + (int64_t)n * k);
}

// ------------------------------------------------------------- logits
// Partial logits over H slice blockIdx.y:
//   partial[slice][n][c] = sum_{h in slice} x[n, h] * row_c[h],
// row_c = router_w[c] for c < E, the shared gate for c == E, zero beyond.
// Every logit is one chain of matrix instructions over the slice's 32-wide
// k-steps in increasing order, from a zero accumulator, whichever kernel
// and tile computes it, so both tilings give the same bits.  The router
// rows are the matrix instruction's first operand and the tokens its second
// (the transposed product: same products and sums, measured bit for bit
// equal), so a lane holds 4 adjacent columns of one token of each 16x16
// sub-tile and writes them with one 16-byte store.

// Column c's router row, offset to this lane's 8-element piece, or null.
__device__ __forceinline__ const uint16_t* router_row(const uint16_t* router_w, const uint16_t* shared_gate, int c,
                                                      int E, int H, int lane) {
  const uint16_t* src = nullptr;
  if (c < E) src = router_w + (int64_t)c * H;
  else if (c == E && shared_gate) src = shared_gate;
  return src ? src + (lane >> 4) * 8 : nullptr;
}

// Small batches: one wave per workgroup, for 16 tokens (blockIdx.x), one H
// slice (blockIdx.y) and kSmallSub column sub-tiles (blockIdx.z).  Many
// small workgroups put the router reads of a small batch on many CUs at
// once; each wave loads its own x fragments (the same 16 rows for every
// sub-tile group, from L2).
__global__ __launch_bounds__(kWave) void route_logits_small_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ router_w, const uint16_t* __restrict__ shared_gate,
    int N, int H, int E, int cols, float* __restrict__ partial) {
  const int lane = lane_id();
  const int t0 = blockIdx.x * kRouteTok;
  const int sub0 = blockIdx.z * kSmallSub;
  const int nsub = cols / 16;
  const int ksteps = H / 32;
  const int per_slice = (ksteps + kSlices - 1) / kSlices;
  const int kb = blockIdx.y * per_slice, ke = min(ksteps, kb + per_slice);
  const uint16_t* a_src = x + (int64_t)min(t0 + (lane & 15), N - 1) * H + (lane >> 4) * 8;
  const uint16_t* b_src[kSmallSub];
  floatx4 acc[kSmallSub];
#pragma unroll
  for (int i = 0; i < kSmallSub; ++i) {
    b_src[i] = (sub0 + i < nsub) ? router_row(router_w, shared_gate, (sub0 + i) * 16 + (lane & 15), E, H, lane)
                                 : nullptr;
    acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 zero = {0u, 0u, 0u, 0u};
  constexpr int kUnroll = 8;                           // one round per slice at H = 2048
  for (int s0 = kb; s0 < ke; s0 += kUnroll) {
    uint4 a[kUnroll];
    uint4 b[kUnroll][kSmallSub];
    // Steps past the slice end reload its last step (in bounds, never used).
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k0 = min(s0 + u, ke - 1) * 32;
      a[u] = *reinterpret_cast<const uint4*>(a_src + k0);
#pragma unroll
      for (int i = 0; i < kSmallSub; ++i) b[u][i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : zero;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (s0 + u < ke) {
#pragma unroll
        for (int i = 0; i < kSmallSub; ++i) acc[i] = mfma16x16x32(b[u][i], a[u], acc[i]);
      }
  }
  float* dst = partial + (int64_t)blockIdx.y * N * cols;
#pragma unroll
  for (int i = 0; i < kSmallSub; ++i) {
    const int n = t0 + (lane & 15);
    if (sub0 + i < nsub && n < N)
      *reinterpret_cast<floatx4*>(dst + (int64_t)n * cols + (sub0 + i) * 16 + (lane >> 4) * 4) = acc[i];
  }
}

// Large batches: one 4-wave workgroup per (tile of kLargeTiles 16-token
// tiles, H slice).  Wave w owns column sub-tiles w, w+4, ... (at most SUBW)
// and all token tiles, so one router fragment feeds kLargeTiles matrix
// instructions.  Wave w < kLargeTiles loads the x fragments of tile w for a
// chunk of k-steps into LDS (in fragment order: lane-linear 1 KB blocks, so
// the reads are conflict-free), and every wave multiplies all tiles with its
// router fragments: each x fragment is loaded from memory once per
// workgroup instead of once per wave.
//
// Placement: workgroups are dealt to the 8 XCDs in turn by linear id, and
// linear id L takes tile 8 (L / 64) + L % 8 and slice (L / 8) % 8.  So all
// slices of tile t are written from XCD t % 8, groups of 8 tiles are
// dispatched one after the other, and the select kernel (which reads tile
// t's partials from XCD t % 8) finds them in that XCD's L2.  The grid holds
// whole groups; workgroups past the last tile leave at once.
__host__ __device__ constexpr int large_tile_groups(int N) {
  return ((N + kRouteTok * kLargeTiles - 1) / (kRouteTok * kLargeTiles) + kXcds - 1) / kXcds;
}

template <int SUBW>
__global__ __launch_bounds__(kLogitsThreads) void route_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ router_w, const uint16_t* __restrict__ shared_gate,
    int N, int H, int E, int cols, float* __restrict__ partial) {
  constexpr int TT = kLargeTiles;
  static_assert(TT <= kLogitsWaves, "one loading wave per token tile");
  const int L = blockIdx.x;
  const int tile = kXcds * (L / (kXcds * kSlices)) + L % kXcds;
  const int slice = (L / kXcds) % kSlices;
  const int t0 = tile * kRouteTok * TT;
  if (t0 >= N) return;                                 // whole workgroup, before any barrier
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int nsub = cols / 16;
  const int ksteps = H / 32;
  const int per_slice = (ksteps + kSlices - 1) / kSlices;
  const int kb = slice * per_slice, ke = min(ksteps, kb + per_slice);

  const uint16_t* b_src[SUBW];
  floatx4 acc[TT][SUBW];
#pragma unroll
  for (int i = 0; i < SUBW; ++i) {
    b_src[i] = router_row(router_w, shared_gate, (wave + kLogitsWaves * i) * 16 + (lane & 15), E, H, lane);
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 zero = {0u, 0u, 0u, 0u};
  constexpr int kChunk = (SUBW <= 3) ? 8 : 2;         // k-steps per LDS round (register budget)
  __shared__ uint4 a_lds[TT][kChunk][kWave];
  const uint16_t* my_a = x + (int64_t)min(t0 + wave * 16 + (lane & 15), N - 1) * H + (lane >> 4) * 8;
  for (int s0 = kb; s0 < ke; s0 += kChunk) {
    const int ns = min(kChunk, ke - s0);
    // Steps past the slice end reload its last step (in bounds, never used).
    if (wave < TT) {
      uint4 a[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) a[u] = *reinterpret_cast<const uint4*>(my_a + min(s0 + u, ke - 1) * 32);
#pragma unroll
      for (int u = 0; u < kChunk; ++u) a_lds[wave][u][lane] = a[u];
    }
    uint4 b[kChunk][SUBW];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int k0 = min(s0 + u, ke - 1) * 32;
#pragma unroll
      for (int i = 0; i < SUBW; ++i) b[u][i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : zero;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (u < ns) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const uint4 af = a_lds[t][u][lane];
#pragma unroll
          for (int i = 0; i < SUBW; ++i)
            if (wave + kLogitsWaves * i < nsub) acc[t][i] = mfma16x16x32(b[u][i], af, acc[t][i]);
        }
      }
    }
    __syncthreads();
  }
  float* dst = partial + (int64_t)slice * N * cols;
#pragma unroll
  for (int i = 0; i < SUBW; ++i) {
    const int sub = wave + kLogitsWaves * i;
    if (sub < nsub) {
      const int c = sub * 16 + (lane >> 4) * 4;         // 4 adjacent columns of one token
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int n = t0 + t * 16 + (lane & 15);
        if (n < N) *reinterpret_cast<floatx4*>(dst + (int64_t)n * cols + c) = acc[t][i];
      }
    }
  }
}

// fp32: one thread per (token, column), plain FMA over the slice.
__global__ __launch_bounds__(kLogitsThreads) void route_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ router_w, const float* __restrict__ shared_gate, int N,
    int H, int E, int cols, float* __restrict__ partial) {
  const int t0 = blockIdx.x * kRouteTok;
  const int per_slice = (H + kSlices - 1) / kSlices;
  const int hb = blockIdx.y * per_slice, he = min(H, hb + per_slice);
  float* dst = partial + (int64_t)blockIdx.y * N * cols;
  for (int q = threadIdx.x; q < kRouteTok * cols; q += kLogitsThreads) {
    const int t = q / cols, c = q % cols;
    const int n = t0 + t;
    if (n >= N) continue;
    const float* wr = (c < E) ? router_w + (int64_t)c * H : ((c == E && shared_gate) ? shared_gate : nullptr);
    float acc = 0.0f;
    if (wr) {
      const float* xr = x + (int64_t)n * H;
      for (int h = hb; h < he; ++h) acc = fmaf(xr[h], wr[h], acc);
    }
    dst[(int64_t)n * cols + c] = acc;
  }
}

int64_t route_scratch_floats(int64_t N, int64_t E, bool shared) {
  return (int64_t)kSlices * N * route_cols((int)E, shared);
}

hipError_t launch_route(const moe_problem& p, const void* x, const void* router_w, const void* shared_gate,
                        int32_t* ids, float* w, float* shared_scale, float* scratch, hipStream_t s) {
  const int N = (int)p.num_tokens, H = (int)p.hidden, E = (int)p.num_experts, k = (int)p.top_k;
  const bool shared = shared_gate != nullptr;
  const int cols = route_cols(E, shared);
  if (p.dtype == MOE_BF16) {
    const uint16_t *xb = (const uint16_t*)x, *rb = (const uint16_t*)router_w, *gb = (const uint16_t*)shared_gate;
    const int nsub = cols / 16;
    if (N >= kLargeBatch) {
      const dim3 lgrid(large_tile_groups(N) * kXcds * kSlices);
      if (cols <= 16 * kLogitsWaves * 3)
        hipLaunchKernelGGL((route_logits_bf16_kernel<3>), lgrid, dim3(kLogitsThreads), 0, s, xb, rb, gb, N, H, E, cols,
                           scratch);
      else
        hipLaunchKernelGGL((route_logits_bf16_kernel<kMaxSubPerWave>), lgrid, dim3(kLogitsThreads), 0, s, xb, rb, gb, N,
                           H, E, cols, scratch);
    } else {
      const dim3 lgrid((N + kRouteTok - 1) / kRouteTok, kSlices, (nsub + kSmallSub - 1) / kSmallSub);
      hipLaunchKernelGGL(route_logits_small_bf16_kernel, lgrid, dim3(kWave), 0, s, xb, rb, gb, N, H, E, cols, scratch);
    }
  } else {
    const dim3 lgrid((N + kRouteTok - 1) / kRouteTok, kSlices);
    hipLaunchKernelGGL(route_logits_f32_kernel, lgrid, dim3(kLogitsThreads), 0, s, (const float*)x,
                       (const float*)router_w, (const float*)shared_gate, N, H, E, cols, scratch);
  }
  const bool by_tile = p.dtype == MOE_BF16 && N >= kLargeBatch;
  const dim3 sgrid(by_tile ? large_tile_groups(N) * kXcds * kSelectPerTile : (N + kSelectWaves - 1) / kSelectWaves);
  const int nw = (int)p.norm_topk_prob;
  auto go = [&](auto per) {
    constexpr int PER = decltype(per)::value;
    hipLaunchKernelGGL(route_select_kernel<PER>, sgrid, dim3(kSelectWaves * kWave), 0, s, scratch, N, E, k, nw,
                       (int)shared, cols, (int)by_tile, ids, w, shared_scale);
  };
  if (E <= 64) go(std::integral_constant<int, 1>{});
  else if (E <= 128) go(std::integral_constant<int, 2>{});
  else if (E <= 256) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

}  // namespace moe
