// Align kernel: stable grouping of the N*k (token, slot) pairs by expert id,
// each expert's segment padded to the GEMM tile height.
//
// Follows "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert",
// 逐步图 steps 1-3 (flatten the pairs, stable sort by expert, per-expert
// counts whose prefix sums start the segments; empty experts do no work) and
// the remark there that this bookkeeping is what aligning tokens to a block
// does in a fused MoE.
//
// One workgroup of 16 waves.  The pair list is cut into 16 contiguous
// chunks, one per wave.
//   pass 1: per-wave histograms with LDS atomics (counts only);
//   scan:   per-expert exclusive prefix over the waves (each wave's base
//           inside an expert), then over experts for the unpadded segment
//           starts, the tile starts and the padded row starts;
//   pass 2: each wave walks its chunk 64 pairs at a time; lanes holding the
//           same expert find each other with one ballot per id bit, a lane's
//           rank is the number of matching lanes below it, and the highest
//           matching lane advances the wave's running position for that
//           expert.  Chunks are in pair order and lanes are in pair order, so
//           positions are ascending in the pair index: the sort is stable
//           without comparing anything.
// Atomics only count; every position comes from prefix sums, so the result
// is the same on every run.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kAlignUnroll = 8;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int P, int E, int BM, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ order, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_rows, int32_t* __restrict__ num_tiles) {
  __shared__ int hist[kAlignWaves][kMaxExperts];   // per-wave counts, then per-wave bases
  __shared__ int cnt[kMaxExperts];
  __shared__ int seg_start[kMaxExperts];
  __shared__ int tile_start[kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;

  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&hist[0][0])[i] = 0;
  __syncthreads();

  // Chunk of this wave: a multiple of 64 pairs.
  const int chunk = ((P + kAlignWaves * kWave - 1) / (kAlignWaves * kWave)) * kWave;
  const int beg = min(P, wave * chunk);
  const int end = min(P, beg + chunk);

  // pass 1: histogram (loads issued in batches so they overlap)
  for (int p0 = beg; p0 < end; p0 += kWave * kAlignUnroll) {
    int e[kAlignUnroll];
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int p = p0 + u * kWave + lane;
      const int v = (p < end) ? ids[p] : -1;
      e[u] = (v < E) ? v : -1;                          // ids outside [0, E) are dropped
    }
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u)
      if (e[u] >= 0) atomicAdd(&hist[wave][e[u]], 1);
  }
  __syncthreads();

  // per-expert: exclusive base of every wave inside the expert, and the total
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = 0;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();

  // exclusive scans over experts (wave 0, 64 experts per step)
  if (wave == 0) {
    int carry_rows = 0, carry_tiles = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int c = (e < E) ? cnt[e] : 0;
      const int nt = (c + BM - 1) / BM;
      int ic = c, it = nt;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int uc = __shfl_up(ic, o, kWave);
        const int ut = __shfl_up(it, o, kWave);
        if (lane >= o) { ic += uc; it += ut; }
      }
      if (e < E) {
        seg_start[e] = carry_rows + ic - c;
        tile_start[e] = carry_tiles + it - nt;
      }
      carry_rows += __shfl(ic, kWave - 1, kWave);
      carry_tiles += __shfl(it, kWave - 1, kWave);
    }
    if (lane == 0) {
      offsets[E] = carry_rows;
      num_tiles[0] = carry_tiles;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    counts[e] = cnt[e];
    offsets[e] = seg_start[e];
  }

  // pass 2: stable scatter
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int p0 = beg; p0 < end; p0 += kWave * kAlignUnroll) {
    int ev[kAlignUnroll];
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int p = p0 + u * kWave + lane;
      const int v = (p < end) ? ids[p] : -1;
      ev[u] = (v < E) ? v : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignUnroll; ++u) {
      const int p = p0 + u * kWave + lane;
      const int e = ev[u];
      const bool valid = e >= 0;
      unsigned long long match = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const unsigned long long m = __ballot(bit);
        match &= bit ? m : ~m;
      }
      if (valid) {
        const int rank = __popcll(match & below);
        const int pos = hist[wave][e] + rank;
        order[seg_start[e] + pos] = p;
        sorted_pairs[tile_start[e] * BM + pos] = p;
        if ((match >> lane) == 1ull) hist[wave][e] = pos + 1;   // highest matching lane
      }
    }
  }

  // padding rows and tile table, one expert per thread
  for (int e = tid; e < E; e += kAlignThreads) {
    const int c = cnt[e];
    const int t0 = tile_start[e];
    const int nt = (c + BM - 1) / BM;
    for (int t = 0; t < nt; ++t) {
      tile_expert[t0 + t] = e;
      tile_rows[t0 + t] = min(BM, c - t * BM);
    }
    for (int r = c; r < nt * BM; ++r) sorted_pairs[t0 * BM + r] = P;
  }
}

hipError_t launch_align(const int32_t* ids, int64_t num_pairs, int64_t num_experts, int64_t block_m,
                        int32_t* counts, int32_t* offsets, int32_t* order, int32_t* sorted_pairs,
                        int32_t* tile_expert, int32_t* tile_rows, int32_t* num_tiles, hipStream_t s) {
  int nbits = 0;
  while ((1ll << nbits) < num_experts) ++nbits;
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, (int)num_pairs,
                     (int)num_experts, (int)block_m, nbits, counts, offsets, order, sorted_pairs,
                     tile_expert, tile_rows, num_tiles);
  return hipGetLastError();
}

}  // namespace moe
