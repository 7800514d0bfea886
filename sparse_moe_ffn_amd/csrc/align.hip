// Align kernels: stable grouping of the N*k (token, slot) pairs by expert id,
// each expert's segment padded to the GEMM tile height.
//
// Follows "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert",
// 逐步图 steps 1-3 (flatten the pairs, stable sort by expert, per-expert
// counts whose prefix sums start the segments; empty experts do no work) and
// the remark there that this bookkeeping is what aligning tokens to a block
// does in a fused MoE.
//
// The pair list is cut into chunks of kChunk pairs and each chunk into 16
// contiguous wave ranges.  Positions are built from counts only:
//   histogram: per-range counts with LDS atomics;
//   scan:      per-expert exclusive prefixes over the ranges (each range's
//              base inside its expert), then over the experts for the
//              unpadded segment starts, the tile starts and the padded rows;
//   scatter:   each wave takes its range 64 pairs at a time; lanes holding
//              the same expert find each other with one ballot per id bit, a
//              lane's rank is the number of matching lanes below it, and the
//              highest matching lane advances the running position.  Ranges
//              are in pair order and lanes are in pair order, so positions are
//              ascending in the pair index: the sort is stable without
//              comparing anything.
// Atomics only count; every position comes from prefix sums, so the result
// is the same on every run.
//
// One chunk (<= 4096 pairs): a single workgroup does everything.  More: two
// launches, with the per-chunk counts in a caller-provided scratch array:
// count per chunk, then scan and scatter per chunk (every workgroup redoes
// the small scan over the per-chunk counts, which saves a one-workgroup
// launch between the two).
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kAlignUnroll = 4;
constexpr int kChunk = kAlignWaves * kWave * kAlignUnroll;     // pairs per chunk (4096)
static_assert(kChunk / kAlignWaves == kWave * kAlignUnroll, "a wave range is one load of kAlignUnroll ids per lane");

// Expert id of pair p, or -1 past the end / outside [0, E) (dropped).
__device__ __forceinline__ int pair_expert(const int32_t* ids, int p, int end, int E) {
  const int v = (p < end) ? ids[p] : -1;
  return (v < E) ? v : -1;
}

// Lanes of this wave holding the same valid expert id as this lane.
__device__ __forceinline__ unsigned long long match_lanes(int e, int nbits) {
  const bool valid = e >= 0;
  unsigned long long match = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const unsigned long long m = __ballot(bit);
    match &= bit ? m : ~m;
  }
  return match;
}

// A wave range holds at most kWave * kAlignUnroll pairs, kAlignUnroll per
// lane: its ids are loaded once, first thing, so that the load overlaps the
// kernel's other start-up reads, and serve both the histogram and the
// scatter.  e[u] is the expert of pair beg + u * kWave + lane, or -1.
__device__ __forceinline__ void load_range(const int32_t* ids, int beg, int end, int E, int (&e)[kAlignUnroll]) {
  const int lane = lane_id();
#pragma unroll
  for (int u = 0; u < kAlignUnroll; ++u) e[u] = pair_expert(ids, beg + u * kWave + lane, end, E);
}

// Histogram of a wave range into h[e] (LDS atomics, counts only).
__device__ __forceinline__ void count_range(const int (&e)[kAlignUnroll], int* h) {
#pragma unroll
  for (int u = 0; u < kAlignUnroll; ++u)
    if (e[u] >= 0) atomicAdd(&h[e[u]], 1);
}

// Stable scatter of a wave range starting at pair beg: pos[e] holds the
// running position of expert e inside its segment for this range (advanced
// in place).
__device__ __forceinline__ void scatter_range(const int (&ev)[kAlignUnroll], int beg, int BM, int nbits, int* pos,
                                              const int* seg_start, const int* tile_start, int32_t* order,
                                              int32_t* sorted_pairs) {
  const int lane = lane_id();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int u = 0; u < kAlignUnroll; ++u) {
    const int p = beg + u * kWave + lane;
    const int e = ev[u];
    const unsigned long long match = match_lanes(e, nbits);
    if (e >= 0) {
      const int rank = __popcll(match & below);
      const int at = pos[e] + rank;
      order[seg_start[e] + at] = p;
      sorted_pairs[tile_start[e] * BM + at] = p;
      if ((match >> lane) == 1ull) pos[e] = at + 1;          // highest matching lane
    }
  }
}

// Inclusive prefix sum over the 16 lanes of each DPP row (Hillis-Steele,
// shifts 1, 2, 4, 8; a lane whose source lies before its row adds 0).
__device__ __forceinline__ int row_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  return v;
}

// Inclusive prefix sum over the wave: row scans, then each row adds the
// totals of the rows before it (row_bcast:15 into rows 1 and 3, then
// row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = row_inclusive_scan(v);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Wave 0: exclusive scans of cnt[] (rows) and of its tile counts over the
// experts; writes seg_start, tile_start and (when not null) offsets and
// num_tiles.
__device__ __forceinline__ void scan_experts(const int* cnt, int E, int BM, int* seg_start, int* tile_start,
                                             int32_t* offsets, int32_t* num_tiles) {
  const int lane = lane_id();
  int carry_rows = 0, carry_tiles = 0;
  for (int e0 = 0; e0 < E; e0 += kWave) {
    const int e = e0 + lane;
    const int c = (e < E) ? cnt[e] : 0;
    const int nt = (c + BM - 1) / BM;
    const int ic = wave_inclusive_scan(c);
    const int it = wave_inclusive_scan(nt);
    if (e < E) {
      seg_start[e] = carry_rows + ic - c;
      tile_start[e] = carry_tiles + it - nt;
      if (offsets) offsets[e] = carry_rows + ic - c;
    }
    carry_rows += __builtin_amdgcn_readlane(ic, kWave - 1);
    carry_tiles += __builtin_amdgcn_readlane(it, kWave - 1);
  }
  if (lane == 0 && offsets) {
    offsets[E] = carry_rows;
    num_tiles[0] = carry_tiles;
  }
}

// Tile table and sentinel padding, by the whole workgroup.
__device__ __forceinline__ void fill_tiles(const int* cnt, const int* tile_start, int E, int BM, int P,
                                           int total_tiles, int32_t* sorted_pairs, int32_t* tile_expert,
                                           int32_t* tile_rows) {
  for (int t = threadIdx.x; t < total_tiles; t += blockDim.x) {
    int lo = 0, hi = E - 1;                  // last expert whose tile range starts at or before t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
    }
    int e = lo;
    while (e > 0 && cnt[e] == 0) --e;        // empty experts own no tiles
    tile_expert[t] = e;
    tile_rows[t] = min(BM, cnt[e] - (t - tile_start[e]) * BM);
  }
  // Sentinel padding: a group of threads per expert, each taking every
  // tpe-th padding row of it.
  const int tpe = max(1, (int)blockDim.x / E);
  const int groups = blockDim.x / tpe;
  for (int e = threadIdx.x / tpe; e < E; e += groups) {
    const int c = cnt[e];
    const int padded = ((c + BM - 1) / BM) * BM;
    int32_t* seg = sorted_pairs + (int64_t)tile_start[e] * BM;
    for (int r = c + (int)(threadIdx.x % tpe); r < padded; r += tpe) seg[r] = P;
  }
}

__device__ __forceinline__ int nbits_of(int E) {
  int n = 0;
  while ((1 << n) < E) ++n;
  return n;
}

// ------------------------------------------------------------ one workgroup

__global__ __launch_bounds__(kAlignThreads) void align_single_kernel(
    const int32_t* __restrict__ ids, int P, int E, int BM, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ order, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_rows, int32_t* __restrict__ num_tiles) {
  __shared__ int hist[kAlignWaves][kMaxExperts];   // per-wave counts, then per-wave bases
  __shared__ int cnt[kMaxExperts];
  __shared__ int seg_start[kMaxExperts];
  __shared__ int tile_start[kMaxExperts];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int nbits = nbits_of(E);
  // P <= kChunk, so a wave range is at most kWave * kAlignUnroll pairs.
  const int range = ((P + kAlignWaves * kWave - 1) / (kAlignWaves * kWave)) * kWave;
  const int beg = min(P, wave * range);
  const int end = min(P, beg + range);
  int ev[kAlignUnroll];
  load_range(ids, beg, end, E, ev);

  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  count_range(ev, hist[wave]);
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = 0;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
    cnt[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  if (wave == 0) scan_experts(cnt, E, BM, seg_start, tile_start, offsets, num_tiles);
  __syncthreads();
  scatter_range(ev, beg, BM, nbits, hist[wave], seg_start, tile_start, order, sorted_pairs);
  const int total = tile_start[E - 1] + (cnt[E - 1] + BM - 1) / BM;
  fill_tiles(cnt, tile_start, E, BM, P, total, sorted_pairs, tile_expert, tile_rows);
}

// ------------------------------------------------------------ many chunks

// Per-chunk expert histogram -> chunk_counts[chunk][E].
__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(const int32_t* __restrict__ ids, int P,
                                                                     int E, int32_t* __restrict__ chunk_counts) {
  __shared__ int h[kMaxExperts];
  const int c0 = blockIdx.x * kChunk;
  const int wave = threadIdx.x / kWave;
  const int range = kChunk / kAlignWaves;
  const int beg = min(P, c0 + wave * range);
  const int end = min(P, beg + range);
  int ev[kAlignUnroll];
  load_range(ids, beg, end, E, ev);
  for (int i = threadIdx.x; i < E; i += kAlignThreads) h[i] = 0;
  __syncthreads();
  count_range(ev, h);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kAlignThreads) chunk_counts[(int64_t)blockIdx.x * E + i] = h[i];
}

// Scan and stable scatter of chunk blockIdx.x in one launch.  Every
// workgroup reads all chunks' histograms (nchunks x E ints, a few KB) and
// forms, in LDS, its chunk's base in every expert segment and the experts'
// totals, segment starts and tile starts; workgroup 0 also writes counts,
// offsets, num_tiles, the tile table and the sentinel padding.  The padding
// rows of a segment lie past its pairs, so they never meet the scatter.
__global__ __launch_bounds__(kAlignThreads) void align_scan_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int BM, int nchunks, const int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ order,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ tile_expert, int32_t* __restrict__ tile_rows,
    int32_t* __restrict__ num_tiles) {
  __shared__ int hist[kAlignWaves][kMaxExperts];
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int seg_start[kMaxExperts];
  __shared__ int tile_start[kMaxExperts];
  __shared__ int part_sum[kAlignThreads];
  __shared__ int part_before[kAlignThreads];
  __shared__ int total_tiles;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int b = blockIdx.x;
  const bool lead = b == 0;
  const int range = kChunk / kAlignWaves;
  const int beg = min(P, b * kChunk + wave * range);
  const int end = min(P, beg + range);
  int ev[kAlignUnroll];
  load_range(ids, beg, end, E, ev);                    // in flight with the chunk counts below
  for (int i = tid; i < kAlignWaves * kMaxExperts; i += kAlignThreads) (&hist[0][0])[i] = 0;
  // Expert totals over all chunks, and this chunk's base in each expert (its
  // pairs in the chunks before it).  Up to 16 chunks: one thread per
  // expert, loads in rounds of 8.  More: G groups of E threads each sum a
  // contiguous run of about 8 chunks, so the loads go out in one round, and
  // the group sums are added in LDS (measured: the extra barrier costs more
  // than a second round of loads saves at 16 chunks, and less at 32).
  auto sum_chunks = [&](int e, int c_lo, int c_hi, int& sum, int& before) {
    for (int c0 = c_lo; c0 < c_hi; c0 += 8) {         // 8 independent loads in flight
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (c0 + u < c_hi) ? chunk_counts[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sum += v[u];
        before += (c0 + u < b) ? v[u] : 0;
      }
    }
  };
  if (nchunks <= 16) {
    for (int e = tid; e < E; e += kAlignThreads) {
      int run = 0, mine = 0;
      sum_chunks(e, 0, nchunks, run, mine);
      cnt[e] = run;
      base[e] = mine;
      if (lead) counts[e] = run;
    }
  } else {
    const int G = min(kAlignThreads / E, (nchunks + 7) / 8);   // E <= kMaxExperts <= kAlignThreads / 2
    const int cpg = (nchunks + G - 1) / G;
    if (tid < G * E) {
      const int g = tid / E, e = tid % E;
      int sum = 0, before = 0;
      sum_chunks(e, g * cpg, min(nchunks, (g + 1) * cpg), sum, before);
      part_sum[tid] = sum;
      part_before[tid] = before;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) {
      int run = 0, mine = 0;
      for (int g = 0; g < G; ++g) {
        run += part_sum[g * E + e];
        mine += part_before[g * E + e];
      }
      cnt[e] = run;
      base[e] = mine;
      if (lead) counts[e] = run;
    }
  }
  __syncthreads();
  if (tid < kWave) scan_experts(cnt, E, BM, seg_start, tile_start, lead ? offsets : nullptr, num_tiles);
  __syncthreads();
  if (lead) {                                          // the whole workgroup takes this branch or none of it
    if (tid == 0) total_tiles = tile_start[E - 1] + (cnt[E - 1] + BM - 1) / BM;
    __syncthreads();
    fill_tiles(cnt, tile_start, E, BM, P, total_tiles, sorted_pairs, tile_expert, tile_rows);
  }
  count_range(ev, hist[wave]);
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = base[e];
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = hist[w][e];
      hist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  scatter_range(ev, beg, BM, nbits_of(E), hist[wave], seg_start, tile_start, order, sorted_pairs);
}

int64_t align_scratch_ints(int64_t num_pairs, int64_t num_experts) {
  const int64_t nchunks = (num_pairs + kChunk - 1) / kChunk;
  return nchunks <= 1 ? 0 : nchunks * num_experts + num_experts;
}

hipError_t launch_align(const int32_t* ids, int64_t num_pairs, int64_t num_experts, int64_t block_m,
                        int32_t* counts, int32_t* offsets, int32_t* order, int32_t* sorted_pairs,
                        int32_t* tile_expert, int32_t* tile_rows, int32_t* num_tiles, int32_t* scratch,
                        hipStream_t s) {
  const int P = (int)num_pairs, E = (int)num_experts, BM = (int)block_m;
  const int nchunks = (P + kChunk - 1) / kChunk;
  if (nchunks <= 1) {
    hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, P, E, BM, counts, offsets,
                       order, sorted_pairs, tile_expert, tile_rows, num_tiles);
    return hipGetLastError();
  }
  int32_t* chunk_counts = scratch;
  hipLaunchKernelGGL(align_count_kernel, dim3(nchunks), dim3(kAlignThreads), 0, s, ids, P, E, chunk_counts);
  hipLaunchKernelGGL(align_scan_scatter_kernel, dim3(nchunks), dim3(kAlignThreads), 0, s, ids, P, E, BM, nchunks,
                     chunk_counts, counts, offsets, order, sorted_pairs, tile_expert, tile_rows, num_tiles);
  return hipGetLastError();
}

}  // namespace moe
