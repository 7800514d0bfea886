// Grouped expert products of the MoE block.
//
//   gate/up: for every tile row r holding pair p (token p / k, expert e)
//              act[r, i] = silu(x[tok] . Wg[e, i]) * (x[tok] . Wu[e, i])
//   down:    y[p, h] = scale[p] * (act[r] . Wd[e, h])
//
// Dense mode (no grouping: every row of x through one weight set) serves the
// shared expert and dense SwiGLU layers; its down product takes a per-row
// scale, or none.
//
// "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert", 题面速览 (expert
// formula, one product per expert over its gathered tokens) and L1 细节
// (Wg, Wu are [I, H], Wd is [H, I]); the gate rows precede the up rows in the
// packed gate/up weight.  The routing-weight multiply in the down epilogue is
// the expert-output scaling of the nano-vLLM Qwen3-30B-A3B notes
// (lshu.cn/news/442807), qwen3_moe.py, Qwen3MoeSparseMoeBlock forward.
//
// Tiles come from the align kernel: tile t is rows [t*BM, (t+1)*BM) of the
// padded pair list, all of one expert.  The launch covers an upper bound of
// tiles; workgroups past the device-side tile count return at once, so the
// host never reads the count.
//
// Scan mode (small batches, 16-row tiles): no align kernel.  Workgroup
// (expert e, column block) copies the top-k ids into its A ring while its
// first weight stages load, and lists the pairs p with ids[p] == e in
// increasing p: the align kernel's stable order.  It then runs those rows 16
// at a time (one pass for nearly every expert at decode sizes), reading act
// and writing act / y at the pair index p.  A row's products are the same
// instructions in the same K order as in the grouped tiles, so act, y and the
// block's output are bit for bit those of the grouped path.
//
// bf16 kernel (gfx950): C = A . B^T with A gathered rows [BM, K] and B the
// expert's weight rows [BN, K], both K-contiguous.  64-wide K steps go from
// global memory straight into LDS (16-byte-per-lane DMA), 2-3 steps ahead of
// the matrix cores, one barrier per step; 128-byte rows with their 16-byte
// chunks XOR-swizzled by row so fragment reads hit distinct banks.  Each wave
// owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 16x16x32 bf16 MFMAs with
// float32 accumulators.  For gate/up a B tile holds BN/2 gate rows and the
// matching BN/2 up rows, and each wave holds matching gate and up columns in
// the same lanes, so the SwiGLU is computed in registers.  Launch order puts
// the tiles of one expert and column block next to each other on one XCD, so
// they meet the same weight tile in that XCD's L2.  Each expert starts its K
// loop at its own stage (stride ROT), so concurrent workgroups spread over
// HBM channels.  Weights are row-major or in the blocked layout of
// moe_pack_weights (BLK: only the weight addresses differ); a weight tile that
// one row tile reads alone is streamed with the non-temporal hint.
//
// fp32 kernel: plain FMA loops, any shape (used for float32 layers).
#include <cmath>
#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

constexpr int kDmaBytes = 64 * 16;      // one wave-wide DMA: 16 bytes per lane

enum { kGateUp = 0, kDown = 1 };

typedef __attribute__((address_space(3))) uint16_t lds_u16_t;

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u16_t*)p));
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_base + 16*i (lds_base wave-uniform, in M0).  Issued as inline
// assembly so that the compiler does not serialise the pipeline with its own
// conservative waits on LDS DMA; completion is tracked by hand with vmcnt
// (vector-memory loads complete in issue order).
__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// The same DMA marked non-temporal, for expert weights that only one row
// tile reads: their lines should not push the reused rows (gathered x, act)
// out of the caches.  Measured at 64 tokens: down 78 -> 69 us, gate/up
// 132 -> 124 us; at 4096 tokens: gate/up 226 -> 223 us, down 147 -> 135 us.
// Weights that several row tiles read (heavy experts of a skewed batch, the
// dense products) keep the normal policy: there the hint costs 3-8%.
__device__ __forceinline__ void dma16_nt(const uint16_t* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// Wait until at most n vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Element offset of 16-byte chunk `chunk` of row `row` in a staged tile of
// BK-element rows.  The chunk index is XOR-ed with bits of the row so that
// the 8 lanes of one LDS read phase (8 consecutive rows, one chunk column)
// land in 8 different 16-byte bank groups of a 128-byte bank window:
// 128-byte rows (BK = 64) use the row's low 3 bits; 64-byte rows (BK = 32)
// pair rows (two rows fill a window) and use bits 1-2.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (BK == 64) return row * BK + ((chunk ^ (row & 7)) << 3);
  else return row * BK + ((chunk ^ ((row >> 1) & 3)) << 3);
}


constexpr int kRot = 13;   // K-start stride of every grouped product (see the launchers)

// The grid may cover two problems of the same mode and tile shape (the routed
// experts and the shared expert's dense rows): workgroups below blocks0 take
// g0, the others g1; each workgroup's arithmetic is that of a launch of its
// problem alone.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int SA, int SB, int MODE, bool BLK, int ROT, int SCAN>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void grouped_gemm_bf16_kernel(GemmProblem g0, GemmProblem g1,
                                                                                    int blocks0) {
  const bool second = (int)blockIdx.x >= blocks0;
  const GemmProblem& g = second ? g1 : g0;
  const int bid = second ? (int)blockIdx.x - blocks0 : (int)blockIdx.x;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(!BLK || BK == 64, "blocked weights come in 64-column blocks, one per stage");
  constexpr int kCpr = BK / 8;                      // 16-byte chunks per staged row
  constexpr int kRowsPerDma = kDmaBytes / (BK * 2); // rows one wave-wide DMA fills
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M;
  constexpr int WN = BN / WAVES_N;
  constexpr int TM = WM / 16;
  constexpr int TN = WN / 16;
  // Wave-wide DMAs per stage: NA_DMA for the A tile, NB_DMA for the weight
  // tile.  DMA gi goes to wave gi % NW, so waves below the remainder issue
  // one more than the others.
  constexpr int NA_DMA = BM / kRowsPerDma, NB_DMA = BN / kRowsPerDma;
  constexpr int kAFull = NA_DMA / NW, kARem = NA_DMA % NW;
  constexpr int kBFull = NB_DMA / NW, kBRem = NB_DMA % NW;
  constexpr int A_PER_WAVE = kAFull + (kARem ? 1 : 0);
  constexpr int B_PER_WAVE = kBFull + (kBRem ? 1 : 0);
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(MODE != kGateUp || TN % 2 == 0, "gate/up needs matching gate and up sub-tiles");
  static_assert(NA_DMA * kRowsPerDma == BM && NB_DMA * kRowsPerDma == BN,
                "tile rows must fill whole DMAs");
  static_assert(SA >= 2 && SA <= 5 && SB >= SA && SB <= 6, "ring depths");

  // Two rings: SA stages of the A tile and SB > SA stages of the weight
  // tile, in one LDS block (the epilogue reuses all of it).
  constexpr int kAStage = BM * BK;                  // elements
  constexpr int kBStage = BN * BK;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SA * kAStage + SB * kBStage];
  uint16_t* const ring_a = smem;
  uint16_t* const ring_b = smem + SA * kAStage;
  // Down: output row (pair index) and routing weight of every tile row,
  // loaded once at the start so the epilogue reads them from LDS.
  __shared__ int32_t ep_row[MODE == kDown ? BM : 1];
  __shared__ float ep_scale[MODE == kDown ? BM : 1];
  // Scan mode (16-row tiles only): the current pass's pairs, and the
  // per-wave match counts of the scan.
  static_assert(!SCAN || BM == 16, "scan mode runs 16-row passes");
  // SCAN 1: scan mode; 2: scan mode for the problem with top-k ids, and
  // a plain dense problem (the shared expert) beside it.
  const bool scan = SCAN == 1 || (SCAN == 2 && g.topk_ids != nullptr);
  __shared__ int32_t scan_rows[SCAN ? BM : 1];
  __shared__ int32_t scan_count[SCAN ? NW : 1];

  const bool grouped = SCAN == 0 && g.sorted_pairs != nullptr;
  const int half = BN / 2;
  const int n_tiles_n = (MODE == kGateUp) ? (g.n_out + half - 1) / half : (g.n_out + BN - 1) / BN;
  // Workgroups past the real number of tiles leave at once; the others are
  // ordered column-block-fastest and chunked per XCD, so one XCD runs all
  // column blocks of a few consecutive row tiles together: they share the
  // gathered A rows and (row tiles of one expert) the expert's weights in
  // that XCD's L2.
  const int m_tiles = grouped ? *g.num_tiles : (scan ? g.num_experts : (g.dense_rows + BM - 1) / BM);
  const int n_blocks = m_tiles * n_tiles_n;
  if (bid >= n_blocks) return;
  const int logical = xcd_swizzle(bid, n_blocks);
  const int mt = logical / n_tiles_n;
  const int nt = logical % n_tiles_n;
  int rows_valid, expert;
  if (grouped) {
    rows_valid = g.tile_rows[mt];
    expert = g.tile_expert[mt];
  } else if (scan) {
    rows_valid = 0;                                    // set by each pass
    expert = mt;
  } else {
    rows_valid = min(BM, g.dense_rows - mt * BM);
    expert = 0;
  }
  const int row0 = mt * BM;
  const int K = g.K;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.a);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.b) + (int64_t)expert * g.expert_stride;
  const int64_t b_rows = (MODE == kGateUp) ? 2 * (int64_t)g.n_out : g.n_out;

  // Sources of this lane's 16-byte pieces.  DMA q of this wave fills staged
  // rows [R gi, R gi + R) of its ring stage, gi = wave + NW q, R rows per
  // DMA; lane i lands in row R gi + i / kCpr, slot i % kCpr, which holds
  // chunk swz^-1(slot) of that row.
  const uint16_t* src_a[A_PER_WAVE];
  const uint16_t* src_b[B_PER_WAVE];
#pragma unroll
  for (int q = 0; q < A_PER_WAVE; ++q) {
    src_a[q] = A;
    if (wave + NW * q >= NA_DMA) continue;             // this wave has no DMA q
    const int r = (wave + NW * q) * kRowsPerDma + lane / kCpr;
    const int chunk = (swz<BK>(r, lane % kCpr) - r * BK) >> 3;   // the swizzle is its own inverse
    int64_t src_row;
    if (MODE == kGateUp) {
      if (grouped) {
        const int pr = g.sorted_pairs[row0 + r];
        src_row = (pr < g.num_pairs) ? pr / g.top_k : 0;     // sentinel rows read token 0
      } else {
        src_row = min(row0 + r, g.dense_rows - 1);
      }
    } else {
      // Padding rows of a grouped tile were never written: they read a real
      // row of the same tile instead (already on its way for another lane),
      // not HBM.  Their results are dropped.  Fetched per launch (counter
      // passes): prefill layer 456.2 MB against 468.8, talker 511.3 against
      // 536.2, skew 924.5 against 955.0; whole forward 213.9 / 228.1 /
      // 901.2 us against 215.1 / 228.8 / 904.0 at 400 / 640 / 8192 tokens
      // (talker), prefill unchanged.  Reading the last real row for all of
      // them instead cost prefill 1-3 us.
      src_row = grouped ? (row0 + (r < rows_valid ? r : r % max(rows_valid, 1)))
                        : min(row0 + r, g.dense_rows - 1);
    }
    src_a[q] = A + src_row * K + chunk * 8;
  }
#pragma unroll
  for (int q = 0; q < B_PER_WAVE; ++q) {
    src_b[q] = B;
    if (wave + NW * q >= NB_DMA) continue;
    const int j = (wave + NW * q) * kRowsPerDma + lane / kCpr;
    const int chunk = (swz<BK>(j, lane % kCpr) - j * BK) >> 3;
    int64_t wrow;
    if (MODE == kGateUp)                             // past the last column: reread a valid row
      wrow = (j < half) ? min((int64_t)nt * half + j, (int64_t)g.n_out - 1)
                        : min((int64_t)g.n_out + nt * half + (j - half), b_rows - 1);
    else
      wrow = min((int64_t)nt * BN + j, b_rows - 1);
    // Row-major: row wrow starts at wrow * K.  Blocked: each 64-column
    // panel holds all b_rows rows, 64 elements each, so row wrow starts at
    // wrow * 64 in every panel; issue_b adds the panel offset (stage start
    // times b_rows).
    src_b[q] = (BLK ? B + wrow * 64 : B + wrow * K) + chunk * 8;
  }

  const int nk = K / BK;
  // The K loop starts at stage kstart = (ROT * expert) mod nk and wraps
  // around.  Rows of 2^n bytes put every stage-kt load of every workgroup on
  // the same low address bits, and so on the same few HBM channels, if all
  // workgroups walk K in step; rotating the start by expert spreads them,
  // while the column blocks of one expert stay in step and keep sharing its
  // A rows in L2.  The stride is the same for every tile shape and the
  // start depends only on the expert, so every output element keeps one
  // summation order whatever the batch.
  const int kstart = (expert * ROT) % nk;
  auto kpos = [&](int kt) { const int k = kt + kstart; return (k >= nk ? k - nk : k) * BK; };
  auto issue_a = [&](int kt) {
    const uint32_t base = lds_addr(ring_a + (kt % SA) * kAStage);
    const int ko = kpos(kt);
#pragma unroll
    for (int q = 0; q < A_PER_WAVE; ++q)
      if (q < kAFull || wave < kARem) dma16(src_a[q] + ko, base + (wave + NW * q) * kDmaBytes);
  };
  // Is this weight tile read by another row tile too?  Tiles of one expert
  // are consecutive in the grouping.
  const bool shared_b = grouped ? ((mt > 0 && g.tile_expert[mt - 1] == expert) ||
                                   (mt + 1 < m_tiles && g.tile_expert[mt + 1] == expert))
                                : (!scan && m_tiles > 1);
  auto issue_b = [&](int kt) {
    const uint32_t base = lds_addr(ring_b + (kt % SB) * kBStage);
    const int64_t ko = BLK ? kpos(kt) * b_rows : kpos(kt);
    if (shared_b) {
#pragma unroll
      for (int q = 0; q < B_PER_WAVE; ++q)
        if (q < kBFull || wave < kBRem) dma16(src_b[q] + ko, base + (wave + NW * q) * kDmaBytes);
    } else {
#pragma unroll
      for (int q = 0; q < B_PER_WAVE; ++q)
        if (q < kBFull || wave < kBRem) dma16_nt(src_b[q] + ko, base + (wave + NW * q) * kDmaBytes);
    }
  };
  // Waits.  Each iteration issues the A DMAs of stage kt + SA - 1 and the
  // weight DMAs of stage kt + SB - 1; with SB > SA the A DMAs go first, with
  // SB == SA last, so either way a stage's A DMAs are issued no earlier than
  // its weight DMAs.  Vector-memory loads complete in issue order, so once
  // only the loads issued after stage kt's A DMAs are in flight, the whole
  // stage has landed.  With SB > SA those are the weight DMAs of the same
  // iteration plus SA - 2 whole iterations; with SB == SA, SA - 2 whole
  // iterations.  The first SA - 1 stages come from the prologue (weights
  // first, then A).  Near the end of the loop, where issues stop, and for
  // short loops, the wait is for everything.
  // The counts below are this wave's DMAs per stage (a_ for A, b_ for the
  // weights), which differ between waves when the DMAs do not split evenly.
  constexpr bool kAFirst = SB > SA;
  static_assert((kAFirst ? B_PER_WAVE : 0) + (SA - 2) * (A_PER_WAVE + B_PER_WAVE) < 64, "vmcnt range");
  auto wait_counts = [&](int kt, auto a_tag, auto b_tag) {
    constexpr int a_ = decltype(a_tag)::value, b_ = decltype(b_tag)::value;
    constexpr int kSteady = (kAFirst ? b_ : 0) + (SA - 2) * (a_ + b_);
    if (nk < SB - 1 || kt + SB - 2 >= nk) { wait_vmcnt<0>(); return; }
    if (kt >= SA - 1) { wait_vmcnt<kSteady>(); return; }
    // kt < SA - 1: stage kt's A DMAs came from the prologue, followed there by
    // those of stages kt+1 .. SA-2 and then by kt whole iterations.
    auto early = [&](auto k_tag) {
      constexpr int k = decltype(k_tag)::value;
      wait_vmcnt<(SA - 2 - k) * a_ + k * (a_ + b_)>();
    };
    if (kt == 0) early(std::integral_constant<int, 0>{});
    else if (kt == 1) early(std::integral_constant<int, (SA > 2 ? 1 : 0)>{});
    else if (kt == 2) early(std::integral_constant<int, (SA > 3 ? 2 : 0)>{});
    else early(std::integral_constant<int, (SA > 4 ? 3 : 0)>{});
  };
  auto wait_stage = [&](int kt) {
    using AF = std::integral_constant<int, kAFull>;
    using AX = std::integral_constant<int, kAFull + 1>;
    using BF = std::integral_constant<int, kBFull>;
    using BX = std::integral_constant<int, kBFull + 1>;
    const bool ax = wave < kARem, bx = wave < kBRem;
    if (ax && bx) wait_counts(kt, AX{}, BX{});
    else if (ax) wait_counts(kt, AX{}, BF{});
    else if (bx) wait_counts(kt, AF{}, BX{});
    else wait_counts(kt, AF{}, BF{});
  };

  // Scan mode: copy the ids into the A ring (free until the first A stage),
  // issue this pass's first weight stages, wait for the ids only (they are
  // older than the weight DMAs), then list the expert's pairs with ranks
  // [c0, c0 + BM) into scan_rows.  Thread t looks at ids [8t, 8t + 8), so the
  // ranks follow the pair index.  Returns the expert's number of pairs.
  auto scan_pass = [&](int c0) -> int {
    if constexpr (SCAN) {
      static_assert(SA * kAStage * 2 >= kScanMaxPairs * 4 && 8 * 64 * NW >= kScanMaxPairs,
                    "the ids must fit the A ring, 8 per thread");
      const int P = g.num_pairs;                       // 4 <= P <= kScanMaxPairs, P % 4 == 0 (launcher)
      const uint32_t ids_lds = lds_addr(ring_a);
      for (int gi = wave; gi < (P + 255) / 256; gi += NW)
        dma16(reinterpret_cast<const uint16_t*>(g.topk_ids + min(gi * 256 + lane * 4, P - 4)),
              ids_lds + gi * kDmaBytes);
      for (int st = 0; st < min(SB - 1, nk); ++st) issue_b(st);
      if (nk >= SB - 1) {
        if (wave < kBRem) wait_vmcnt<(SB - 1) * (kBFull + 1)>();
        else wait_vmcnt<(SB - 1) * kBFull>();
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
      const int32_t* ids = reinterpret_cast<const int32_t*>(ring_a);
      const int p0 = threadIdx.x * 8;
      int c = 0;
      uint32_t bits = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p0 + u < P && ids[p0 + u] == expert) {
          bits |= 1u << u;
          ++c;
        }
      int incl = c;                                    // inclusive prefix over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      if (lane == 63) scan_count[wave] = incl;
      __syncthreads();
      int rank = incl - c, total = 0;
      for (int w = 0; w < NW; ++w) {
        const int t = scan_count[w];
        if (w < wave) rank += t;
        total += t;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if ((bits >> u) & 1u) {
          const int r = rank++ - c0;
          if (r >= 0 && r < BM) scan_rows[r] = p0 + u;
        }
      __syncthreads();                                 // scan_rows written; the ids are no longer read
      rows_valid = min(BM, max(0, total - c0));
      return total;
    }
    return 0;
  };

  floatx4 acc[TM][TN];
  // One pass over the tile's rows (scan mode: one per BM pairs of the expert).
  for (int c0 = 0, scan_total = 0;; c0 += BM) {
  if (scan) {
    scan_total = scan_pass(c0);
    if (c0 >= scan_total) {                            // nothing (left) for this expert
      wait_vmcnt<0>();                                 // the weight stages have landed
      break;
    }
    // Sources of this lane's A pieces: the pass's pairs (rows past them read pair 0).
#pragma unroll
    for (int q = 0; q < A_PER_WAVE; ++q) {
      src_a[q] = A;
      if (wave + NW * q >= NA_DMA) continue;
      const int r = (wave + NW * q) * kRowsPerDma + lane / kCpr;
      const int chunk = (swz<BK>(r, lane % kCpr) - r * BK) >> 3;
      const int pr = r < rows_valid ? scan_rows[r] : 0;
      src_a[q] = A + (int64_t)((MODE == kGateUp) ? pr / g.top_k : pr) * K + chunk * 8;
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Row groups: the tile's 16-row groups are dealt to the wave rows in turn
  // (group wm + WAVES_M tm is this wave's tm-th), so the padding at the end
  // of a tile is spread over all waves.  Each wave computes only its groups
  // that hold real rows.
  auto group_row = [&](int tm) { return 16 * (wm + WAVES_M * tm); };
  const int groups_valid = (rows_valid + 15) / 16;
  const int tm_valid = min(TM, (max(0, groups_valid - wm) + WAVES_M - 1) / WAVES_M);

  auto b_tile_row = [&](int tn) {
    if (MODE == kGateUp) {
      constexpr int kHalfTN = TN / 2;
      const int part = tn / kHalfTN, t = tn % kHalfTN;
      return part * half + wn * (WN / 2) + t * 16 + (lane & 15);
    }
    return wn * WN + tn * 16 + (lane & 15);
  };

  // The K loop, in one copy per count of real row groups (chosen outside the
  // loop, so every body is branch-free and the accumulators stay put).
  // Waves with no real rows still issue their share of the DMAs and take
  // part in every barrier.
  auto fill_tables = [&] {
    if constexpr (MODE == kDown) {
      for (int r = threadIdx.x; r < BM; r += 64 * NW) {
        int prow = -1;
        float sc = 0.0f;
        if (r < rows_valid) {
          prow = grouped ? g.sorted_pairs[row0 + r] : (scan ? scan_rows[r] : row0 + r);
          sc = g.scale ? g.scale[prow] : 1.0f;
        }
        ep_row[r] = prow;
        ep_scale[r] = sc;
      }
    }
  };
  auto main_loop = [&](auto compute) {
    if (!scan)                                         // scan mode: issued by scan_pass
      for (int s = 0; s < min(SB - 1, nk); ++s) issue_b(s);
    for (int s = 0; s < min(SA - 1, nk); ++s) issue_a(s);
    fill_tables();                                     // in the shadow of the first stage's loads
    for (int kt = 0; kt < nk; ++kt) {
      wait_stage(kt);
      __syncthreads();
      if constexpr (kAFirst) {
        if (kt + SA - 1 < nk) issue_a(kt + SA - 1);
        if (kt + SB - 1 < nk) issue_b(kt + SB - 1);
      } else {
        if (kt + SB - 1 < nk) issue_b(kt + SB - 1);
        if (kt + SA - 1 < nk) issue_a(kt + SA - 1);
      }
      constexpr int TMV = decltype(compute)::value;
      if constexpr (TMV > 0) {
        const uint16_t* As = ring_a + (kt % SA) * kAStage;
        const uint16_t* Bs = ring_b + (kt % SB) * kBStage;
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
          const int ch = kk * 4 + (lane >> 4);
          uint4 af[TMV], bfr[TN];
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            bfr[tn] = *reinterpret_cast<const uint4*>(Bs + swz<BK>(b_tile_row(tn), ch));
#pragma unroll
          for (int tm = 0; tm < TMV; ++tm)
            af[tm] = *reinterpret_cast<const uint4*>(As + swz<BK>(group_row(tm) + (lane & 15), ch));
#pragma unroll
          for (int tm = 0; tm < TMV; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = mfma16x16x32(bfr[tn], af[tm], acc[tm][tn]);
        }
      }
    }
  };
  static_assert(TM <= 5, "the row-group dispatch covers TM <= 5");
  switch (tm_valid) {
    case 0: main_loop(std::integral_constant<int, 0>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (TM >= 2) main_loop(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (TM >= 3) main_loop(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (TM >= 4) main_loop(std::integral_constant<int, 4>{}); break;
    default: if constexpr (TM >= 5) main_loop(std::integral_constant<int, 5>{}); break;
  }

  // Epilogue.  The products were taken with the weight fragment as the MFMA's
  // row operand, so lane l holds output columns 4*(l/16) .. +3 of row l%16 of
  // each 16x16 sub-tile.  The tile is finished in registers (SwiGLU, or the
  // routing weight), packed to bf16 four columns at a time into LDS (the
  // rings are free now), then written out as whole rows with 16-byte stores.
  constexpr int OUT_COLS = (MODE == kGateUp) ? BN / 2 : BN;
  constexpr int OUT_LD = OUT_COLS + 8;                 // staged row pitch (+16 B against bank conflicts)
  // Rows staged per pass: whole row groups, as many as fit in the LDS.
  constexpr int kFitRows = (int)sizeof(smem) / (OUT_LD * 2);
  constexpr int EPI_ROWS = (kFitRows >= BM) ? BM : (kFitRows / 16) * 16;
  static_assert(EPI_ROWS >= 16, "one row group of the output tile must fit the LDS");
  constexpr int kThreads = 64 * NW;
  constexpr int CPR = OUT_COLS / 8;                    // 16-byte chunks per output row
  uint16_t* so = smem;
  const int col0 = (MODE == kGateUp) ? nt * half : nt * BN;
  uint16_t* __restrict__ C = static_cast<uint16_t*>(g.c);
  for (int e0 = 0; e0 < BM; e0 += EPI_ROWS) {
    __syncthreads();                                   // LDS free: last stage or last pass consumed
    {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        if (tm >= tm_valid || group_row(tm) < e0 || group_row(tm) >= e0 + EPI_ROWS) continue;
        const int m = group_row(tm) + (lane & 15);
        const int ml = m - e0;
        const float sc = (MODE == kDown) ? ep_scale[m] : 1.0f;
        if (MODE == kGateUp) {
          constexpr int kHalfTN = TN / 2;
#pragma unroll
          for (int t = 0; t < kHalfTN; ++t) {
            const int n = wn * (WN / 2) + t * 16 + (lane >> 4) * 4;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = silu_fast(acc[tm][t][i]) * acc[tm][t + kHalfTN][i];
            *reinterpret_cast<uint2*>(so + ml * OUT_LD + n) =
                uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
        } else {
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const int n = wn * WN + tn * 16 + (lane >> 4) * 4;
            const floatx4 a = acc[tm][tn];
            *reinterpret_cast<uint2*>(so + ml * OUT_LD + n) =
                uint2{pack_bf16x2(sc * a[0], sc * a[1]), pack_bf16x2(sc * a[2], sc * a[3])};
          }
        }
      }
    }
    __syncthreads();
    const int rows_here = min(EPI_ROWS, rows_valid - e0);
    for (int c = threadIdx.x; c < rows_here * CPR; c += kThreads) {
      const int rl = c / CPR, j = c % CPR;
      if (col0 + j * 8 >= g.n_out) continue;
      const int r = e0 + rl;
      const int64_t orow = (MODE == kGateUp) ? (scan ? scan_rows[r] : row0 + r) : ep_row[r];
      *reinterpret_cast<uint4*>(C + orow * g.n_out + col0 + j * 8) =
          *reinterpret_cast<const uint4*>(so + rl * OUT_LD + j * 8);
    }
  }
  if constexpr (SCAN == 0) {
    break;
  } else {
    if (!scan || c0 + BM >= scan_total) break;
    __syncthreads();                                   // the staged output is read; the next pass reuses the LDS
  }
  }  // passes
}

// ---------------------------------------------------------------- float32

constexpr int64_t kOneRound = 256;   // workgroups of one round at one per CU
constexpr int kF32Cols = 64;
constexpr int kF32Threads = 256;

template <int MODE>
__global__ __launch_bounds__(kF32Threads) void grouped_gemm_f32_kernel(GemmProblem g) {
  const bool grouped = g.sorted_pairs != nullptr;
  const int mt = blockIdx.x;
  const int col = blockIdx.y * kF32Cols + (threadIdx.x % kF32Cols);
  int rows_valid, expert;
  if (grouped) {
    if (mt >= *g.num_tiles) return;
    rows_valid = g.tile_rows[mt];
    expert = g.tile_expert[mt];
  } else {
    rows_valid = min(g.block_m, g.dense_rows - mt * g.block_m);
    if (rows_valid <= 0) return;
    expert = 0;
  }
  if (col >= g.n_out) return;
  const float* A = static_cast<const float*>(g.a);
  const float* B = static_cast<const float*>(g.b) + (int64_t)expert * g.expert_stride;
  float* C = static_cast<float*>(g.c);
  const int K = g.K;
  const int row0 = mt * g.block_m;
  for (int r = threadIdx.x / kF32Cols; r < rows_valid; r += kF32Threads / kF32Cols) {
    if (MODE == kGateUp) {
      int64_t tok = row0 + r;
      if (grouped) tok = g.sorted_pairs[row0 + r] / g.top_k;
      const float* xr = A + tok * K;
      const float* wg = B + (int64_t)col * K;
      const float* wu = B + (int64_t)(g.n_out + col) * K;
      float gv = 0.f, uv = 0.f;
      for (int h = 0; h < K; ++h) {
        gv = fmaf(xr[h], wg[h], gv);
        uv = fmaf(xr[h], wu[h], uv);
      }
      C[(int64_t)(row0 + r) * g.n_out + col] = silu_f32(gv) * uv;
    } else {
      const int64_t prow = grouped ? g.sorted_pairs[row0 + r] : row0 + r;
      const float* ar = A + (int64_t)(row0 + r) * K;
      const float* wd = B + (int64_t)col * K;
      float acc = 0.f;
      for (int i = 0; i < K; ++i) acc = fmaf(ar[i], wd[i], acc);
      C[prow * g.n_out + col] = g.scale ? g.scale[prow] * acc : acc;
    }
  }
}

// ---------------------------------------------------------------- weight packing
// dst (blocked) from src (row-major [batch, rows, cols]): each thread moves one
// 16-byte piece (8 elements of one row inside one 64-column panel).
__global__ __launch_bounds__(256) void pack_weights_bf16_kernel(const uint16_t* __restrict__ src,
                                                                uint16_t* __restrict__ dst, int64_t pieces,
                                                                int64_t rows, int64_t cols) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int64_t per_row = cols / 8;
  const int64_t r_all = i / per_row;                 // batch * rows + row
  const int64_t c = (i % per_row) * 8;               // first column of the piece
  const int64_t b = r_all / rows, r = r_all % rows;
  const int64_t d = b * rows * cols + (c >> 6) * (rows * 64) + r * 64 + (c & 63);
  *reinterpret_cast<uint4*>(dst + d) = *reinterpret_cast<const uint4*>(src + r_all * cols + c);
}

hipError_t launch_pack_weights(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols,
                               hipStream_t s) {
  const int64_t pieces = batch * rows * cols / 8;
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weights_bf16_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                     (const uint16_t*)src, (uint16_t*)dst, pieces, rows, cols);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

// Workgroups of one problem's launch with BN-wide tiles: row tiles times
// column blocks (a gate/up tile covers BN / 2 gate and as many up columns).
template <int BN, int MODE>
static int64_t blocks_of(const GemmProblem& g) {
  const int n_tiles_n = (MODE == kGateUp) ? (g.n_out + BN / 2 - 1) / (BN / 2) : (g.n_out + BN - 1) / BN;
  return (int64_t)g.max_tiles * n_tiles_n;
}

// ROT: K-start stride, kRot for every tile shape and both weight layouts,
// so every output element is summed in one order whatever the tile height:
// a token's output does not depend on the batch it comes in, nor on the
// weight layout.  Measured with blocked weights: 16-row tiles at 64 tokens,
// gate/up 116.6 -> 115.2 us and down 60.7 -> 59.9 us from stride 5 to 13
// (row-major 116.6 -> 117.3 and 63.1 -> 62.2 us); moe_forward with the
// 32-, 64-, 128- and 320-row tiles (512 to 16384 tokens) within 1.2 us of
// strides 7 and 5.
// SCAN: 1 for the small-batch products that scan the top-k ids (16-row
// tiles); 2 for such a product with a dense problem beside it (either
// order), a separate instance so that the scan-only kernel keeps its code.
// g1 (optional, max_tiles 0 for none) must have the same mode, tile height
// and weight layout as g0; its workgroups follow g0's, from a multiple of 8
// (the XCD count) so each problem keeps its own XCD-aware tile order.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int SA, int SB, int MODE, int ROT = kRot, int SCAN = 0>
static hipError_t launch_bf16(const GemmProblem& g0, const GemmProblem& g1, hipStream_t s) {
  if (g0.block_m != BM || (g1.max_tiles && g1.block_m != BM)) return hipErrorInvalidValue;
  if (g1.max_tiles && g1.weights_blocked != g0.weights_blocked) return hipErrorInvalidValue;
  int64_t blocks0 = blocks_of<BN, MODE>(g0);
  const int64_t blocks1 = g1.max_tiles ? blocks_of<BN, MODE>(g1) : 0;
  if (blocks1) blocks0 = (blocks0 + 7) / 8 * 8;
  const int64_t blocks = blocks0 + blocks1;
  if (blocks == 0) return hipSuccess;
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * WAVES_M * WAVES_N);
  if (g0.weights_blocked)
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, BK, WAVES_M, WAVES_N, SA, SB, MODE, true, ROT, SCAN>),
                       grid, block, 0, s, g0, g1, (int)blocks0);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, BK, WAVES_M, WAVES_N, SA, SB, MODE, false, ROT, SCAN>),
                       grid, block, 0, s, g0, g1, (int)blocks0);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const GemmProblem& g, const GemmProblem& g1, hipStream_t s) {
  const GemmProblem& sp = (g1.max_tiles && g1.topk_ids) ? g1 : g;   // the scan problem, if any
  if (sp.topk_ids && !sp.sorted_pairs &&
      (sp.dtype != MOE_BF16 || sp.block_m != 16 || sp.max_tiles != sp.num_experts || sp.num_pairs < 4 ||
       sp.num_pairs > kScanMaxPairs || sp.num_pairs % 4 != 0))
    return hipErrorInvalidValue;                       // outside what scan mode is built for
  if (g1.max_tiles && (g.dtype != MOE_BF16 || g1.dtype != MOE_BF16 || (g.topk_ids && g1.topk_ids) ||
                       ((g.topk_ids || g1.topk_ids) && (g.sorted_pairs || g1.sorted_pairs))))
    return hipErrorInvalidValue;                       // pairs: bf16 tiles; a scan problem pairs with a dense one
  if (g.dtype == MOE_F32) {
    const dim3 grid(g.max_tiles, (g.n_out + kF32Cols - 1) / kF32Cols);
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<MODE>, grid, dim3(kF32Threads), 0, s, g);
    return hipGetLastError();
  }
  if (sp.topk_ids && !sp.sorted_pairs) {
    // Scan mode: one workgroup per (expert, column block) whatever the
    // routing, so the tile width sets the number of workgroup rounds
    // directly.  Measured at 32 / 64 / 128 tokens (H=2048, E=128, top-8,
    // blocked weights), against 16x128 tiles for both products:
    //   gate/up 16x256 (4 waves, 3 weight slots): 108.3 / 118.3 / 130.7 us
    //     against 109.7 / 118.7 / 132.9;
    //   down 16x256 (8 waves, 2 slots): 55.1 / 60.1 / 70.5 us against
    //     59.2 / 62.3 / 64.5: better while experts average at most 4 pairs
    //     (then nearly all take one 16-row pass), worse at 8, where the odd
    //     expert with a second pass ends the last of exactly two rounds late.
    //     With 4 waves (two workgroups per CU) and the panel weight layout,
    //     50.2 / 54.1 / 59.2 us at 24 / 32 / 64 tokens against 51.6 / 54.8 /
    //     60.0 with 8 waves.
    // Results are the same bit for bit: the tile width does not change any
    // row's arithmetic.
    if (g1.max_tiles) {
      if constexpr (MODE == kGateUp) return launch_bf16<16, 256, 64, 1, 4, 2, 3, MODE, kRot, 2>(g, g1, s);
      else if (sp.num_pairs <= 4 * sp.num_experts) return launch_bf16<16, 256, 64, 1, 4, 2, 2, MODE, kRot, 2>(g, g1, s);
      else return launch_bf16<16, 128, 64, 1, 2, 2, 3, MODE, kRot, 2>(g, g1, s);
    }
    if constexpr (MODE == kGateUp) return launch_bf16<16, 256, 64, 1, 4, 2, 3, MODE, kRot, 1>(g, g1, s);
    else if (sp.num_pairs <= 4 * sp.num_experts) return launch_bf16<16, 256, 64, 1, 4, 2, 2, MODE, kRot, 1>(g, g1, s);
    else return launch_bf16<16, 128, 64, 1, 2, 2, 3, MODE, kRot, 1>(g, g1, s);
  }
  // Grouped launches (the routed experts, alone or with the shared expert's
  // tiles) take 8 waves at 32 and 64 rows; dense launches keep the shapes
  // below.  Whole forward, H=2048, E=128, top-8, I=768, blocked weights:
  // 160 / 256 tokens (32-row tiles) 199.9 / 205.5 us against 202.3 / 208.5
  // with 32x128 tiles of 4 waves; 400 / 640 tokens (64-row tiles) 215.4 /
  // 230.8 us against 218.9 / 235.7 with 4 waves.  A dense layer (one weight,
  // few row tiles) lost up to 30% with them: 32x256 tiles halve its
  // workgroups.  A dense down launch at 16 and 32 rows takes 64-column
  // tiles (twice the workgroups over its long K): dense layer (H=2048,
  // I=6144) at 16 / 32 / 64 tokens 52.0 / 53.2 / 54.3 us against 58.5 /
  // 56.4 / 55.3 with 128 columns.  While such a launch has at most one
  // workgroup per CU, each workgroup's 96 K stages are bound by load
  // latency, so it keeps three A stages and five weight stages in flight (4
  // and 6 slots): the same layer at 16 / 64 / 128 / 256 tokens 45.4 / 47.2
  // / 60.3 / 63.0 us against 52.1 / 54.4 / 68.3 / 73.1 with 2 and 4 slots,
  // 49.4 / 49.0 / 61.8 / 64.3 with 3 and 6, 49.1 / 48.2 / 61.1 / 63.4 with
  // 5 and 6.  Only the A ring's depth counts: 2 and 6 slots gave 51.8 /
  // 55.6 / 68.4 / 73.7.  Past 256 workgroups the deeper rings' LDS (64 KB
  // against 40 at 32 rows) cuts the workgroups a CU holds from three to two,
  // and co-resident workgroups hide the latency anyway: at 768 tokens (768
  // workgroups) 132.0 us against 102.8 with 2 and 4 slots.  Past three
  // workgroups per CU a 32-row launch takes 128-column tiles (two per CU)
  // rather than a second round: 896 / 1024 tokens 102.0 / 105.2 us against
  // 134.6 / 140.3 with 64 columns.  A dense gate/up launch of one round at
  // 16 and 32 rows keeps three A stages in flight too (4 A and 4 weight
  // slots): the layer at 16 / 32 / 64 tokens 42.9 / 45.6 / 46.7 us against
  // 44.7 / 46.3 / 47.3, the talker layer (with the shared expert on dense
  // tiles) at 32 / 64 / 128 tokens 199.3 / 214.9 / 235.4 us against 200.7 /
  // 215.8 / 238.4.  A 16-row dense gate/up launch whose 64-column tiles
  // still fit one round takes them (twice the workgroups): the layer at 8 /
  // 16 tokens 38.2 / 38.8 us against 41.2 / 41.8, the talker layer at 48 /
  // 64 tokens (shared expert in launches of its own) 207.4 / 212.6 against
  // 211.3 / 215.1; at 32 rows they brought nothing.  A 16-row dense down
  // launch likewise takes 32-column tiles (2 waves) while they fit one
  // round: the layer at 1 / 8 / 16 / 24 tokens 35.5 / 35.9 / 36.7 / 42.2 us
  // against 38.3 / 38.7 / 39.0 / 45.1 with 64 columns.
  const bool grouped = g.sorted_pairs != nullptr || (g1.max_tiles && g1.sorted_pairs != nullptr);
  switch (g.block_m) {
    case 16:   // small batches; grouped down one weight slot shorter (75 -> 74 us)
      if constexpr (MODE == kGateUp) {
        if (!grouped && blocks_of<64, MODE>(g) <= kOneRound)     // 32 gate + 32 up columns per workgroup
          return launch_bf16<16, 64, 64, 1, 2, 4, 4, MODE>(g, g1, s);
        if (!grouped && blocks_of<128, MODE>(g) <= kOneRound)
          return launch_bf16<16, 128, 64, 1, 2, 4, 4, MODE>(g, g1, s);
        // Grouped, at most one round with 64-column tiles (a single token:
        // 8 experts x 24 blocks): 38.8 against 40.4 us for the whole forward.
        if (grouped && blocks_of<64, MODE>(g) + (g1.max_tiles ? blocks_of<64, MODE>(g1) : 0) <= kOneRound)
          return launch_bf16<16, 64, 64, 1, 2, 2, 4, MODE>(g, g1, s);
        return launch_bf16<16, 128, 64, 1, 2, 2, 4, MODE>(g, g1, s);
      } else if (!grouped) {
        if (blocks_of<32, MODE>(g) <= kOneRound) return launch_bf16<16, 32, 64, 1, 2, 4, 6, MODE>(g, g1, s);
        if (blocks_of<64, MODE>(g) <= kOneRound) return launch_bf16<16, 64, 64, 1, 4, 4, 6, MODE>(g, g1, s);
        return launch_bf16<16, 64, 64, 1, 4, 2, 4, MODE>(g, g1, s);
      }
      return launch_bf16<16, 128, 64, 1, 2, 2, 3, MODE>(g, g1, s);
    case 32:
      if (grouped) return launch_bf16<32, 256, 64, 2, 4, 2, 3, MODE>(g, g1, s);
      if constexpr (MODE == kDown) {
        const int64_t b = blocks_of<64, MODE>(g);
        if (b <= kOneRound) return launch_bf16<32, 64, 64, 1, 4, 4, 6, MODE>(g, g1, s);
        if (b <= 3 * kOneRound) return launch_bf16<32, 64, 64, 1, 4, 2, 4, MODE>(g, g1, s);
        return launch_bf16<32, 128, 64, 1, 4, 2, 4, MODE>(g, g1, s);
      }
      if (blocks_of<128, MODE>(g) <= kOneRound) return launch_bf16<32, 128, 64, 1, 4, 4, 4, MODE>(g, g1, s);
      return launch_bf16<32, 128, 64, 1, 4, 2, 4, MODE>(g, g1, s);
    case 64:
      if (grouped) return launch_bf16<64, 256, 64, 2, 4, 2, 3, MODE>(g, g1, s);
      return launch_bf16<64, 256, 64, 1, 4, 2, 3, MODE>(g, g1, s);
    case 128:   // 3 A slots (144 KB): 704 / 1024 / 1280 tokens 235.5 / 246.8 / 255.4 us against 236.5 / 249.9 / 257.4
      return launch_bf16<128, 256, 64, 2, 4, 3, 3, MODE>(g, g1, s);
    case 320: return launch_bf16<320, 256, 64, 4, 2, 2, 2, MODE>(g, g1, s);
    case 256: return launch_bf16<256, 256, 64, 4, 2, 2, 2, MODE>(g, g1, s);   // dense layers
    default: return hipErrorInvalidValue;
  }
}

// Expected experts with at least one of P pairs under uniform routing, the
// routed scan launch's workgroups (one per hit expert and column block), and
// the idle slots of its last round: the shared expert's tiles join the
// launch when their work (in routed-workgroup lengths: the K ratio) fits
// there.  Workgroups per CU follow from the scan configurations above:
// gate/up 16x256 one per CU, down 16x256 two (at most 4 pairs per expert)
// or 16x128 three.  Talker layer (H=2048, E=128, top-8, I=768, I_s=2048),
// whole forward, bit for bit equal: 24 / 32 tokens (both merged) 168.1 /
// 181.3 us against 189.7 / 199.3 with separate shared launches; 80 / 96
// tokens (down merged) 209.4 / 213.3 against 217.5 / 220.8; merging a
// product that the rule keeps apart lost 2-8 us (48 / 64 tokens, gate/up
// at 80 / 96 tokens).
int scan_shared_merge(int64_t num_pairs, int64_t num_experts, int64_t num_tokens, int64_t hidden, int64_t inter,
                      int64_t shared_inter) {
  const double E = (double)num_experts, P = (double)num_pairs;
  const double hit = E * (1.0 - std::pow(1.0 - 1.0 / E, P));
  const double row_tiles = (double)((num_tokens + 15) / 16);
  auto fits = [](double routed, double per_round, double shared) {
    return shared <= std::ceil(routed / per_round) * per_round - routed;
  };
  auto cdiv = [](int64_t a, int64_t b) { return (double)((a + b - 1) / b); };
  int mask = 0;
  if (fits(hit * cdiv(inter, 128), 256, row_tiles * cdiv(shared_inter, 128))) mask |= 1;
  const bool wide = num_pairs <= 4 * num_experts;
  const int64_t cols = wide ? 256 : 128;
  if (fits(hit * cdiv(hidden, cols), wide ? 512 : 768,
           row_tiles * cdiv(hidden, cols) * (double)shared_inter / (double)inter))
    mask |= 2;
  return mask;
}

static const GemmProblem kNoProblem{};

hipError_t launch_gate_up(const GemmProblem& g, hipStream_t s) { return launch_mode<kGateUp>(g, kNoProblem, s); }
hipError_t launch_down(const GemmProblem& g, hipStream_t s) { return launch_mode<kDown>(g, kNoProblem, s); }
hipError_t launch_gate_up_pair(const GemmProblem& g0, const GemmProblem& g1, hipStream_t s) {
  return launch_mode<kGateUp>(g0, g1, s);
}
hipError_t launch_down_pair(const GemmProblem& g0, const GemmProblem& g1, hipStream_t s) {
  return launch_mode<kDown>(g0, g1, s);
}

}  // namespace moe
