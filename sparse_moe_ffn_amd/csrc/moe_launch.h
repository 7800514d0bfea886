// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;

// Router: logits, float32 softmax, top-k, optional renormalisation and the
// optional shared-expert gate.  `scratch` holds route_scratch_floats(...)
// floats of partial logits.
int64_t route_scratch_floats(int64_t N, int64_t E, bool shared);
hipError_t launch_route(const moe_problem& p, const void* x, const void* router_w,
                        const void* shared_gate, int32_t* ids, float* w, float* shared_scale,
                        float* scratch, hipStream_t s);

// Stable grouping of the pairs by expert, padded to block_m.  `scratch`
// holds align_scratch_ints(...) int32 values (none for one chunk).
int64_t align_scratch_ints(int64_t num_pairs, int64_t num_experts);
hipError_t launch_align(const int32_t* ids, int64_t num_pairs, int64_t num_experts, int64_t block_m,
                        int32_t* counts, int32_t* offsets, int32_t* order, int32_t* sorted_pairs,
                        int32_t* tile_expert, int32_t* tile_rows, int32_t* num_tiles, int32_t* scratch,
                        hipStream_t s);

// One grouped (or dense, when sorted_pairs == nullptr) product.
struct GemmProblem {
  const void* a;               // gate/up: x [N, K];  down: act [rows, K]
  const void* b;               // expert weights, expert e at b + e * expert_stride
  const int32_t* sorted_pairs; // nullptr: dense rows 0..dense_rows-1, expert 0
  const int32_t* tile_expert;
  const int32_t* tile_rows;
  const int32_t* num_tiles;
  const float* scale;          // down only: per-pair (grouped) or per-row (dense) factor; nullptr: 1
  void* c;                     // gate/up: act [rows, Nout];  down: y [pairs or rows, Nout]
  int64_t expert_stride;       // elements
  int32_t K;                   // reduction length
  int32_t n_out;               // gate/up: I (act columns);  down: H
  int32_t top_k;
  int32_t num_pairs;           // sentinel value
  int32_t dense_rows;
  int32_t block_m;
  int32_t max_tiles;
  int32_t dtype;               // MOE_F32 / MOE_BF16
  int32_t weights_blocked;     // b in the blocked layout of moe_pack_weights (bf16 only)
  // Scan mode (sorted_pairs == nullptr, topk_ids != nullptr; bf16, block_m 16,
  // max_tiles = num_experts, 4 <= num_pairs <= kScanMaxPairs, num_pairs % 4 == 0):
  // workgroup e lists the pairs with topk_ids[p] == e itself; act and y rows
  // are pair indices.
  const int32_t* topk_ids;
  int32_t num_experts;
};

constexpr int kScanMaxPairs = 1024;   // ids that fit the 16-row tile's A ring (and 8 per thread)

hipError_t launch_gate_up(const GemmProblem& g, hipStream_t s);
hipError_t launch_down(const GemmProblem& g, hipStream_t s);
// Two problems in one launch (bf16, same tile height and weight layout): the
// routed experts' tiles (grouped, or in scan mode with 16-row tiles) and the
// shared expert's dense rows, in either order.
hipError_t launch_gate_up_pair(const GemmProblem& g0, const GemmProblem& g1, hipStream_t s);
hipError_t launch_down_pair(const GemmProblem& g0, const GemmProblem& g1, hipStream_t s);
// Which scan-mode products take the shared expert's 16-row dense tiles into
// their launch: bit 0 gate/up, bit 1 down.  A product merges when the
// shared tiles' work fits the idle slots of the routed launch's last round
// of workgroups (pairs P over E experts, shared intermediate size I_s).
int scan_shared_merge(int64_t num_pairs, int64_t num_experts, int64_t num_tokens, int64_t hidden, int64_t inter,
                      int64_t shared_inter);

// Row-major bf16 [batch, rows, cols] -> the blocked layout (rows % 8 == 0,
// cols % 64 == 0).
hipError_t launch_pack_weights(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols,
                               hipStream_t s);

// residual_out = x (+ residual_in); normed = RMSNorm(residual_out) * weight.
int64_t add_rmsnorm_max_hidden();
hipError_t launch_add_rmsnorm(const void* x, const void* residual_in, void* residual_out, const void* weight,
                              void* normed, int64_t N, int64_t H, float eps, int32_t dtype, hipStream_t s);

// out[n] = sum_j y[n*k + j] (+ shared_y[n]), float32 sum in slot order.
hipError_t launch_combine(const void* y, const void* shared_y, void* out, int64_t N, int64_t H,
                          int64_t top_k, int32_t dtype, hipStream_t s);

// Matrix-unit rate probe: MOE_PROBE_WORKGROUPS workgroups of back-to-back
// bf16 matrix instructions on register operands; mfma_probe_flops gives the
// launch's flop count.
hipError_t launch_mfma_probe(const void* ops, int64_t num_ops, int64_t iters, float* sink, hipStream_t s);
double mfma_probe_flops(int64_t iters);

}  // namespace moe
