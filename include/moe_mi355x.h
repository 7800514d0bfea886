/*
 * moe_mi355x.h -- C ABI of the sparse MoE FFN block for AMD Instinct MI355X
 * (gfx950).
 *
 * The block (Qwen3-style sparse MoE FFN) is defined on the page "M03 · Sparse
 * MoE：路由、按 expert 分组计算、shared expert", section 题面速览:
 *
 *   logits = x . router_w^T                       [N, E]
 *   probs  = softmax over all E experts, float32
 *   (w, ids) = top-k of probs, descending
 *   if norm_topk_prob: w /= sum_j w
 *   out[n] = sum_j w[n,j] * Expert_{ids[n,j]}(x[n])
 *            (+ sigmoid(x[n] . g) * Shared(x[n]) for the shared-expert variant)
 *   Expert(h) = (silu(h Wg^T) * (h Wu^T)) Wd^T
 *
 * and computed "the serving way" of the same section: (token, slot) pairs
 * grouped by expert with a stable sort, one grouped product per expert over
 * its gathered tokens, and a weighted accumulation back to each token.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (HBM of the current HIP device)
 *   to dense row-major arrays; the caller owns and allocates every buffer.
 *   The library keeps no device memory between calls.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on that stream and returns; nothing synchronises the host
 *   and no buffer is read on the host, so calls can be captured in a graph.
 * - Pair index: p = n*top_k + j for token n and slot j (token-major).
 * - dtype: MOE_F32 -- x, every weight, out and the internal activations are
 *   float32 (any shapes).  MOE_BF16 -- x, every weight and out are bfloat16,
 *   all products accumulate in float32; requires hidden, inter and
 *   shared_inter to be multiples of 64 and 16-byte aligned pointers.
 * - Router logits, probabilities and routing weights are float32 in both
 *   dtypes; expert ids are int32.
 * - Return value: MOE_OK (0) or a negative MOE_E* code.  Arguments are fully
 *   validated before any HIP call; on error nothing is enqueued and
 *   moe_last_error() describes the problem.  num_tokens == 0 is valid and
 *   enqueues nothing.
 * - Limits: 1 <= top_k <= num_experts <= 512, top_k <= 32.
 * - Expert weights are row-major unless p->weight_layout is
 *   MOE_LAYOUT_BLOCKED (see moe_pack_weights); shapes below are the
 *   row-major ones.
 * - An entry point validates only the moe_problem fields it uses (moe_route:
 *   tokens, hidden, experts, top_k, dtype, norm_topk_prob; moe_gate_up and
 *   moe_down add inter; moe_shared_expert: tokens, hidden, top_k, dtype and
 *   shared_inter; moe_dense_mlp: tokens, hidden, top_k, dtype and inter;
 *   moe_combine: tokens, hidden, top_k, dtype).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer, bad shape, top_k outside [1, E] */
  MOE_ENOSPC = -2,        /* workspace too small */
  MOE_EUNSUPPORTED = -3,  /* dtype, alignment or size outside the limits */
  MOE_EHIP = -4           /* a HIP launch failed */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Storage of the expert weights (w_gate_up, w_down, and the shared-expert
 * and dense-layer weights; the router weight and the shared gate are always
 * row-major).  MOE_LAYOUT_ROW_MAJOR is the shapes as written (M03 L1 细节);
 * MOE_LAYOUT_BLOCKED is what moe_pack_weights produces (bf16 only). */
enum { MOE_LAYOUT_ROW_MAJOR = 0, MOE_LAYOUT_BLOCKED = 1 };

/* Shape and options of one MoE layer call.  A zero-initialised struct with
 * the sizes filled in means row-major weights. */
typedef struct moe_problem {
  int64_t num_tokens;      /* N  */
  int64_t hidden;          /* H  */
  int64_t num_experts;     /* E  */
  int64_t top_k;           /* k  */
  int64_t inter;           /* I  : expert intermediate size */
  int64_t shared_inter;    /* I_s: shared-expert intermediate size, 0 = none */
  int32_t dtype;           /* MOE_F32 or MOE_BF16 */
  int32_t norm_topk_prob;  /* 1: renormalise the k kept weights to sum 1 */
  int32_t weight_layout;   /* MOE_LAYOUT_ROW_MAJOR or MOE_LAYOUT_BLOCKED */
  int32_t reserved;        /* must be 0 */
} moe_problem;

/* Byte offsets of the regions moe_forward carves out of its workspace, and
 * the tile height (block_m) it groups with.  Offsets are 256-byte aligned;
 * a region of size 0 has offset equal to the previous end. */
typedef struct moe_workspace_layout {
  int64_t block_m;         /* rows per grouped-GEMM tile */
  int64_t max_rows;        /* capacity of sorted_pairs / act rows */
  int64_t max_tiles;       /* capacity of tile_expert / tile_rows */
  int64_t ids_products;    /* 1: moe_forward runs moe_gate_up_ids / moe_down_ids
                              (no grouping; act rows are pair indices) */
  int64_t shared_block_m;  /* rows per tile of the shared expert's gate/up
                              product (0 without a shared expert) */
  int64_t shared_merged;   /* products that moe_forward runs in one launch with
                              the shared expert's tiles: bit 0 gate/up, bit 1
                              down.  bf16, shared and routed tiles of one
                              height: 3 for grouped products; for the ids
                              products each one whose routed launch leaves
                              room for the shared tiles in its last round of
                              workgroups (0 otherwise) */
  size_t route_scratch, topk_ids, topk_w, shared_scale;
  size_t counts, offsets, order, sorted_pairs, tile_expert, tile_rows, num_tiles, align_scratch;
  size_t act, y, shared_act, shared_y;
  size_t total_bytes;
} moe_workspace_layout;

/* Workspace moe_forward needs for `p` (bytes) and where each region lies.
 * Pure host arithmetic; never touches the GPU. */
int moe_workspace_size(const moe_problem* p, size_t* bytes);
int moe_get_workspace_layout(const moe_problem* p, moe_workspace_layout* layout);

/* Expert weights in the blocked layout.  The pages fix only the weight
 * shapes (M03 L1 细节: Wg, Wu [I, H], Wd [H, I]); the layout is this
 * library's.  Each matrix is stored as cols/64 panels of 64 columns, one
 * after the other, and each panel holds all rows, 64 elements per row.
 * One K stage of a grouped product (64 columns of a run of weight rows)
 * is then one contiguous piece of memory instead of 128 bytes from each
 * row, 2*cols bytes apart.  The products run faster and give bit for bit
 * the same results as with row-major weights.  Meant as a one-time step
 * when the weights are loaded.
 *   src [batch, rows, cols] bf16 row-major; dst the same number of bf16
 *   elements, element (b, r, c) at
 *     b*rows*cols + (c/64)*rows*64 + r*64 + c%64.
 *   w_gate_up: batch E, rows 2I, cols H;  w_down: batch E, rows H, cols I;
 *   shared expert and dense layers: batch 1.
 * dtype must be MOE_BF16; rows % 8 == 0 and cols % 64 == 0; src and dst
 * 16-byte aligned and not overlapping.  Asynchronous on stream. */
int moe_pack_weights(int64_t batch, int64_t rows, int64_t cols, int32_t dtype,
                     const void* src, void* dst, void* stream);

/* Capacity of the padded grouping for num_pairs pairs over num_experts
 * experts with tile height block_m: max_rows = max_tiles * block_m, where
 * max_tiles = (num_pairs + min(E, num_pairs) * (block_m - 1)) / block_m.
 * Pure host arithmetic. */
int moe_align_capacity(int64_t num_pairs, int64_t num_experts, int64_t block_m,
                       int64_t* max_rows, int64_t* max_tiles);

/* Router (M03 题面速览, routing block; the nano-vLLM Qwen3-30B-A3B notes
 * (lshu.cn/news/442807), qwen3_moe.py, Qwen3MoeSparseMoeBlock forward).
 *   x          [N, H]  dtype
 *   router_w   [E, H]  dtype
 *   shared_gate [H]    dtype or NULL; if given, shared_scale[n] =
 *                      sigmoid(x[n] . shared_gate) is written (float32 [N])
 *   topk_ids   [N, k]  int32 out: experts by descending probability, equal
 *                      probabilities to the lower expert id
 *   topk_w     [N, k]  float32 out: the probabilities of those experts,
 *                      divided by their sum when norm_topk_prob is set
 *   scratch            float32 device array of moe_route_scratch_size bytes
 *                      (partial logits; overwritten, need not be cleared),
 *                      16-byte aligned in bf16
 * Logits are accumulated in float32 (8 fixed slices of H, summed in slice
 * order, so a token's routing does not depend on the batch); softmax runs
 * over all E in float32. */
int moe_route(const moe_problem* p, const void* x, const void* router_w,
              const void* shared_gate, int32_t* topk_ids, float* topk_w,
              float* shared_scale, float* scratch, void* stream);

/* Scratch moe_route needs for p (bytes).  Pure host arithmetic. */
int moe_route_scratch_size(const moe_problem* p, size_t* bytes);

/* Grouping of the N*k pairs by expert (M03 逐步图 steps 1-3: flatten, stable
 * sort by expert id, per-expert counts and segment starts; the padding to
 * the tile height is what the pages call aligning to a block).
 *   topk_ids     [N*k]       int32 in, each in [0, E)
 *   counts       [E]         int32 out: pairs per expert
 *   offsets      [E+1]       int32 out: exclusive prefix sum of counts
 *   order        [N*k]       int32 out: pair indices sorted by expert id,
 *                            ascending pair index within an expert (stable)
 *   sorted_pairs [max_rows]  int32 out: each expert's segment of `order`
 *                            padded with the sentinel N*k to a multiple of
 *                            block_m, experts ascending, empty ones skipped;
 *                            entries past the last tile are not written
 *   tile_expert  [max_tiles] int32 out: expert of tile t (rows
 *                            [t*block_m, (t+1)*block_m) of sorted_pairs)
 *   tile_rows    [max_tiles] int32 out: real (non-sentinel) rows of tile t
 *   num_tiles    [1]         int32 out: number of tiles written
 *   scratch      device array of moe_align_scratch_size bytes (may be NULL
 *                when that size is 0, i.e. up to 4096 pairs); its contents
 *                are overwritten, nothing needs to be cleared beforehand
 * Capacities come from moe_align_capacity.  block_m in [1, 1024].  Ids
 * outside [0, E) are dropped (not counted, not placed). */
int moe_align(const int32_t* topk_ids, int64_t num_tokens, int64_t top_k,
              int64_t num_experts, int64_t block_m, int32_t* counts,
              int32_t* offsets, int32_t* order, int32_t* sorted_pairs,
              int32_t* tile_expert, int32_t* tile_rows, int32_t* num_tiles,
              int32_t* scratch, void* stream);

/* Scratch moe_align needs for num_pairs pairs over num_experts experts.
 * Pure host arithmetic. */
int moe_align_scratch_size(int64_t num_pairs, int64_t num_experts, size_t* bytes);

/* Grouped gate/up product with the SwiGLU epilogue (M03 题面速览 expert
 * formula; L1 细节 weight shapes): for every tile row r holding pair p,
 *   act[r, i] = silu(x[p / k] . Wg[e, i]) * (x[p / k] . Wu[e, i]),
 * with w_gate_up[e] = [Wg[e] (rows 0..I-1); Wu[e] (rows I..2I-1)].
 *   w_gate_up [E, 2I, H] dtype;  act [max_rows, I] dtype out (sentinel rows
 *   are left unwritten).  Grouping arrays as produced by moe_align with the
 *   same block_m; max_tiles bounds the launch, *num_tiles is read on the
 *   device.  block_m: bf16 takes 16, 32, 64, 128 or 320; fp32 any in
 *   [1, 1024]. */
int moe_gate_up(const moe_problem* p, const void* x, const void* w_gate_up,
                const int32_t* sorted_pairs, const int32_t* tile_expert,
                const int32_t* tile_rows, const int32_t* num_tiles,
                int64_t block_m, int64_t max_tiles, void* act, void* stream);

/* Grouped down product with the routing-weight epilogue (M03 题面速览;
 * the nano-vLLM Qwen3-30B-A3B notes (lshu.cn/news/442807), qwen3_moe.py,
 * Qwen3MoeSparseMoeBlock forward: the expert output times its routing weight):
 * for every tile row r holding pair p,
 *   y[p, h] = topk_w[p] * (act[r] . Wd[e, h]),
 *   w_down [E, H, I] dtype;  topk_w [N*k] float32;  y [N*k, H] dtype out,
 *   every row written once. */
int moe_down(const moe_problem* p, const void* act, const void* w_down,
             const float* topk_w, const int32_t* sorted_pairs,
             const int32_t* tile_expert, const int32_t* tile_rows,
             const int32_t* num_tiles, int64_t block_m, int64_t max_tiles,
             void* y, void* stream);

/* The same two products for small batches without a grouping: each
 * (expert, column block) workgroup finds the pairs p with topk_ids[p] == e
 * itself, in increasing p (the stable order of M03 逐步图 steps 1-2), and
 * runs them 16 rows at a time.  act and y are indexed by the pair:
 *   moe_gate_up_ids:  act[p, i] = silu(x[p / k] . Wg[e, i]) * (x[p / k] . Wu[e, i])
 *   moe_down_ids:     y[p, h]   = topk_w[p] * (act[p] . Wd[e, h])
 * with e = topk_ids[p];  act [N*k, I] and y [N*k, H] dtype, every row written
 * once.  Each row is computed with the instructions and K order of the
 * grouped products at block_m 16, so act[p] and y[p] are bit for bit the
 * grouped results for the same pair.  moe_forward uses them when the
 * grouped path would take 16-row tiles.  bf16 only, with 4 <= N*k <= 1024
 * and N*k a multiple of 4 (otherwise MOE_EUNSUPPORTED); topk_ids [N, k]
 * int32, 16-byte aligned; an id outside [0, E) matches no expert, and the
 * rows of its pair are left unwritten (as moe_align drops such pairs); no
 * scratch. */
int moe_gate_up_ids(const moe_problem* p, const void* x, const void* w_gate_up,
                    const int32_t* topk_ids, void* act, void* stream);
int moe_down_ids(const moe_problem* p, const void* act, const void* w_down,
                 const int32_t* topk_ids, const float* topk_w, void* y, void* stream);

/* Shared expert (M03 题面速览, talker's shared expert; "Qwen3.5 推理全流程"
 * 2.5B formula, second term): dense over all N tokens,
 *   shared_act[n] = silu(x[n] Wg_s^T) * (x[n] Wu_s^T)        [N, I_s]
 *   shared_y[n]   = shared_scale[n] * (shared_act[n] Wd_s^T)  [N, H]
 *   shared_w_gate_up [2 I_s, H], shared_w_down [H, I_s], dtype. */
int moe_shared_expert(const moe_problem* p, const void* x,
                      const void* shared_w_gate_up, const void* shared_w_down,
                      const float* shared_scale, void* shared_act,
                      void* shared_y, void* stream);

/* Dense SwiGLU layer ("Qwen3.5 推理全流程" 2.5A Dense MLP; the nano-vLLM
 * Qwen3 notes (lshu.cn/news/442807), Qwen3MLP / Qwen3MoeMLP of the layers in
 * mlp_only_layers): the expert formula over every token, no router, no
 * routing weight -- the E = k = 1 case of the block, on the same kernels as
 * the shared expert:
 *   act[n] = silu(x[n] Wg^T) * (x[n] Wu^T)        [N, I]  (caller's scratch)
 *   out[n] = act[n] Wd^T                            [N, H]
 *   w_gate_up [2I, H] (gate rows first), w_down [H, I], all dtype.
 * Reads num_tokens, hidden, inter, top_k (any valid value) and dtype of p.
 * out and act are fully overwritten. */
int moe_dense_mlp(const moe_problem* p, const void* x, const void* w_gate_up,
                  const void* w_down, void* act, void* out, void* stream);

/* Residual add + RMSNorm in front of the block (the nano-vLLM Qwen3 notes
 * (lshu.cn/news/442807), Qwen3DecoderLayer and question 4: the norm before
 * the MLP adds the incoming activations to the residual stream, keeps the
 * sum as the new residual and returns its normalisation, in one kernel;
 * "Step 19: Real Model — Qwen3ForCausalLM", section "RMSNorm：去掉均值中心化"):
 *   residual_out[n] = x[n] + residual_in[n]   (x[n] when residual_in is NULL:
 *                     the first layer), summed in float32, rounded to dtype
 *   normed[n]       = residual_out[n] / sqrt(mean_h residual_out[n,h]^2 + eps)
 *                     * weight, float32, rounded once to dtype
 *   x, residual_in, residual_out, normed [N, H] dtype;  weight [H] dtype.
 * residual_out may be the same buffer as x or residual_in (each element is
 * read before it is written, by the same thread); normed must not overlap
 * residual_out.  hidden must be a multiple of 8 and at most 16384; eps > 0.
 * One workgroup per token with a fixed reduction order, so a token's result
 * does not depend on the batch. */
int moe_add_rmsnorm(int64_t num_tokens, int64_t hidden, int32_t dtype,
                    const void* x, const void* residual_in, void* residual_out,
                    const void* weight, float eps, void* normed, void* stream);

/* Deterministic combine (M03 逐步图 step 4 and 易错点: contributions of a
 * token's slots are added, never assigned):
 *   out[n] = sum_{j = 0..k-1} y[n*k + j]  (+ shared_y[n] if non-NULL),
 * summed in float32 in that fixed order and rounded once to dtype.
 * out [N, H] dtype is fully overwritten. */
int moe_combine(const moe_problem* p, const void* y, const void* shared_y,
                void* out, void* stream);

/* The whole block: moe_route, moe_align, moe_gate_up, moe_down,
 * [moe_shared_expert], moe_combine on one stream, in that order (for bf16
 * batches that moe_gate_up_ids takes, that reach most experts, N*k >= 1.5 E,
 * with under 9 pairs per expert, N*k < 9 E: moe_route, moe_gate_up_ids,
 * moe_down_ids, [moe_shared_expert], moe_combine, with the same output bit
 * for bit; moe_workspace_layout.ids_products says which), with every
 * intermediate in `workspace` (moe_workspace_size bytes, 256-byte aligned,
 * laid out as moe_get_workspace_layout says).  shared_w_gate_up == NULL means
 * no shared expert (then shared_w_down and shared_gate are ignored and
 * p->shared_inter must be 0). */
int moe_forward(const moe_problem* p, const void* x, const void* router_w,
                const void* w_gate_up, const void* w_down,
                const void* shared_w_gate_up, const void* shared_w_down,
                const void* shared_gate, void* out, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of the fixed scratch array behind moe_forward_noalloc (64 MiB per
 * GPU).  At the Qwen3-30B-A3B layer shape (H=2048, E=128, top-8, I=768) that
 * holds the workspace of batches up to about 800 tokens. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* The whole block without any allocation, for callers that cannot call
 * hipMalloc or take a caller workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, kernels
 * and results (bit for bit) as moe_forward, but every intermediate lives in
 * a fixed array of MOE_NOALLOC_SCRATCH_BYTES in device memory that the
 * library holds on each GPU it runs on until the process ends.
 *   - The current HIP device must be the one `stream` belongs to.  The
 *     first call on a device looks up that device's copy of the array.
 *   - A problem whose moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     is rejected with MOE_ENOSPC before any HIP call.
 *   - No hipMalloc, hipFree or other allocation happens in the call.
 *   - Every call on one GPU shares the one array, which keeps the last
 *     call's contents: calls that overlap on one GPU (several streams or
 *     host threads at once) race and must be serialised by the caller. */
int moe_forward_noalloc(const moe_problem* p, const void* x, const void* router_w,
                        const void* w_gate_up, const void* w_down,
                        const void* shared_w_gate_up, const void* shared_w_down,
                        const void* shared_gate, void* out, void* stream);

/* Matrix-unit rate probe (measurement only, not part of the block): one
 * launch of MOE_PROBE_WORKGROUPS workgroups of 8 waves, each wave running
 * `iters` rounds of 8 independent 16x16x32 bf16 matrix instructions on
 * operands it loads once from `operands` into registers; no memory traffic
 * in the loop.  The products' MFMA fractions are quoted against the
 * datasheet peak; timing this launch (events on `stream`) gives the rate the
 * part sustains with realistic, toggling data as a second reference.
 *   operands:     device, bf16, num_operands elements (>= 512, a multiple of
 *                 512), ideally random values; read only.
 *   iters:        1 .. 1048576.
 *   sink:         device, MOE_PROBE_SINK_FLOATS floats; receives per-lane sums
 *                 of the accumulators (meaningless values; they keep the loop).
 *   flops:        host; receives the launch's matrix flops
 *                 (MOE_PROBE_WORKGROUPS * 8 * 8 * iters * 16384).
 * Errors: MOE_EINVAL for null pointers or out-of-range sizes (nothing is
 * enqueued); MOE_EHIP if the launch fails. */
#define MOE_PROBE_WORKGROUPS 512
#define MOE_PROBE_SINK_FLOATS (MOE_PROBE_WORKGROUPS * 8 * 64)
int moe_mfma_probe(const void* operands, int64_t num_operands, int64_t iters, float* sink, double* flops,
                   void* stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
