// C ABI of the MoE block: argument validation, workspace layout and the
// stream-ordered launch sequence.  Every check runs on the host before any
// HIP call; no call synchronises or reads device memory on the host.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe_launch.h"
#include "moe_mi355x.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

size_t elt_size(int32_t dtype) { return dtype == MOE_BF16 ? 2 : 4; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// What a call reads of moe_problem; fields a call does not use are not checked.
enum : unsigned { kUsesExperts = 1, kUsesInter = 2, kUsesShared = 4, kUsesAll = 7 };

int check_problem(const moe_problem* p, unsigned uses = kUsesAll) {
  if (!p) return fail(MOE_EINVAL, "problem is NULL");
  if (p->num_tokens < 0) return fail(MOE_EINVAL, "num_tokens must be >= 0");
  if (p->hidden < 1) return fail(MOE_EINVAL, "hidden must be >= 1");
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "unknown dtype");
  if (p->reserved != 0) return fail(MOE_EINVAL, "reserved must be 0");
  if (p->weight_layout != MOE_LAYOUT_ROW_MAJOR && p->weight_layout != MOE_LAYOUT_BLOCKED)
    return fail(MOE_EINVAL, "unknown weight_layout");
  if (p->weight_layout == MOE_LAYOUT_BLOCKED && p->dtype != MOE_BF16)
    return fail(MOE_EUNSUPPORTED, "the blocked weight layout is bf16 only");
  if (p->top_k < 1) return fail(MOE_EINVAL, "top_k must be >= 1");
  if (p->top_k > moe::kMaxTopK) return fail(MOE_EUNSUPPORTED, "top_k > %d", moe::kMaxTopK);
  const int64_t lim = (int64_t)1 << 30;
  if (p->num_tokens > lim || p->hidden > lim || p->num_tokens * p->top_k >= lim ||
      p->num_tokens * p->top_k * p->hidden >= ((int64_t)1 << 40))
    return fail(MOE_EUNSUPPORTED, "sizes too large");
  if (p->dtype == MOE_BF16 && p->hidden % 64)
    return fail(MOE_EUNSUPPORTED, "bf16 needs hidden to be a multiple of 64");
  if (uses & kUsesExperts) {
    if (p->num_experts < 1) return fail(MOE_EINVAL, "num_experts must be >= 1");
    if (p->top_k > p->num_experts)
      return fail(MOE_EINVAL, "top_k=%lld outside [1, num_experts=%lld]", (long long)p->top_k,
                  (long long)p->num_experts);
    if (p->num_experts > moe::kMaxExperts)
      return fail(MOE_EUNSUPPORTED, "num_experts > %d", moe::kMaxExperts);
    if (p->norm_topk_prob != 0 && p->norm_topk_prob != 1)
      return fail(MOE_EINVAL, "norm_topk_prob must be 0 or 1");
  }
  if (uses & kUsesInter) {
    if (p->inter < 1 || p->inter > lim) return fail(MOE_EINVAL, "inter must be in [1, 2^30]");
    if (p->dtype == MOE_BF16 && p->inter % 64)
      return fail(MOE_EUNSUPPORTED, "bf16 needs inter to be a multiple of 64");
  }
  if (uses & kUsesShared) {
    if (p->shared_inter < 0 || p->shared_inter > lim) return fail(MOE_EINVAL, "shared_inter must be in [0, 2^30]");
    if (p->dtype == MOE_BF16 && p->shared_inter % 64)
      return fail(MOE_EUNSUPPORTED, "bf16 needs shared_inter to be a multiple of 64");
  }
  return MOE_OK;
}

// Row-tile height of the grouped products, from the pairs per expert the
// host can see (avg = N*k / E): the shortest height that holds nearly every
// expert's pairs in one tile, since a second tile re-reads the expert's
// weights, while taller tiles only add padding rows; 16-row tiles only
// while experts average under 2 pairs, where their doubled column blocks
// (twice the workgroups) still pay.  The boundaries are measured (H=2048,
// E=128, top-8, I=768, blocked weights; route + align + products +
// combine): 136 tokens (avg 8.5) 16-row tiles 211.9 us, 32-row 199.5; at
// E=512, 80 tokens (avg 1.25) 527.2 / 529.0 and 144 tokens (avg 2.25)
// 645.6 / 643.2 (16 / 32); 256 tokens (avg 16) 205.8 / 209.1 and 264 (avg
// 16.5) 230.4 / 209.6 (32 / 64: past 16 pairs a few experts need a second
// 32-row tile, and the launch a fourth round of workgroups); 640 (avg 40)
// 232.1 / 239.3 and 704 (avg 44) 260.8 / 242.3 (64 / 128); 1900 (avg 119)
// 299.0 / 319.5 and 2048 (avg 128) 335.9 / 321.8 (128 / 320).
int64_t choose_block_m(const moe_problem* p) {
  if (p->dtype == MOE_F32) return 16;
  const double avg = (double)(p->num_tokens * p->top_k) / (double)p->num_experts;
  if (avg < 2) return 16;
  if (avg <= 16) return 32;
  if (avg < 42) return 64;
  if (avg < 124) return 128;
  return 320;                       // one tile holds a typical prefill expert
}

// Row-tile height of the dense products (shared expert, dense layers) for
// `inter` gate and up columns: the tallest tile (fewest bytes per flop)
// whose gate/up launch still keeps at least half of the GPU's 256 CUs busy,
// ceil(N / h) row tiles times the column blocks (128 gate and 128 up columns
// per workgroup from 64 rows up, 64 and 64 below) >= 128 workgroups.
// Measured on the dense SwiGLU layer (H=2048, I=6144, blocked weights):
// 64 tokens 32-row tiles 55.1 us against 68.1 with 16 rows; 128 tokens
// 32 rows 68.2 against 93.4 with 64; 1024 tokens 320 rows 126.9 against
// 138.8 with 128; 3072 tokens 320 rows 207.5 against 274.7 with 128.  The
// talker's shared expert (8192 rows, I_s = 2048) keeps 320-row tiles (416
// workgroups; 128-row tiles took 218 against 199 us there).
// A dense layer (dense_layer set) takes 256-row tiles instead of 320-row
// ones when that is fewer rows per CU over the launch: rounds of 256
// workgroups (one per CU) times the tile height, ties to 320.  The same
// layer, whole: 768 / 1024 / 2048 / 2560 / 4096 tokens 98.2 / 97.8 / 179.0
// / 199.0 / 277.7 us with 256 rows against 103.1 / 105.9 / 193.7 / 209.0 /
// 285.4 with 320 (the same rounds of shorter tiles); where 256 rows add a
// round they lose: 1536 / 3072 tokens 172.6 / 250.1 against 135.3 / 221.9.
// The shared expert keeps 320 rows, the routed products' height, so the two
// still share their launches.
int64_t dense_block_m(const moe_problem* p, int64_t inter, bool dense_layer = false) {
  if (p->dtype == MOE_F32) return 16;
  const int64_t N = p->num_tokens;
  auto blocks = [&](int64_t h) {
    const int64_t cols = (h >= 64) ? 128 : 64;        // gate (and as many up) columns per workgroup
    return ((N + h - 1) / h) * ((inter + cols - 1) / cols);
  };
  for (int64_t h : {320, 128, 64, 32}) {
    if (blocks(h) < 128) continue;
    if (h == 320 && dense_layer && (blocks(256) + 255) / 256 * 256 < (blocks(320) + 255) / 256 * 320) return 256;
    return h;
  }
  return 16;
}

// Row-tile height of a dense down product: the tallest height up to the
// gate/up one whose launch still has 160 workgroups, ceil(N / h) row tiles
// times 256-column blocks of H; else 32 rows while the launch of 32x128
// tiles fits one round (512 workgroups, two per CU; the launcher narrows
// them to 64 columns while that fits a round too); else 64 rows.  The down
// product's K (the intermediate size) is long for dense layers, so a launch
// with few workgroups keeps most CUs idle throughout, and a launch a little
// past one round pays for a whole second one.  Measured on the dense SwiGLU
// layer (H=2048, I=6144, blocked weights), whole layer: 256 tokens 32-row
// down tiles 72.8 us against 99.3 with 64; 512 tokens 32 rows 76.6 against
// 101.9 with 64; 1024 tokens 32x128 tiles 105.2 against 127.6 with 64 rows
// and 140.3 with 32x64 (1024 workgroups, three per CU); 1152 tokens 64 rows
// 126.8 against 137.9 with 32x128 (576 workgroups); 2048 tokens 64 rows
// 189.0 against 201.0 with 128; 2560 tokens 128 rows 204.7 against 252.0
// with 64; 4096 tokens 128 rows 278.3 against 321.4 with 64.  16-row tiles
// were never faster than 32-row ones there, so they are left to 16-row
// gate/up tiles.  Every tile height sums each element in one K order, so
// the result does not change.
int64_t dense_down_block_m(const moe_problem* p, int64_t bm) {
  if (p->dtype == MOE_F32) return bm;
  const int64_t N = p->num_tokens, H = p->hidden;
  auto blocks = [&](int64_t h, int64_t cols) { return ((N + h - 1) / h) * ((H + cols - 1) / cols); };
  for (int64_t h : {320, 128, 64})
    if (h <= bm && blocks(h, 256) >= 160) return h;
  if (bm < 32) return bm;
  if (bm == 32 || blocks(32, 128) <= 512) return 32;
  return 64;
}

bool block_m_supported(int32_t dtype, int64_t bm) {
  if (dtype == MOE_F32) return bm >= 1 && bm <= 1024;
  return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 320;
}

void capacity(int64_t pairs, int64_t experts, int64_t bm, int64_t* rows, int64_t* tiles) {
  const int64_t t = (pairs + std::min(experts, pairs) * (bm - 1)) / bm;
  *tiles = t;
  *rows = t * bm;
}

// moe_forward's small-batch schedule: the grouped products scan the top-k
// ids themselves instead of reading an align table (16-row tiles, and the
// ids must fit the tile's A ring).
bool ids_supported(const moe_problem* p) {
  const int64_t P = p->num_tokens * p->top_k;
  return p->dtype == MOE_BF16 && P >= 4 && P <= moe::kScanMaxPairs && P % 4 == 0;
}

// The ids products run one workgroup per (expert, column block) whatever the
// routing, and every one of them loads its first weight stages before it
// knows whether its expert has pairs.  So they pay only when most experts
// are hit: measured with H=2048, E=128, top-8, blocked weights (moe_forward
// against the grouped stages), 1 token 64 against 58 us, 16 tokens 152
// against 138 us, 24 tokens 167 against 175 us, 64 tokens 193 against
// 204 us, 128 tokens 214 against 218 us.  Taken from N*k >= 1.5 E, while
// experts average under 9 pairs.
bool scan_mode(const moe_problem* p) {
  const int64_t P = p->num_tokens * p->top_k;
  return ids_supported(p) && 2 * P >= 3 * p->num_experts && P < 9 * p->num_experts;
}

void layout_of(const moe_problem* p, moe_workspace_layout* L) {
  memset(L, 0, sizeof(*L));
  const int64_t N = p->num_tokens, P = N * p->top_k, E = p->num_experts;
  const size_t es = elt_size(p->dtype);
  L->ids_products = scan_mode(p) ? 1 : 0;
  L->block_m = L->ids_products ? 16 : choose_block_m(p);   // the ids products run 16-row passes
  capacity(P, E, L->block_m, &L->max_rows, &L->max_tiles);
  L->shared_block_m = p->shared_inter > 0 ? dense_block_m(p, p->shared_inter) : 0;
  // Products whose launch also runs the shared expert's tiles (bit 0 gate/up,
  // bit 1 down): both for grouped tiles of the same height; for the ids
  // products (16-row tiles) those where the shared tiles fit the last round.
  L->shared_merged = 0;
  if (p->shared_inter > 0 && p->dtype == MOE_BF16 && L->shared_block_m == L->block_m)
    L->shared_merged = L->ids_products ? moe::scan_shared_merge(P, p->num_experts, N, p->hidden, p->inter,
                                                                p->shared_inter)
                                       : 3;
  size_t off = 0;
  auto region = [&](size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    const size_t r = off;
    off += bytes;
    return r;
  };
  L->route_scratch = region(moe::route_scratch_floats(N, E, true) * 4);
  L->topk_ids = region(P * 4);
  L->topk_w = region(P * 4);
  L->shared_scale = region(p->shared_inter ? N * 4 : 0);
  L->counts = region(E * 4);
  L->offsets = region((E + 1) * 4);
  L->order = region(P * 4);
  L->sorted_pairs = region(L->max_rows * 4);
  L->tile_expert = region(L->max_tiles * 4);
  L->tile_rows = region(L->max_tiles * 4);
  L->num_tiles = region(4);
  L->align_scratch = region(moe::align_scratch_ints(P, E) * 4);
  L->act = region(L->max_rows * p->inter * es);
  L->y = region(P * p->hidden * es);
  L->shared_act = region(N * p->shared_inter * es);
  L->shared_y = region(p->shared_inter ? N * p->hidden * es : 0);
  L->total_bytes = (off + 255) & ~(size_t)255;
}

moe::GemmProblem gemm_common(const moe_problem* p) {
  moe::GemmProblem g;
  memset(&g, 0, sizeof(g));
  g.top_k = (int32_t)p->top_k;
  g.num_pairs = (int32_t)(p->num_tokens * p->top_k);
  g.dtype = p->dtype;
  g.weights_blocked = p->weight_layout == MOE_LAYOUT_BLOCKED;
  return g;
}

// Gate/up or down in scan mode (arguments checked by the caller).
moe::GemmProblem ids_problem(const moe_problem* p, const int32_t* topk_ids) {
  moe::GemmProblem g = gemm_common(p);
  g.topk_ids = topk_ids;
  g.num_experts = (int32_t)p->num_experts;
  g.block_m = 16;
  g.max_tiles = (int32_t)p->num_experts;
  return g;
}

moe::GemmProblem ids_gate_up_problem(const moe_problem* p, const void* x, const void* w_gate_up,
                                     const int32_t* topk_ids, void* act) {
  moe::GemmProblem g = ids_problem(p, topk_ids);
  g.a = x;
  g.b = w_gate_up;
  g.c = act;
  g.expert_stride = 2 * p->inter * p->hidden;
  g.K = (int32_t)p->hidden;
  g.n_out = (int32_t)p->inter;
  return g;
}

moe::GemmProblem ids_down_problem(const moe_problem* p, const void* act, const void* w_down,
                                  const int32_t* topk_ids, const float* topk_w, void* y) {
  moe::GemmProblem g = ids_problem(p, topk_ids);
  g.a = act;
  g.b = w_down;
  g.c = y;
  g.scale = topk_w;
  g.expert_stride = p->hidden * p->inter;
  g.K = (int32_t)p->inter;
  g.n_out = (int32_t)p->hidden;
  return g;
}

int check_ptrs_bf16(const moe_problem* p, std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (q && p->dtype == MOE_BF16 && !aligned16(q))
      return fail(MOE_EUNSUPPORTED, "bf16 tensors must be 16-byte aligned");
  return MOE_OK;
}

// The two products of a dense SwiGLU over all rows of x:
//   gate/up: act = silu(x Wg^T) * (x Wu^T);  down: c = scale[n] * (act Wd^T)
// (scale NULL: 1).  With fill_down the down product takes its own tile
// height (dense_down_block_m); a down launch shared with the routed experts
// keeps the gate/up height.
void dense_problems(const moe_problem* p, int64_t inter, const void* x, const void* w_gate_up, const void* w_down,
                    const float* scale, void* act, void* c, moe::GemmProblem* gu, moe::GemmProblem* dn,
                    bool fill_down = true, bool dense_layer = false) {
  const int64_t N = p->num_tokens;
  const int64_t bm = dense_block_m(p, inter, dense_layer);
  moe::GemmProblem g = gemm_common(p);
  g.dense_rows = (int32_t)N;
  g.block_m = (int32_t)bm;
  g.max_tiles = (int32_t)((N + bm - 1) / bm);
  g.a = x;
  g.b = w_gate_up;
  g.c = act;
  g.K = (int32_t)p->hidden;
  g.n_out = (int32_t)inter;
  *gu = g;
  g.a = act;
  g.b = w_down;
  g.c = c;
  g.scale = scale;
  g.K = (int32_t)inter;
  g.n_out = (int32_t)p->hidden;
  if (fill_down) {
    const int64_t dbm = dense_down_block_m(p, bm);
    g.block_m = (int32_t)dbm;
    g.max_tiles = (int32_t)((N + dbm - 1) / dbm);
  }
  *dn = g;
}

int dense_swiglu(const moe_problem* p, int64_t inter, const void* x, const void* w_gate_up,
                 const void* w_down, const float* scale, void* act, void* c, hipStream_t stream,
                 const char* what_gate_up, const char* what_down, bool dense_layer = false) {
  moe::GemmProblem gu, dn;
  dense_problems(p, inter, x, w_gate_up, w_down, scale, act, c, &gu, &dn, true, dense_layer);
  if (int rc = hip_status(moe::launch_gate_up(gu, stream), what_gate_up)) return rc;
  return hip_status(moe::launch_down(dn, stream), what_down);
}

// The grouped products over an align table.
moe::GemmProblem grouped_gate_up_problem(const moe_problem* p, const void* x, const void* w_gate_up,
                                         const int32_t* sorted_pairs, const int32_t* tile_expert,
                                         const int32_t* tile_rows, const int32_t* num_tiles, int64_t block_m,
                                         int64_t max_tiles, void* act) {
  moe::GemmProblem g = gemm_common(p);
  g.a = x;
  g.b = w_gate_up;
  g.sorted_pairs = sorted_pairs;
  g.tile_expert = tile_expert;
  g.tile_rows = tile_rows;
  g.num_tiles = num_tiles;
  g.c = act;
  g.expert_stride = 2 * p->inter * p->hidden;
  g.K = (int32_t)p->hidden;
  g.n_out = (int32_t)p->inter;
  g.block_m = (int32_t)block_m;
  g.max_tiles = (int32_t)max_tiles;
  return g;
}

moe::GemmProblem grouped_down_problem(const moe_problem* p, const void* act, const void* w_down, const float* topk_w,
                                      const int32_t* sorted_pairs, const int32_t* tile_expert,
                                      const int32_t* tile_rows, const int32_t* num_tiles, int64_t block_m,
                                      int64_t max_tiles, void* y) {
  moe::GemmProblem g = gemm_common(p);
  g.a = act;
  g.b = w_down;
  g.sorted_pairs = sorted_pairs;
  g.tile_expert = tile_expert;
  g.tile_rows = tile_rows;
  g.num_tiles = num_tiles;
  g.scale = topk_w;
  g.c = y;
  g.expert_stride = p->hidden * p->inter;
  g.K = (int32_t)p->inter;
  g.n_out = (int32_t)p->hidden;
  g.block_m = (int32_t)block_m;
  g.max_tiles = (int32_t)max_tiles;
  return g;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_mfma_probe(const void* operands, int64_t num_operands, int64_t iters, float* sink, double* flops,
                   void* stream) {
  if (!operands || !sink || !flops) return fail(MOE_EINVAL, "null pointer");
  if (num_operands < 512 || num_operands % 512 != 0)
    return fail(MOE_EINVAL, "num_operands must be a positive multiple of 512, got %lld", (long long)num_operands);
  if (iters < 1 || iters > (1 << 20)) return fail(MOE_EINVAL, "iters must be in [1, 1048576], got %lld", (long long)iters);
  if (!aligned16(operands)) return fail(MOE_EINVAL, "operands must be 16-byte aligned");
  *flops = moe::mfma_probe_flops(iters);
  return hip_status(moe::launch_mfma_probe(operands, num_operands, iters, sink, (hipStream_t)stream), "mfma probe");
}

int moe_align_capacity(int64_t num_pairs, int64_t num_experts, int64_t block_m, int64_t* max_rows,
                       int64_t* max_tiles) {
  if (!max_rows || !max_tiles) return fail(MOE_EINVAL, "output pointer is NULL");
  if (num_pairs < 0 || num_experts < 1 || block_m < 1)
    return fail(MOE_EINVAL, "need num_pairs >= 0, num_experts >= 1, block_m >= 1");
  capacity(num_pairs, num_experts, block_m, max_rows, max_tiles);
  return ok();
}

int moe_pack_weights(int64_t batch, int64_t rows, int64_t cols, int32_t dtype, const void* src, void* dst,
                     void* stream) {
  if (dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "the blocked weight layout is bf16 only");
  if (batch < 0 || rows < 0 || cols < 0) return fail(MOE_EINVAL, "negative size");
  if (rows % 8 || cols % 64) return fail(MOE_EUNSUPPORTED, "blocked weights need rows %% 8 == 0 and cols %% 64 == 0");
  if (batch > 0 && rows > 0 && cols > 0 && batch * rows >= ((int64_t)1 << 40) / cols)
    return fail(MOE_EUNSUPPORTED, "sizes too large");
  const int64_t n = batch * rows * cols;
  if (n == 0) return ok();
  if (!src || !dst) return fail(MOE_EINVAL, "NULL tensor");
  if (!aligned16(src) || !aligned16(dst)) return fail(MOE_EUNSUPPORTED, "tensors must be 16-byte aligned");
  const char *s0 = static_cast<const char*>(src), *d0 = static_cast<const char*>(dst);
  if (s0 < d0 + n * 2 && d0 < s0 + n * 2) return fail(MOE_EINVAL, "src and dst overlap");
  return hip_status(moe::launch_pack_weights(src, dst, batch, rows, cols, (hipStream_t)stream), "pack_weights")
             ?: ok();
}

int moe_get_workspace_layout(const moe_problem* p, moe_workspace_layout* layout) {
  if (int rc = check_problem(p)) return rc;
  if (!layout) return fail(MOE_EINVAL, "layout is NULL");
  layout_of(p, layout);
  return ok();
}

int moe_workspace_size(const moe_problem* p, size_t* bytes) {
  if (int rc = check_problem(p)) return rc;
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  moe_workspace_layout L;
  layout_of(p, &L);
  *bytes = L.total_bytes;
  return ok();
}

int moe_route_scratch_size(const moe_problem* p, size_t* bytes) {
  if (int rc = check_problem(p, kUsesExperts)) return rc;
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = (size_t)moe::route_scratch_floats(p->num_tokens, p->num_experts, true) * 4;
  return ok();
}

int moe_route(const moe_problem* p, const void* x, const void* router_w, const void* shared_gate,
              int32_t* topk_ids, float* topk_w, float* shared_scale, float* scratch, void* stream) {
  if (int rc = check_problem(p, kUsesExperts)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!x || !router_w || !topk_ids || !topk_w || !scratch) return fail(MOE_EINVAL, "NULL tensor");
  if (shared_gate && !shared_scale) return fail(MOE_EINVAL, "shared_gate given without shared_scale");
  if (int rc = check_ptrs_bf16(p, {x, router_w, shared_gate, scratch})) return rc;   // partials: 16-byte stores
  if (int rc = hip_status(moe::launch_route(*p, x, router_w, shared_gate, topk_ids, topk_w,
                                            shared_scale, scratch, (hipStream_t)stream), "route"))
    return rc;
  return ok();
}

int moe_align_scratch_size(int64_t num_pairs, int64_t num_experts, size_t* bytes) {
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  if (num_pairs < 0 || num_experts < 1) return fail(MOE_EINVAL, "need num_pairs >= 0, num_experts >= 1");
  *bytes = (size_t)moe::align_scratch_ints(num_pairs, num_experts) * 4;
  return ok();
}

int moe_align(const int32_t* topk_ids, int64_t num_tokens, int64_t top_k, int64_t num_experts,
              int64_t block_m, int32_t* counts, int32_t* offsets, int32_t* order,
              int32_t* sorted_pairs, int32_t* tile_expert, int32_t* tile_rows, int32_t* num_tiles,
              int32_t* scratch, void* stream) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1) return fail(MOE_EINVAL, "bad sizes");
  if (num_experts > moe::kMaxExperts) return fail(MOE_EUNSUPPORTED, "num_experts > %d", moe::kMaxExperts);
  if (block_m < 1 || block_m > 1024) return fail(MOE_EINVAL, "block_m outside [1, 1024]");
  if (num_tokens * top_k >= ((int64_t)1 << 30)) return fail(MOE_EUNSUPPORTED, "too many pairs");
  if (!counts || !offsets || !num_tiles) return fail(MOE_EINVAL, "NULL output");
  if (num_tokens > 0 && (!topk_ids || !order || !sorted_pairs || !tile_expert || !tile_rows))
    return fail(MOE_EINVAL, "NULL tensor");
  if (moe::align_scratch_ints(num_tokens * top_k, num_experts) > 0 && !scratch)
    return fail(MOE_EINVAL, "this many pairs needs the align scratch array");
  if (int rc = hip_status(moe::launch_align(topk_ids, num_tokens * top_k, num_experts, block_m, counts,
                                            offsets, order, sorted_pairs, tile_expert, tile_rows,
                                            num_tiles, scratch, (hipStream_t)stream), "align"))
    return rc;
  return ok();
}

int moe_gate_up(const moe_problem* p, const void* x, const void* w_gate_up, const int32_t* sorted_pairs,
                const int32_t* tile_expert, const int32_t* tile_rows, const int32_t* num_tiles,
                int64_t block_m, int64_t max_tiles, void* act, void* stream) {
  if (int rc = check_problem(p, kUsesExperts | kUsesInter)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!x || !w_gate_up || !sorted_pairs || !tile_expert || !tile_rows || !num_tiles || !act)
    return fail(MOE_EINVAL, "NULL tensor");
  if (!block_m_supported(p->dtype, block_m)) return fail(MOE_EUNSUPPORTED, "block_m %lld", (long long)block_m);
  if (max_tiles < 0 || max_tiles >= ((int64_t)1 << 24)) return fail(MOE_EINVAL, "bad max_tiles");
  if (int rc = check_ptrs_bf16(p, {x, w_gate_up, act})) return rc;
  const moe::GemmProblem g = grouped_gate_up_problem(p, x, w_gate_up, sorted_pairs, tile_expert, tile_rows,
                                                     num_tiles, block_m, max_tiles, act);
  return hip_status(moe::launch_gate_up(g, (hipStream_t)stream), "gate_up") ?: ok();
}

int moe_down(const moe_problem* p, const void* act, const void* w_down, const float* topk_w,
             const int32_t* sorted_pairs, const int32_t* tile_expert, const int32_t* tile_rows,
             const int32_t* num_tiles, int64_t block_m, int64_t max_tiles, void* y, void* stream) {
  if (int rc = check_problem(p, kUsesExperts | kUsesInter)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!act || !w_down || !topk_w || !sorted_pairs || !tile_expert || !tile_rows || !num_tiles || !y)
    return fail(MOE_EINVAL, "NULL tensor");
  if (!block_m_supported(p->dtype, block_m)) return fail(MOE_EUNSUPPORTED, "block_m %lld", (long long)block_m);
  if (max_tiles < 0 || max_tiles >= ((int64_t)1 << 24)) return fail(MOE_EINVAL, "bad max_tiles");
  if (int rc = check_ptrs_bf16(p, {act, w_down, y})) return rc;
  const moe::GemmProblem g = grouped_down_problem(p, act, w_down, topk_w, sorted_pairs, tile_expert, tile_rows,
                                                  num_tiles, block_m, max_tiles, y);
  return hip_status(moe::launch_down(g, (hipStream_t)stream), "down") ?: ok();
}

int moe_gate_up_ids(const moe_problem* p, const void* x, const void* w_gate_up, const int32_t* topk_ids,
                    void* act, void* stream) {
  if (int rc = check_problem(p, kUsesExperts | kUsesInter)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!x || !w_gate_up || !topk_ids || !act) return fail(MOE_EINVAL, "NULL tensor");
  if (!ids_supported(p))
    return fail(MOE_EUNSUPPORTED, "needs bf16 and 4 <= N*k <= %d with N*k a multiple of 4", moe::kScanMaxPairs);
  if (!aligned16(topk_ids)) return fail(MOE_EUNSUPPORTED, "topk_ids must be 16-byte aligned");
  if (int rc = check_ptrs_bf16(p, {x, w_gate_up, act})) return rc;
  return hip_status(moe::launch_gate_up(ids_gate_up_problem(p, x, w_gate_up, topk_ids, act), (hipStream_t)stream),
                    "gate_up_ids") ?: ok();
}

int moe_down_ids(const moe_problem* p, const void* act, const void* w_down, const int32_t* topk_ids,
                 const float* topk_w, void* y, void* stream) {
  if (int rc = check_problem(p, kUsesExperts | kUsesInter)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!act || !w_down || !topk_ids || !topk_w || !y) return fail(MOE_EINVAL, "NULL tensor");
  if (!ids_supported(p))
    return fail(MOE_EUNSUPPORTED, "needs bf16 and 4 <= N*k <= %d with N*k a multiple of 4", moe::kScanMaxPairs);
  if (!aligned16(topk_ids)) return fail(MOE_EUNSUPPORTED, "topk_ids must be 16-byte aligned");
  if (int rc = check_ptrs_bf16(p, {act, w_down, y})) return rc;
  return hip_status(moe::launch_down(ids_down_problem(p, act, w_down, topk_ids, topk_w, y), (hipStream_t)stream),
                    "down_ids") ?: ok();
}

int moe_shared_expert(const moe_problem* p, const void* x, const void* shared_w_gate_up,
                      const void* shared_w_down, const float* shared_scale, void* shared_act,
                      void* shared_y, void* stream) {
  if (int rc = check_problem(p, kUsesShared)) return rc;
  if (p->shared_inter < 1) return fail(MOE_EINVAL, "shared_inter must be >= 1 for the shared expert");
  if (p->num_tokens == 0) return ok();
  if (!x || !shared_w_gate_up || !shared_w_down || !shared_scale || !shared_act || !shared_y)
    return fail(MOE_EINVAL, "NULL tensor");
  if (int rc = check_ptrs_bf16(p, {x, shared_w_gate_up, shared_w_down, shared_act, shared_y})) return rc;
  return dense_swiglu(p, p->shared_inter, x, shared_w_gate_up, shared_w_down, shared_scale, shared_act,
                      shared_y, (hipStream_t)stream, "shared gate_up", "shared down") ?: ok();
}

int moe_dense_mlp(const moe_problem* p, const void* x, const void* w_gate_up, const void* w_down, void* act,
                  void* out, void* stream) {
  if (int rc = check_problem(p, kUsesInter)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!x || !w_gate_up || !w_down || !act || !out) return fail(MOE_EINVAL, "NULL tensor");
  if (int rc = check_ptrs_bf16(p, {x, w_gate_up, w_down, act, out})) return rc;
  return dense_swiglu(p, p->inter, x, w_gate_up, w_down, nullptr, act, out, (hipStream_t)stream,
                      "dense gate_up", "dense down", true) ?: ok();
}

int moe_add_rmsnorm(int64_t num_tokens, int64_t hidden, int32_t dtype, const void* x, const void* residual_in,
                    void* residual_out, const void* weight, float eps, void* normed, void* stream) {
  if (num_tokens < 0 || hidden < 1) return fail(MOE_EINVAL, "need num_tokens >= 0 and hidden >= 1");
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "unknown dtype");
  if (hidden % 8 || hidden > moe::add_rmsnorm_max_hidden())
    return fail(MOE_EUNSUPPORTED, "hidden must be a multiple of 8 and at most %lld",
                (long long)moe::add_rmsnorm_max_hidden());
  if (num_tokens >= ((int64_t)1 << 31) || num_tokens * hidden >= ((int64_t)1 << 40))
    return fail(MOE_EUNSUPPORTED, "sizes too large");
  if (!(eps > 0.0f) || !(eps < 1e30f)) return fail(MOE_EINVAL, "eps must be positive and finite");
  if (num_tokens == 0) return ok();
  if (!x || !residual_out || !weight || !normed) return fail(MOE_EINVAL, "NULL tensor");
  if (normed == residual_out) return fail(MOE_EINVAL, "normed and residual_out must be different buffers");
  for (const void* q : {x, residual_in, (const void*)residual_out, weight, (const void*)normed})
    if (q && !aligned16(q)) return fail(MOE_EUNSUPPORTED, "tensors must be 16-byte aligned");
  return hip_status(moe::launch_add_rmsnorm(x, residual_in, residual_out, weight, normed, num_tokens, hidden, eps,
                                            dtype, (hipStream_t)stream), "add_rmsnorm") ?: ok();
}

int moe_combine(const moe_problem* p, const void* y, const void* shared_y, void* out, void* stream) {
  if (int rc = check_problem(p, 0)) return rc;
  if (p->num_tokens == 0) return ok();
  if (!y || !out) return fail(MOE_EINVAL, "NULL tensor");
  if (int rc = check_ptrs_bf16(p, {y, shared_y, out})) return rc;
  return hip_status(moe::launch_combine(y, shared_y, out, p->num_tokens, p->hidden, p->top_k,
                                        p->dtype, (hipStream_t)stream), "combine") ?: ok();
}

}  // extern "C"

namespace {

// Argument checks of the whole block, shared by moe_forward and
// moe_forward_noalloc (everything but the workspace).  Returns MOE_OK, or an
// error code with the message set; *empty is set when there is nothing to do.
int check_forward(const moe_problem* p, const void* x, const void* router_w, const void* w_gate_up,
                  const void* w_down, const void* shared_w_gate_up, const void* shared_w_down,
                  const void* shared_gate, const void* out, bool* empty) {
  *empty = false;
  if (int rc = check_problem(p)) return rc;
  const bool shared = shared_w_gate_up != nullptr;
  if (shared != (p->shared_inter > 0))
    return fail(MOE_EINVAL, "shared_w_gate_up must be given exactly when shared_inter > 0");
  if (shared && (!shared_w_down || !shared_gate)) return fail(MOE_EINVAL, "shared expert needs all three tensors");
  if (p->num_tokens == 0) {
    *empty = true;
    return MOE_OK;
  }
  if (!x || !router_w || !w_gate_up || !w_down || !out) return fail(MOE_EINVAL, "NULL tensor");
  return check_ptrs_bf16(p, {x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out});
}

// The launch sequence of the whole block over a workspace laid out as L.
int run_forward(const moe_problem* p, const moe_workspace_layout& L, const void* x, const void* router_w,
                const void* w_gate_up, const void* w_down, const void* shared_w_gate_up,
                const void* shared_w_down, const void* shared_gate, void* out, char* ws, void* stream) {
  const bool shared = shared_w_gate_up != nullptr;
  // Products whose launch also runs the shared expert's tiles (bit 0
  // gate/up, bit 1 down; see the layout).
  const int merge = shared ? (int)L.shared_merged : 0;
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  int32_t* ids = (int32_t*)at(L.topk_ids);
  float* w = (float*)at(L.topk_w);
  float* sscale = shared ? (float*)at(L.shared_scale) : nullptr;
  if (int rc = moe_route(p, x, router_w, shared ? shared_gate : nullptr, ids, w, sscale,
                         (float*)at(L.route_scratch), stream))
    return rc;
  if (L.ids_products) {
    // Small batch: the products find their expert's pairs themselves (no
    // align launch); act and y rows are pair indices.
    const moe::GemmProblem gu = ids_gate_up_problem(p, x, w_gate_up, ids, at(L.act));
    const moe::GemmProblem dn = ids_down_problem(p, at(L.act), w_down, ids, w, at(L.y));
    if (merge) {
      // The shared expert's 16-row tiles first, so that its long workgroups
      // (the down product's K is I_s) start in the first round; a product
      // that does not merge runs them in a launch of their own after it.
      moe::GemmProblem sgu, sdn;
      dense_problems(p, p->shared_inter, x, shared_w_gate_up, shared_w_down, sscale, at(L.shared_act),
                     at(L.shared_y), &sgu, &sdn, /*fill_down=*/(merge & 2) == 0);
      if (merge & 1) {
        if (int rc = hip_status(moe::launch_gate_up_pair(sgu, gu, (hipStream_t)stream), "gate_up_ids with shared"))
          return rc;
      } else {
        if (int rc = hip_status(moe::launch_gate_up(gu, (hipStream_t)stream), "gate_up_ids")) return rc;
        if (int rc = hip_status(moe::launch_gate_up(sgu, (hipStream_t)stream), "shared gate_up")) return rc;
      }
      if (merge & 2) {
        if (int rc = hip_status(moe::launch_down_pair(sdn, dn, (hipStream_t)stream), "down_ids with shared"))
          return rc;
      } else {
        if (int rc = hip_status(moe::launch_down(dn, (hipStream_t)stream), "down_ids")) return rc;
        if (int rc = hip_status(moe::launch_down(sdn, (hipStream_t)stream), "shared down")) return rc;
      }
    } else {
      if (int rc = hip_status(moe::launch_gate_up(gu, (hipStream_t)stream), "gate_up_ids")) return rc;
      if (int rc = hip_status(moe::launch_down(dn, (hipStream_t)stream), "down_ids")) return rc;
    }
  } else {
    int32_t* sorted = (int32_t*)at(L.sorted_pairs);
    int32_t* texp = (int32_t*)at(L.tile_expert);
    int32_t* trows = (int32_t*)at(L.tile_rows);
    int32_t* ntiles = (int32_t*)at(L.num_tiles);
    if (int rc = moe_align(ids, p->num_tokens, p->top_k, p->num_experts, L.block_m, (int32_t*)at(L.counts),
                           (int32_t*)at(L.offsets), (int32_t*)at(L.order), sorted, texp, trows, ntiles,
                           (int32_t*)at(L.align_scratch), stream))
      return rc;
    if (merge) {
      // One gate/up and one down launch cover the routed tiles and the shared
      // expert's dense tiles (same tile height): one ramp-up and one tail per
      // product instead of two, and the small shared launches no longer run
      // a partial round of workgroups on their own.
      moe::GemmProblem sgu, sdn;
      dense_problems(p, p->shared_inter, x, shared_w_gate_up, shared_w_down, sscale, at(L.shared_act),
                     at(L.shared_y), &sgu, &sdn, /*fill_down=*/false);
      const moe::GemmProblem gu = grouped_gate_up_problem(p, x, w_gate_up, sorted, texp, trows, ntiles, L.block_m,
                                                          L.max_tiles, at(L.act));
      // Gate/up: the shared expert's tiles first.  They are all full and of
      // one length, so the routed tiles (partial ones among them) make up
      // the launch's last round; talker layer 899 -> 895 us in interleaved
      // runs.  The same order for down brought nothing.
      if (int rc = hip_status(moe::launch_gate_up_pair(sgu, gu, (hipStream_t)stream), "gate_up with shared"))
        return rc;
      const moe::GemmProblem dn = grouped_down_problem(p, at(L.act), w_down, w, sorted, texp, trows, ntiles,
                                                       L.block_m, L.max_tiles, at(L.y));
      if (int rc = hip_status(moe::launch_down_pair(dn, sdn, (hipStream_t)stream), "down with shared")) return rc;
    } else {
      if (int rc = moe_gate_up(p, x, w_gate_up, sorted, texp, trows, ntiles, L.block_m, L.max_tiles,
                               at(L.act), stream))
        return rc;
      if (int rc = moe_down(p, at(L.act), w_down, w, sorted, texp, trows, ntiles, L.block_m, L.max_tiles,
                            at(L.y), stream))
        return rc;
    }
  }
  if (shared && !merge) {
    if (int rc = moe_shared_expert(p, x, shared_w_gate_up, shared_w_down, sscale, at(L.shared_act),
                                   at(L.shared_y), stream))
      return rc;
  }
  if (int rc = moe_combine(p, at(L.y), shared ? at(L.shared_y) : nullptr, out, stream)) return rc;
  return ok();
}

// ------------------------------------------------- allocation-free variant
// The workspace of moe_forward_noalloc: one fixed array in device memory,
// one copy per GPU the library runs on, held until the process ends.  In
// host code `noalloc_scratch` names a host-side stand-in, not the device
// copy: its device address comes from hipGetSymbolAddress, once per device,
// and only that address is ever passed to a kernel.  Every call on one GPU
// shares the array (the last call's contents stay in it); nothing in it has
// to start at zero, because each call writes every region before reading
// it.  Calls that overlap on one GPU (two streams, two host threads) race.
static __device__ __align__(256) unsigned char noalloc_scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// Device address of noalloc_scratch on the current device.
int noalloc_scratch_ptr(char** ptr) {
  int dev = -1;
  if (int rc = hip_status(hipGetDevice(&dev), "hipGetDevice")) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EUNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* addr = nullptr;
    if (int rc = hip_status(hipGetSymbolAddress(&addr, HIP_SYMBOL(noalloc_scratch)),
                            "hipGetSymbolAddress(noalloc_scratch)"))
      return rc;
    if (!addr || (reinterpret_cast<uintptr_t>(addr) & 255u))
      return fail(MOE_EHIP, "noalloc scratch has no usable device address");
    g_noalloc_ptr[dev] = addr;
  }
  *ptr = static_cast<char*>(g_noalloc_ptr[dev]);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const moe_problem* p, const void* x, const void* router_w, const void* w_gate_up,
                const void* w_down, const void* shared_w_gate_up, const void* shared_w_down,
                const void* shared_gate, void* out, void* workspace, size_t workspace_bytes,
                void* stream) {
  bool empty = false;
  if (int rc = check_forward(p, x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out,
                             &empty))
    return rc;
  if (empty) return ok();
  if (!workspace) return fail(MOE_EINVAL, "NULL tensor");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_EUNSUPPORTED, "workspace must be 256-byte aligned");
  moe_workspace_layout L;
  layout_of(p, &L);
  if (workspace_bytes < L.total_bytes)
    return fail(MOE_ENOSPC, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total_bytes);
  return run_forward(p, L, x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out,
                     static_cast<char*>(workspace), stream);
}

int moe_forward_noalloc(const moe_problem* p, const void* x, const void* router_w, const void* w_gate_up,
                        const void* w_down, const void* shared_w_gate_up, const void* shared_w_down,
                        const void* shared_gate, void* out, void* stream) {
  bool empty = false;
  if (int rc = check_forward(p, x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out,
                             &empty))
    return rc;
  if (empty) return ok();
  moe_workspace_layout L;
  layout_of(p, &L);
  if (L.total_bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ENOSPC,
                "moe_forward_noalloc: this problem needs %zu bytes of scratch, more than its fixed %zu "
                "(use moe_forward with a caller workspace)",
                L.total_bytes, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  char* ws = nullptr;
  if (int rc = noalloc_scratch_ptr(&ws)) return rc;
  return run_forward(p, L, x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out, ws,
                     stream);
}

}  // extern "C"
