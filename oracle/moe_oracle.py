"""CPU oracle for the sparse MoE FFN block.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product path never does.  It
shares no code with the GPU library (it imports numpy and the standard library
only, plus torch's float32-to-bfloat16 conversion where a value is rounded
to the activation dtype) and is deliberately plain and slow.

Sources (the pages this follows, by title and section):

* [M03] "M03 · Sparse MoE：路由、按 expert 分组计算、shared expert" --
  sections "题面速览" (routing and block formula, the serving way, shared
  expert), "框架视角 · shape trace", "易错点", "逐步图：按 expert 分组的
  bookkeeping" (worked grouping and scalar examples), "三级提示" L1-L3.
* [NANO] the nano-vLLM Qwen3-30B-A3B notes at lshu.cn/news/442807,
  qwen3_moe.py, class ``Qwen3MoeSparseMoeBlock``
  (router linear, float32 softmax, top-k, renormalisation, cast of the
  routing weights to the input dtype, scaled expert outputs added per token).
* [Q35] "Qwen3.5 推理全流程", section 2.5B "Sparse MoE" (shared expert gated
  by a sigmoid of a per-token scalar) and 2.5A "Dense MLP".
* [STEP19] "Step 19: Real Model — Qwen3ForCausalLM", section "RMSNorm：去掉
  均值中心化" (the RMSNorm formula in front of the MLP).

Precision.  The pages fix the routing precision: probabilities come from a
float32 softmax over all E experts and renormalisation is done in float32
([M03] 题面速览 and L1 "细节").  The oracle therefore takes every routing
decision in float32: logits are the exact products of the (bf16 or fp32)
inputs summed in float64 and rounded once to float32; softmax, top-k and
renormalisation are float32.  Everything after routing (gate/up/down
products, SiLU, the weighted sum, the shared expert and its gate) is float64
on the exactly-upcast inputs, with the float32 routing weights.  The
routing weights are not rounded to the input dtype before use (the pages cast
them to x.dtype; that rounding is below the comparison tolerance and the GPU
keeps float32 as well).

Readings where the pages are silent (also listed in the design notes):

* top-k ties go to the lower expert id; slots within a token are in
  descending weight order;
* the flattened pair index is p = n*k + j (token-major, ``repeat_interleave``);
* SiLU is z * sigmoid(z);
* the shared-expert gate is one scalar per token, sigmoid(x . g), applied to
  the shared SwiGLU output and never renormalised with the routed weights;
* padded layout (the pages only name ``moe_align_block_size``): each
  expert's segment of the stable order is padded with the sentinel N*k up to
  a multiple of the tile height, in expert order, empty experts taking no
  rows; tile t covers padded rows [t*BM, (t+1)*BM).
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# Routing ([M03] 题面速览, routing block; [NANO] Qwen3MoeSparseMoeBlock
# forward): router product, float32 softmax over all experts, top-k of the
# probabilities, optional division by the sum of the k kept probabilities.
# --------------------------------------------------------------------------

def router_logits(x, router_w) -> np.ndarray:
    """logits[n, e] = x[n] . router_w[e], summed in float64, rounded to float32."""
    x64 = np.asarray(x, dtype=F64)
    r64 = np.asarray(router_w, dtype=F64)
    return (x64 @ r64.T).astype(F32)


def softmax_f32(logits) -> np.ndarray:
    """Float32 softmax over all experts (last axis): exp(l - max) / sum, the
    sum taken sequentially in expert order in float32."""
    l = np.asarray(logits, dtype=F32)
    m = l.max(axis=-1, keepdims=True)
    z = np.exp(l - m).astype(F32)
    s = np.add.accumulate(z, axis=-1, dtype=F32)[..., -1:]
    return (z / s).astype(F32)


def topk_desc(values, k: int):
    """The k largest values along the last axis, in descending order; equal
    values keep ascending index order (a stable sort of the negated values)."""
    v = np.asarray(values, dtype=F32)
    ids = np.argsort(-v, axis=-1, kind="stable")[..., :k].astype(np.int64)
    return ids, np.take_along_axis(v, ids, axis=-1)


def topk_margin(probs, k: int):
    """Smallest gap between adjacent values of the descending probabilities at
    ranks 0..k (the k-th/(k+1)-th gap included when k < E); inf when E = 1.
    A token whose margin is tiny can be routed either way by float32 rounding."""
    p = np.asarray(probs, dtype=F64)
    s = -np.sort(-p, axis=-1)
    last = min(k + 1, p.shape[-1])
    if last < 2:
        return np.full(p.shape[:-1], math.inf) if p.ndim > 1 else math.inf
    gaps = np.min(s[..., : last - 1] - s[..., 1:last], axis=-1)
    return gaps if p.ndim > 1 else float(gaps)


def route(x, router_w, top_k: int, norm_topk_prob: bool):
    """Routing of every token.

    Returns (ids [N,k] int64, weights [N,k] float32, probs [N,E] float32,
    margin [N] float64)."""
    logits = router_logits(x, router_w)
    N, E = logits.shape
    if not (1 <= top_k <= E):
        raise ValueError("top_k must be in [1, E]")
    probs = softmax_f32(logits)
    ids, w = topk_desc(probs, top_k)
    if norm_topk_prob:
        s = np.zeros((N, 1), dtype=F32)
        for j in range(top_k):                    # sequential float32 sum in slot order
            s = (s + w[:, j:j + 1]).astype(F32)
        w = (w / s).astype(F32)
    margin = topk_margin(probs, top_k) if N else np.zeros(0)
    return ids, w.astype(F32), probs, np.asarray(margin, dtype=F64).reshape(N)


# --------------------------------------------------------------------------
# Grouping ([M03] 逐步图 steps 1-2, L2 flatten/grouping items): the pair
# arrays are the row-major flattening of ids and weights plus each pair's
# token (every token repeated k times in a row); the order is a stable sort of
# pair indices by expert id, counts a per-expert histogram, and a segment
# starts at the prefix sum of the counts before it.
# --------------------------------------------------------------------------

def flatten_pairs(ids, weights):
    ids = np.asarray(ids)
    N, k = ids.shape
    flat_e = ids.reshape(-1).astype(np.int64)
    flat_w = np.asarray(weights).reshape(-1)
    flat_tok = np.repeat(np.arange(N, dtype=np.int64), k)     # 0,0,1,1,2,2 for k=2
    return flat_e, flat_w, flat_tok


def group_pairs(flat_e, E: int):
    """(order, counts, offsets): order is the stable sort of the pair indices
    by expert id, counts[e] the pairs of expert e, offsets the segment starts."""
    flat_e = np.asarray(flat_e, dtype=np.int64)
    order = np.argsort(flat_e, kind="stable").astype(np.int64)
    counts = np.bincount(flat_e, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return order, counts, offsets


def pad_segments(order, counts, block_m: int, sentinel: int):
    """Padded layout for a grouped GEMM with tile height block_m.

    Returns (sorted_pairs, tile_expert, tile_rows, num_tiles): expert e's
    pairs (in stable order) followed by sentinels up to a multiple of
    block_m, experts in ascending order, empty experts skipped; tile t covers
    padded rows [t*block_m, (t+1)*block_m), belongs to tile_expert[t] and has
    tile_rows[t] real pairs."""
    sorted_pairs, tile_expert, tile_rows = [], [], []
    start = 0
    for e, c in enumerate(np.asarray(counts, dtype=np.int64)):
        c = int(c)
        seg = list(np.asarray(order[start:start + c]))
        start += c
        if c == 0:
            continue
        ntile = -(-c // block_m)
        seg += [sentinel] * (ntile * block_m - c)
        sorted_pairs += seg
        for t in range(ntile):
            tile_expert.append(e)
            tile_rows.append(min(block_m, c - t * block_m))
    return (np.array(sorted_pairs, dtype=np.int64), np.array(tile_expert, dtype=np.int64),
            np.array(tile_rows, dtype=np.int64), len(tile_expert))


# --------------------------------------------------------------------------
# Expert math ([M03] 题面速览 block formula and L1 细节): an expert is a
# SwiGLU, silu of the gate projection times the up projection, then the down
# projection; gate and up weights are [I, H], down is [H, I].  The packed
# gate/up weight keeps the gate rows first and the up rows after them
# ([M08] "M08 · 串起来：tiny thinker 的 KV-cache greedy 解码", L3 answer 1).
# --------------------------------------------------------------------------

def silu(z):
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=F64)))


def swiglu(h, w_gate, w_up, w_down):
    """(silu(h Wg^T) * (h Wu^T)) Wd^T in float64 for h of shape [H] or [n, H]."""
    h = np.asarray(h, dtype=F64)
    g = h @ np.asarray(w_gate, dtype=F64).T
    u = h @ np.asarray(w_up, dtype=F64).T
    return (silu(g) * u) @ np.asarray(w_down, dtype=F64).T


class _ExpertCache:
    """Float64 copies of the expert weights, made on first use."""

    def __init__(self, w_gate_up, w_down):
        self.w_gate_up, self.w_down = w_gate_up, w_down
        self.I = np.asarray(w_gate_up).shape[1] // 2
        self._c = {}

    def __getitem__(self, e):
        if e not in self._c:
            gu = np.asarray(self.w_gate_up[e], dtype=F64)
            self._c[e] = (gu[: self.I], gu[self.I:], np.asarray(self.w_down[e], dtype=F64))
        return self._c[e]


def shared_term(x_row, shared):
    """sigmoid(x . g) * SharedSwiGLU(x) for one token ([M03] 题面速览, shared
    expert of the talker; [Q35] 2.5B formula, second term)."""
    gu = np.asarray(shared["w_gate_up"], dtype=F64)
    Is = gu.shape[0] // 2
    gate = float(sigmoid(np.dot(np.asarray(x_row, dtype=F64), np.asarray(shared["gate"], dtype=F64).reshape(-1))))
    return gate * swiglu(x_row, gu[:Is], gu[Is:], shared["w_down"])


def moe_forward(x, router_w, w_gate_up, w_down, top_k, norm_topk_prob, shared=None,
                rows=None, routing=None):
    """The block by its definition, one token at a time:

        out[n] = sum_j w[n, j] * Expert_{ids[n, j]}(x[n])
                 (+ sigmoid(x[n] . g) * Shared(x[n]) when a shared expert is given)

    ([M03] 题面速览 block formula).  ``rows`` restricts the evaluation to the
    listed tokens (routing still covers every token); ``routing`` may pass a
    precomputed ``route`` result.  Returns (out [len(rows), H] float64,
    (ids, weights, probs, margin))."""
    x = np.asarray(x)
    N, H = x.shape
    if routing is None:
        routing = route(x, router_w, top_k, norm_topk_prob)
    ids, w, _, _ = routing
    rows = range(N) if rows is None else list(rows)
    experts = _ExpertCache(w_gate_up, w_down)
    out = np.zeros((len(rows), H), dtype=F64)
    for r, n in enumerate(rows):
        xn = np.asarray(x[n], dtype=F64)
        acc = np.zeros(H, dtype=F64)
        for j in range(top_k):
            wg, wu, wd = experts[int(ids[n, j])]
            acc += float(w[n, j]) * swiglu(xn, wg, wu, wd)
        if shared is not None:
            acc += shared_term(xn, shared)
        out[r] = acc
    return out, routing


def moe_forward_grouped(x, router_w, w_gate_up, w_down, top_k, norm_topk_prob, shared=None, routing=None):
    """The "serving way" of [M03] 题面速览 and L2: group the pairs by expert,
    run each non-empty expert once over its gathered tokens, scale by the
    routing weights and index-add back to the tokens.  A second formulation,
    used to cross-check ``moe_forward``; ``routing`` may pass a precomputed
    ``route`` result."""
    x = np.asarray(x, dtype=F64)
    N, H = x.shape
    E = np.asarray(router_w).shape[0]
    if routing is None:
        routing = route(x, router_w, top_k, norm_topk_prob)
    ids, w, probs, margin = routing
    flat_e, flat_w, flat_tok = flatten_pairs(ids, w)
    order, counts, offsets = group_pairs(flat_e, E)
    experts = _ExpertCache(w_gate_up, w_down)
    out = np.zeros((N, H), dtype=F64)
    for e in range(E):
        n_e = int(counts[e])
        if n_e == 0:
            continue
        sel = order[offsets[e]:offsets[e] + n_e]
        toks = flat_tok[sel]
        wg, wu, wd = experts[e]
        y = swiglu(x[toks], wg, wu, wd) * flat_w[sel].astype(F64)[:, None]
        np.add.at(out, toks, y)                        # index_add_: repeats accumulate
    if shared is not None:
        gu = np.asarray(shared["w_gate_up"], dtype=F64)
        Is = gu.shape[0] // 2
        gate = sigmoid(x @ np.asarray(shared["gate"], dtype=F64).reshape(-1, 1))   # [N, 1]
        out += gate * swiglu(x, gu[:Is], gu[Is:], shared["w_down"])
    return out, (ids, w, probs, margin), (order, counts, offsets)


def moe_forward_by_slot(x, router_w, w_gate_up, w_down, top_k, norm_topk_prob, shared=None):
    """A third formulation, slot by slot: the block formula's sum over the k
    routed experts of a token ([M03] 题面速览) taken with the slot index
    outermost.  For slot j, the tokens whose j-th choice is expert e form one
    batch through that expert; each token occurs once per slot, so the batch
    rows are distinct and are added to their tokens directly."""
    x = np.asarray(x, dtype=F64)
    N, H = x.shape
    ids, w, _, _ = route(x, router_w, top_k, norm_topk_prob)
    experts = _ExpertCache(w_gate_up, w_down)
    out = np.zeros((N, H), dtype=F64)
    for j in range(top_k):
        col = ids[:, j]
        for e in sorted(set(int(v) for v in col)):
            rows = np.flatnonzero(col == e)
            wg, wu, wd = experts[e]
            out[rows] += w[rows, j].astype(F64)[:, None] * swiglu(x[rows], wg, wu, wd)
    if shared is not None:
        for n in range(N):
            out[n] += shared_term(x[n], shared)
    return out


# --------------------------------------------------------------------------
# Dense SwiGLU layer ("Qwen3.5 推理全流程" 2.5A Dense MLP; [NANO] the
# Qwen3MLP / Qwen3MoeMLP used for the layers listed in mlp_only_layers or
# skipped by decoder_sparse_step): the expert formula applied to every token,
# with no router and no weight -- the E = k = 1 case of the block.
# --------------------------------------------------------------------------

def dense_mlp(x, w_gate_up, w_down):
    """(silu(x Wg^T) * (x Wu^T)) Wd^T for every row of x, float64; w_gate_up
    is [2I, H] with the gate rows first, w_down is [H, I]."""
    gu = np.asarray(w_gate_up, dtype=F64)
    I = gu.shape[0] // 2
    return swiglu(x, gu[:I], gu[I:], w_down)


# --------------------------------------------------------------------------
# Residual add + RMSNorm in front of the block.  [NANO] Qwen3DecoderLayer
# and question 4 of the notes: the layer norm before the MLP is called with
# the residual stream -- the incoming activations are added to it, the sum
# is the new residual, and its normalisation is what the MLP (here the MoE
# block) reads; with no residual yet (first layer) the input itself is the
# residual.  "Step 19: Real Model — Qwen3ForCausalLM", section "RMSNorm：去掉
# 均值中心化": RMSNorm(h) = h / sqrt(mean(h^2) + eps) * weight, no mean
# subtraction and no bias.  [M08] 细节: the residual carries the
# un-normalised sum.
# --------------------------------------------------------------------------

def rms_norm(h, weight, eps: float):
    """h / sqrt(mean(h^2 over the last axis) + eps) * weight, float64."""
    h = np.asarray(h, dtype=F64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * np.asarray(weight, dtype=F64)


def round_to(a, dtype: str) -> np.ndarray:
    """Round float32 values to the activation dtype ("bf16": round to nearest
    even, the rounding of a stored bfloat16 tensor; "f32": unchanged)."""
    a = np.asarray(a, dtype=F32)
    if dtype == "f32":
        return a
    import torch  # dtype conversion only (a library primitive)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).float().numpy()


def add_rmsnorm(x, residual, weight, eps: float, dtype: str):
    """(normed float64, new residual float32 holding dtype values).

    The new residual is x + residual (x alone when residual is None), added
    in float32 and rounded once to the activation dtype -- the value a
    caller stores; normed is the RMSNorm of that stored residual."""
    h = np.asarray(x, dtype=F32)
    if residual is not None:
        h = (h + np.asarray(residual, dtype=F32)).astype(F32)
    r = round_to(h, dtype)
    return rms_norm(r, weight, eps), r


def tolerance(ref: np.ndarray, dtype: str) -> float:
    """Absolute bound on |gpu - ref| for a whole output: 2e-2*max|ref| + 1e-3
    in bf16, 1e-4*max|ref| in fp32."""
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return (1e-4 * m) if dtype == "f32" else (2e-2 * m + 1e-3)
