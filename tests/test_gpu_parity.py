"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer results (expert ids, counts, stable order, padded layout) must match
bit for bit; tokens whose top-k margin in the oracle is below 1e-6 are left
out of the id and output comparisons (and their number is printed).  Outputs:
|gpu - ref| <= 2e-2 * max|ref| + 1e-3 in bf16, <= 1e-4 * max|ref| in fp32.
"""
import json
import os

import numpy as np
import pytest
import torch

import sparse_moe_ffn_amd as moe
from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MARGIN = 1e-6
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def host(t):
    return None if t is None else t.float().cpu().numpy()


def shared_of(h):
    if h.get("shared_w_gate_up") is None:
        return None
    return {"w_gate_up": h["shared_w_gate_up"], "w_down": h["shared_w_down"], "gate": h["shared_gate"]}


def to_host(t):
    return {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in t.items()}


def run_forward(t, cfg):
    return moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                           t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])


def compare_routing(h, cfg, ids_gpu, w_gpu):
    ids_ref, w_ref, probs, margin = O.route(h["x"], h["router_w"], cfg.top_k, cfg.norm_topk_prob)
    keep = margin >= MARGIN
    ids_gpu = ids_gpu.cpu().numpy()
    w_gpu = w_gpu.cpu().numpy()
    bad = np.nonzero((ids_gpu[keep] != ids_ref[keep]).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} routed tokens differ, first {np.nonzero(keep)[0][bad[:5]]}"
    np.testing.assert_allclose(w_gpu[keep], w_ref[keep], rtol=2e-5, atol=2e-6)
    return (ids_ref, w_ref, probs, margin), keep


def full_reference(h, hw, sh, cfg, routing, sample):
    """The oracle's output for every token, in the grouped formulation (one
    float64 product per expert over its gathered tokens, then index-add),
    after checking it against the per-token definition on `sample` rows."""
    ref, _, _ = O.moe_forward_grouped(h["x"], h["router_w"], hw["w_gate_up"], hw["w_down"], cfg.top_k,
                                      cfg.norm_topk_prob, shared=sh, routing=routing)
    defn, _ = O.moe_forward(h["x"], h["router_w"], hw["w_gate_up"], hw["w_down"], cfg.top_k, cfg.norm_topk_prob,
                            shared=sh, rows=sample, routing=routing)
    scale = max(1.0, float(np.abs(defn).max()))
    assert np.abs(ref[sample] - defn).max() <= 1e-12 * scale, "grouped oracle differs from the definition"
    return ref


def check_output(out_rows, ref_rows, dtype, what=""):
    tol = O.tolerance(ref_rows, dtype)
    err = float(np.abs(out_rows - ref_rows).max()) if ref_rows.size else 0.0
    assert np.isfinite(out_rows).all(), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max|gpu-ref| = {err:.4e} > tol {tol:.4e}"
    return err, tol


# --------------------------------------------------------------- the pages' examples

def test_route_example_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "m03_route_example.json")))
    x = torch.tensor(g["x"], dtype=torch.float32, device=DEV)
    eye = torch.eye(g["E"], g["H"], dtype=torch.float32, device=DEV)
    for renorm, key in ((True, "weights_renorm"), (False, "weights_no_renorm")):
        ids, w, _ = moe.moe_route(x, eye, g["top_k"], renorm)
        assert ids.cpu().tolist() == g["ids"]
        assert np.round(w.cpu().double().numpy(), 4).tolist() == g[key]


def scalar_block(g, device):
    E = g["E"]
    gu = torch.tensor([[[g["w_gate"][e]], [g["w_up"][e]]] for e in range(E)], dtype=torch.float32, device=device)
    wd = torch.tensor([[[g["w_down"][e]]] for e in range(E)], dtype=torch.float32, device=device)
    r = torch.tensor(g["router_w"], dtype=torch.float32, device=device)
    x = torch.tensor(g["x"], dtype=torch.float32, device=device)
    return x, r, gu, wd


def test_scalar_block_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "m03_scalar_block.json")))
    x, r, gu, wd = scalar_block(g, DEV)
    ids, w, _ = moe.moe_route(x, r, g["top_k"], True)
    assert ids.cpu().tolist() == g["ids"]
    assert np.round(w.cpu().double().numpy(), 4).tolist() == g["weights"]
    out = moe.moe_forward(x, r, gu, wd, g["top_k"], True)
    assert np.round(out.cpu().double().numpy(), 4).tolist() == g["out"]
    s = g["shared"]
    sgu = torch.tensor(s["gate_proj"] + s["up_proj"], dtype=torch.float32, device=DEV)
    sdn = torch.tensor(s["down_proj"], dtype=torch.float32, device=DEV)
    sg = torch.tensor(s["gate"], dtype=torch.float32, device=DEV).reshape(-1)
    out = moe.moe_forward(x, r, gu, wd, g["top_k"], True, sgu, sdn, sg)
    assert np.round(out.cpu().double().numpy(), 4).tolist() == s["out_with_shared"]


def test_align_walkthrough_on_gpu():
    g = json.load(open(os.path.join(GOLDEN, "m03_grouping_walkthrough.json")))
    ids = torch.tensor(g["ids"], dtype=torch.int32, device=DEV)
    gr = moe.moe_align(ids, g["E"], 2)
    assert gr.counts.cpu().tolist() == g["counts"]
    assert gr.order.cpu().tolist() == g["order"]
    assert gr.offsets.cpu().tolist() == [0, 1, 2, 5, 6, 6]
    nt = int(gr.num_tiles.item())
    S = g["N"] * g["k"]
    assert nt == 5
    assert gr.sorted_pairs[:nt * 2].cpu().tolist() == [1, S, 2, S, 0, 3, 4, S, 5, S]
    assert gr.tile_expert[:nt].cpu().tolist() == [0, 1, 2, 2, 3]
    assert gr.tile_rows[:nt].cpu().tolist() == [1, 1, 2, 1, 1]


# --------------------------------------------------------------- align, random ids

@pytest.mark.parametrize("N,k,E,bm,dist", [
    (3, 2, 5, 16, "uniform"), (64, 8, 128, 16, "uniform"), (4096, 8, 128, 128, "uniform"),
    (16384, 8, 128, 128, "zipf"), (1000, 4, 7, 32, "one"), (333, 1, 1, 64, "uniform"),
    (1, 8, 8, 16, "uniform"), (5000, 6, 512, 16, "zipf"), (777, 3, 60, 1, "uniform"),
    (513, 8, 64, 16, "uniform"), (2048, 2, 3, 320, "one"), (9000, 4, 128, 320, "zipf"),
    # more than 16 chunks of 4096 pairs: the chunk counts are summed by thread groups
    (12000, 8, 512, 64, "zipf"), (20000, 4, 7, 32, "one"), (70000, 1, 1, 16, "uniform")])
def test_align_matches_oracle(N, k, E, bm, dist):
    rng = np.random.default_rng(N * 31 + E)
    if dist == "uniform":
        ids = np.stack([rng.permutation(E)[:k] for _ in range(N)]) if N * k < 200000 else None
    elif dist == "zipf":
        wts = 1.0 / np.arange(1, E + 1) ** 1.2
        ids = np.stack([rng.choice(E, size=k, replace=False, p=wts / wts.sum()) for _ in range(N)])
    else:                       # every token also picks expert 0
        ids = np.stack([np.concatenate([[0], 1 + rng.permutation(E - 1)[:k - 1]]) for _ in range(N)])
    gr = moe.moe_align(torch.tensor(ids, dtype=torch.int32, device=DEV), E, bm)
    flat_e, _, _ = O.flatten_pairs(ids, np.zeros(ids.shape, np.float32))
    order, counts, offsets = O.group_pairs(flat_e, E)
    sp, te, tr, nt = O.pad_segments(order, counts, bm, N * k)
    assert np.array_equal(gr.counts.cpu().numpy(), counts)
    assert np.array_equal(gr.offsets.cpu().numpy(), offsets)
    assert np.array_equal(gr.order.cpu().numpy(), order)
    assert int(gr.num_tiles.item()) == nt
    assert np.array_equal(gr.sorted_pairs[:nt * bm].cpu().numpy(), sp)
    assert np.array_equal(gr.tile_expert[:nt].cpu().numpy(), te)
    assert np.array_equal(gr.tile_rows[:nt].cpu().numpy(), tr)


# --------------------------------------------------------------- whole block, small shapes

SMALL = [
    random_case(37, 64, 10, 3, 64, dtype="bf16", seed=1),
    random_case(1, 128, 16, 4, 128, dtype="bf16", seed=2),
    random_case(200, 128, 16, 4, 192, I_shared=128, dtype="bf16", seed=3),
    random_case(50, 64, 6, 6, 64, dtype="bf16", seed=4),                       # k = E
    random_case(70, 192, 9, 1, 64, dtype="bf16", seed=5, norm_topk_prob=False),  # k = 1
    random_case(40, 64, 1, 1, 128, dtype="bf16", seed=6),                      # E = 1: a dense SwiGLU
    random_case(300, 256, 32, 8, 128, dtype="bf16", seed=7, norm_topk_prob=False),
    random_case(1500, 128, 8, 2, 64, dtype="bf16", seed=8),                    # block_m 320 path
    random_case(700, 128, 8, 2, 64, dtype="bf16", seed=15),                    # block_m 128 path
    random_case(600, 128, 16, 2, 64, dtype="bf16", seed=9),                    # block_m 64 path
    random_case(300, 128, 16, 2, 64, dtype="bf16", seed=10),                   # block_m 32 path
    random_case(2000, 320, 8, 2, 192, dtype="bf16", seed=13),                  # partial column tiles
    random_case(1500, 256, 8, 2, 256, dtype="bf16", seed=16),                  # 320 rows, A in registers
    random_case(2000, 320, 8, 2, 256, dtype="bf16", seed=17),                  # same, partial down columns
    random_case(1200, 1024, 4, 1, 512, dtype="bf16", seed=18, norm_topk_prob=False),  # same, longer K
    random_case(700, 192, 600 // 2, 8, 64, I_shared=192, dtype="bf16", seed=14),  # E = 300: two route passes
    random_case(4100, 128, 8, 2, 64, I_shared=192, dtype="bf16", seed=19),   # shared expert on 320-row tiles
    random_case(48, 128, 512, 32, 64, dtype="bf16", seed=20),                  # the limits: E = 512, k = 32
    random_case(9, 128, 32, 32, 64, dtype="bf16", seed=21, norm_topk_prob=False),  # k = E = 32
    random_case(13, 33, 5, 2, 17, I_shared=9, dtype="f32", seed=11),
    random_case(64, 40, 12, 3, 24, dtype="f32", seed=12, norm_topk_prob=False),
]


@pytest.mark.parametrize("cfg", [CONFIGS["tiny"]] + SMALL, ids=lambda c: c.name)
def test_forward_small(cfg):
    t = make_inputs(cfg, DEV)
    out = run_forward(t, cfg)
    ids_gpu, w_gpu, s_gpu = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob, t["shared_gate"])
    torch.cuda.synchronize()
    h = to_host(t)
    routing, keep = compare_routing(h, cfg, ids_gpu, w_gpu)
    if s_gpu is not None:
        ref_s = O.sigmoid(h["x"].astype(np.float64) @ h["shared_gate"].astype(np.float64))
        np.testing.assert_allclose(s_gpu.cpu().numpy(), ref_s, rtol=1e-5, atol=1e-6)
    ref, _ = O.moe_forward(h["x"], h["router_w"], h["w_gate_up"], h["w_down"], cfg.top_k, cfg.norm_topk_prob,
                           shared=shared_of(h), routing=routing)
    err, tol = check_output(host(out)[keep], ref[keep], cfg.dtype, cfg.name)
    print(f"{cfg.name}: err {err:.3e} tol {tol:.3e} excluded {int((~keep).sum())}")


def test_empty_batch():
    """N = 0 is a no-op for every entry point: each returns empty outputs
    of the right shape without an error."""
    cfg = random_case(4, 64, 4, 2, 64, I_shared=64, dtype="bf16")
    t = make_inputs(cfg, DEV)
    x0 = t["x"][:0]
    out = moe.moe_forward(x0, t["router_w"], t["w_gate_up"], t["w_down"], 2, True)
    assert out.shape == (0, 64)
    out = moe.moe_forward(x0, t["router_w"], t["w_gate_up"], t["w_down"], 2, True, t["shared_w_gate_up"],
                          t["shared_w_down"], t["shared_gate"])
    assert out.shape == (0, 64)
    out = moe.moe_forward_noalloc(x0, t["router_w"], t["w_gate_up"], t["w_down"], 2, True)
    assert out.shape == (0, 64)
    ids, w, sc = moe.moe_route(x0, t["router_w"], 2, True, t["shared_gate"])
    assert ids.shape == (0, 2) and w.shape == (0, 2) and sc.shape == (0,)
    gr = moe.moe_align(ids, cfg.E, 16)
    assert int(gr.counts.sum()) == 0
    act = moe.moe_gate_up(x0, t["w_gate_up"], gr, 2)
    y = moe.moe_down(act, t["w_down"], w, gr, 0, 2)
    assert moe.moe_combine(y, 0, 2).shape == (0, 64)
    sa, sy = moe.moe_shared_expert(x0, t["shared_w_gate_up"], t["shared_w_down"], sc)
    assert sy.shape == (0, 64)
    assert moe.moe_dense_mlp(x0, t["shared_w_gate_up"], t["shared_w_down"]).shape == (0, 64)
    normed, res = moe.moe_add_rmsnorm(x0, torch.empty_like(x0), t["shared_gate"])
    assert normed.shape == (0, 64) and res.shape == (0, 64)
    torch.cuda.synchronize()


# --------------------------------------------------------------- full-size workloads

_full_cache = {}


def full_inputs(name):
    if name not in _full_cache:
        _full_cache.clear()
        torch.cuda.empty_cache()
        cfg = CONFIGS[name]
        _full_cache[name] = (cfg, make_inputs(cfg, DEV))
    return _full_cache[name]


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode", "prefill", "skew", "talker"])
def test_full_size_parity(name):
    cfg, t = full_inputs(name)
    out = run_forward(t, cfg)
    out2 = run_forward(t, cfg)
    ids_gpu, w_gpu, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob, None)
    lay = moe.moe_get_workspace_layout(moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], cfg.top_k,
                                                        cfg.norm_topk_prob, t["shared_w_gate_up"]))
    gr = moe.moe_align(ids_gpu, cfg.E, lay["block_m"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "two runs differ"
    h = {"x": host(t["x"]), "router_w": host(t["router_w"])}
    routing, keep = compare_routing(h, cfg, ids_gpu, w_gpu)
    ids_ref = routing[0]
    # grouping: exact, with the excluded tokens' pairs removed on both sides
    k = cfg.top_k
    excluded = np.nonzero(~keep)[0]
    ids_g = ids_gpu.cpu().numpy()
    counts_g = gr.counts.cpu().numpy().astype(np.int64)
    flat_ref, _, _ = O.flatten_pairs(ids_ref, routing[1])
    order_r, counts_r, _ = O.group_pairs(flat_ref, cfg.E)
    for n in excluded:
        for j in range(k):
            counts_g[ids_g[n, j]] -= 1
            counts_r[ids_ref[n, j]] -= 1
    assert np.array_equal(counts_g, counts_r)
    drop = np.zeros(cfg.N * k, bool)
    for n in excluded:
        drop[n * k:(n + 1) * k] = True
    order_g = gr.order.cpu().numpy()
    assert np.array_equal(order_g[~drop[order_g]], order_r[~drop[order_r]])
    # outputs: every token the margin rule keeps, element by element
    rng = np.random.default_rng(5)
    sample = sorted(set([0, cfg.N - 1] + rng.choice(cfg.N, size=min(cfg.N, 6), replace=False).tolist()))
    hw = {"w_gate_up": host(t["w_gate_up"]), "w_down": host(t["w_down"])}
    h["x"] = host(t["x"])
    sh = None
    if cfg.I_shared:
        sh = {"w_gate_up": host(t["shared_w_gate_up"]), "w_down": host(t["shared_w_down"]),
              "gate": host(t["shared_gate"])}
    ref = full_reference(h, hw, sh, cfg, routing, sample)
    err, tol = check_output(host(out)[keep], ref[keep], cfg.dtype, name)
    print(f"{name}: all {int(keep.sum())} kept rows compared")
    nz = int((counts_r == 0).sum())
    print(f"{name}: err {err:.3e} tol {tol:.3e} excluded tokens {excluded.size} "
          f"counts min/max {counts_r.min()}/{counts_r.max()} empty experts {nz}")
    if cfg.skew:
        assert nz >= cfg.skew_dead


@pytest.mark.slow
@pytest.mark.parametrize("N", [64, 1024, 4096])
def test_larger_layer_shape(N):
    """A larger layer of the same family (H=4096, E=128, top-8, I=1536:
    twice the reduction length of both products and of the router).  64
    tokens take the ids products, 1024 and 4096 the grouped tiles.  Routing
    and outputs are compared on every token."""
    cfg = random_case(N, 4096, 128, 8, 1536, dtype="bf16", seed=31)
    t = make_inputs(cfg, DEV)
    out = run_forward(t, cfg)
    ids_gpu, w_gpu, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    torch.cuda.synchronize()
    h = {"x": host(t["x"]), "router_w": host(t["router_w"])}
    (ids_ref, w_ref, probs, margin), keep = compare_routing(h, cfg, ids_gpu, w_gpu)
    hw = {"w_gate_up": host(t["w_gate_up"]), "w_down": host(t["w_down"])}
    del t["w_gate_up"], t["w_down"]
    ref = full_reference(h, hw, None, cfg, (ids_ref, w_ref, probs, margin), [0, N // 2, N - 1])
    err, tol = check_output(host(out)[keep], ref[keep], cfg.dtype, cfg.name)
    print(f"{cfg.name}: err {err:.3e} tol {tol:.3e} all {int(keep.sum())} kept rows, "
          f"excluded {int((~keep).sum())}")


@pytest.mark.slow
def test_offsets_past_32_bits():
    """A batch of 2^18 + 37 tokens of the 30B-A3B layer shape (H=2048,
    E=128, top-8, I=768): the (token, slot) rows of y then hold more than
    2^32 elements, and tokens from 2^18 on have all their down outputs and
    combine inputs past element 2^32, so any 32-bit offset in the down
    epilogue, the combine or the grouping would show in their rows.  Their
    ids, weights and outputs, and those of a few tokens before, are
    compared with the oracle's per-token definition."""
    N = (1 << 18) + 37
    cfg = random_case(N, 2048, 128, 8, 768, dtype="bf16", seed=41)
    assert N * cfg.top_k * cfg.H > 1 << 32
    t = make_inputs(cfg, DEV)
    out = run_forward(t, cfg)
    ids_gpu, w_gpu, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    torch.cuda.synchronize()
    sample = [0, 1, N // 2, (1 << 18) - 1] + list(range(1 << 18, N))
    idx = torch.tensor(sample, device=DEV)
    xs = host(t["x"][idx])
    rw = host(t["router_w"])
    routing = O.route(xs, rw, cfg.top_k, cfg.norm_topk_prob)
    ids_ref, w_ref, _, margin = routing
    keep = margin >= MARGIN
    ids_s = ids_gpu[idx].cpu().numpy()
    w_s = w_gpu[idx].cpu().numpy()
    assert (ids_s[keep] == ids_ref[keep]).all(), "routed ids differ"
    np.testing.assert_allclose(w_s[keep], w_ref[keep], rtol=2e-5, atol=2e-6)
    ref, _ = O.moe_forward(xs, rw, host(t["w_gate_up"]), host(t["w_down"]), cfg.top_k, cfg.norm_topk_prob,
                           routing=routing)
    err, tol = check_output(host(out[idx])[keep], ref[keep], cfg.dtype, cfg.name)
    print(f"{cfg.name}: {int(keep.sum())} of {len(sample)} sampled tokens compared, err {err:.3e} tol {tol:.3e}")


@pytest.mark.slow
def test_batch_invariance_decode_layer():
    cfg, t = full_inputs("decode")
    full = run_forward(t, cfg)
    for i in (0, 17, 63):
        one = moe.moe_forward(t["x"][i:i + 1].contiguous(), t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k,
                              cfg.norm_topk_prob)
        assert torch.equal(one[0], full[i]), f"token {i}"


@pytest.mark.slow
@pytest.mark.parametrize("name,sizes", [("prefill", [1, 64, 200, 600, 1024, 2048]),
                                        ("talker", [1, 24, 100, 200, 600, 1000, 2000, 4096])])
def test_batch_invariance_across_tile_heights(name, sizes):
    """A token's output is the same bit for bit in any batch.  The first n
    tokens of the layer run, by batch size, 16-row grouped tiles (1 token),
    the ids products (24 to 100), 32-row tiles (200), 64-row tiles (600),
    128-row tiles (1000, 1024) and 320-row tiles (2000 and up, the whole
    batch included).  The talker's shared expert takes its own dense tile
    height: 16 rows up to 24 tokens, then 32, 32, 64, 128, 128 and 320 rows,
    in one launch with the routed tiles where the heights agree (1, 200,
    600, 1000, 4096 and the whole batch) and in launches of its own where
    they do not.  Routing sums fixed H slices and every product sums each
    output element in one K order whatever its tile, so the rows must agree
    exactly."""
    cfg, t = full_inputs(name)
    full = run_forward(t, cfg)
    for n in sizes:
        sub = moe.moe_forward(t["x"][:n].contiguous(), t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k,
                              cfg.norm_topk_prob, t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])
        torch.cuda.synchronize()
        assert torch.equal(sub, full[:n]), f"{name}: the first {n} tokens differ from the whole batch"


@pytest.mark.slow
def test_staged_calls_equal_forward():
    cfg, t = full_inputs("decode")
    out = run_forward(t, cfg)
    lay = moe.moe_get_workspace_layout(moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], cfg.top_k,
                                                        cfg.norm_topk_prob))
    ids, w, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    gr = moe.moe_align(ids, cfg.E, lay["block_m"])
    act = moe.moe_gate_up(t["x"], t["w_gate_up"], gr, cfg.top_k)
    y = moe.moe_down(act, t["w_down"], w, gr, cfg.N, cfg.top_k)
    out2 = moe.moe_combine(y, cfg.N, cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("N,H,E,k,Is", [(1100, 256, 128, 8, 64), (1200, 128, 64, 4, 0), (1031, 192, 160, 6, 32),
                                        (2048, 2048, 128, 8, 0), (2100, 256, 128, 8, 64),
                                        (4099, 128, 160, 6, 32), (3000, 192, 512, 32, 0),
                                        (8200, 128, 128, 8, 64), (16400, 64, 128, 8, 64),
                                        (1500, 256, 100, 12, 64)])
def test_router_tilings_bitwise_equal(N, H, E, k, Is):
    """Batches of 1024 tokens and more compute their logits in 64-token
    tiles (x fragments shared through LDS) placed by XCD, smaller ones in
    one-wave workgroups of 16 tokens and three 16-column sub-tiles;
    a token's ids, weights and shared gate must be bit for bit the same
    whichever batch routed it (also at the layer's own H = 2048, at H = 64
    where most slices are empty, at E = 512, and with k > 8, the
    radix-select path)."""
    cfg = random_case(N, H, E, k, 64, I_shared=Is, dtype="bf16", seed=3)
    t = make_inputs(cfg, DEV)
    gate = t["shared_gate"]
    ids, w, sc = moe.moe_route(t["x"], t["router_w"], k, True, gate)
    windows = [(0, 64), (N - 37, N), (511, 512)]
    if N >= 2048:
        windows += [(N - 1100, N - 3), (1500, 1600)]               # 64-token tiles; 16-token tiles
    if N >= 8192:
        windows += [(N - 2100, N - 1), (5, 8200)]                  # other tile and XCD alignments
    for lo, hi in windows:
        ids_s, w_s, sc_s = moe.moe_route(t["x"][lo:hi].contiguous(), t["router_w"], k, True, gate)
        torch.cuda.synchronize()
        assert torch.equal(ids[lo:hi], ids_s), f"ids differ in [{lo}, {hi})"
        assert torch.equal(w[lo:hi], w_s), f"weights differ in [{lo}, {hi})"
        if Is:
            assert torch.equal(sc[lo:hi], sc_s), f"shared gate differs in [{lo}, {hi})"
    h = {"x": host(t["x"]), "router_w": host(t["router_w"])}
    compare_routing(h, cfg, ids, w)


@pytest.mark.parametrize("N,H,E,k,I,Is", [(700, 256, 64, 8, 128, 0), (2100, 128, 16, 4, 64, 64)])
def test_forward_multichunk_grouping_equals_staged(N, H, E, k, I, Is):
    """Groupings of several 4096-pair chunks (count, scan and scatter
    launches): moe_forward must equal the staged public calls bit for bit."""
    cfg = random_case(N, H, E, k, I, I_shared=Is, dtype="bf16", seed=13)
    t = make_inputs(cfg, DEV)
    out = run_forward(t, cfg)
    lay = moe.moe_get_workspace_layout(moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], k,
                                                        cfg.norm_topk_prob, t["shared_w_gate_up"]))
    assert lay["ids_products"] == 0 and N * k > 4096
    ids, w, sc = moe.moe_route(t["x"], t["router_w"], k, cfg.norm_topk_prob, t["shared_gate"])
    gr = moe.moe_align(ids, E, lay["block_m"])
    act = moe.moe_gate_up(t["x"], t["w_gate_up"], gr, k)
    y = moe.moe_down(act, t["w_down"], w, gr, N, k)
    sy = None
    if Is:
        _, sy = moe.moe_shared_expert(t["x"], t["shared_w_gate_up"], t["shared_w_down"], sc)
    ref = moe.moe_combine(y, N, k, sy)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("N,H,E,k,I,Is,height,merged", [
    (4100, 128, 8, 2, 64, 1280, 320, 3),      # routed and shared tiles both 320 rows: one launch per product
    (1000, 128, 80, 8, 64, 2048, 128, 3),
    (600, 128, 128, 8, 64, 1664, 64, 3),
    (200, 128, 128, 8, 64, 1216, 32, 3),
    (20, 128, 128, 8, 64, 128, 16, 3),        # grouped 16-row tiles (too few pairs for the ids products)
    (700, 192, 300, 8, 64, 192, 16, 0),       # routed 64, shared 16: launches of its own
    (24, 2048, 128, 8, 768, 2048, 16, 3),     # ids products, both take the shared tiles
    (80, 2048, 128, 8, 768, 2048, 16, 2),     # ids products, down only
    (53, 960, 92, 8, 64, 128, 16, 1),         # ids products, gate/up only
    (64, 2048, 128, 8, 768, 2048, 16, 0),     # ids products, shared launches of its own
])
def test_forward_with_shared_equals_staged(N, H, E, k, I, Is, height, merged):
    """moe_forward runs the shared expert's products in the routed products'
    launches (bit 0 gate/up, bit 1 down) when both take the same tile height
    and, for the ids products, the shared tiles fit the last round of the
    routed launch; the output must equal the staged public calls, whose
    shared expert runs its own tile heights, bit for bit."""
    cfg = random_case(N, H, E, k, I, I_shared=Is, dtype="bf16", seed=23)
    t = make_inputs(cfg, DEV)
    for layout in (moe.MOE_LAYOUT_ROW_MAJOR, moe.MOE_LAYOUT_BLOCKED):
        tw = dict(t)
        if layout == moe.MOE_LAYOUT_BLOCKED:
            for name in ("w_gate_up", "w_down", "shared_w_gate_up", "shared_w_down"):
                tw[name] = moe.moe_pack_weights(t[name])
        out = moe.moe_forward(tw["x"], tw["router_w"], tw["w_gate_up"], tw["w_down"], k, cfg.norm_topk_prob,
                              tw["shared_w_gate_up"], tw["shared_w_down"], tw["shared_gate"], weight_layout=layout)
        lay = moe.moe_get_workspace_layout(moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], k,
                                                            cfg.norm_topk_prob, t["shared_w_gate_up"]))
        assert (lay["shared_block_m"], lay["shared_merged"]) == (height, merged)
        ids, w, sc = moe.moe_route(t["x"], t["router_w"], k, cfg.norm_topk_prob, t["shared_gate"])
        if lay["ids_products"]:
            act = moe.moe_gate_up_ids(t["x"], tw["w_gate_up"], ids, weight_layout=layout)
            y = moe.moe_down_ids(act, tw["w_down"], ids, w, weight_layout=layout)
        else:
            gr = moe.moe_align(ids, E, lay["block_m"])
            act = moe.moe_gate_up(t["x"], tw["w_gate_up"], gr, k, weight_layout=layout)
            y = moe.moe_down(act, tw["w_down"], w, gr, N, k, weight_layout=layout)
        _, sy = moe.moe_shared_expert(t["x"], tw["shared_w_gate_up"], tw["shared_w_down"], sc, weight_layout=layout)
        ref = moe.moe_combine(y, N, k, sy)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"layout {layout}: moe_forward differs from the staged calls"
