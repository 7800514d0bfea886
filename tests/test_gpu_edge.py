"""Degenerate inputs on the HIP path: every expert equally likely, and a
token with non-finite inputs.

With a zero router weight every logit is exactly 0, so every expert has
probability exactly 1/E and the top-k is decided by the tie rule alone:
equal probabilities go to the lower expert id, so every token takes experts
0..k-1 in that order, with weight 1/k (renormalised) or the float32 1/E.
All N*k pairs then land on k experts, N rows each: the grouping has k
segments of several tiles and E - k empty experts, and the grouped products
run experts whose weights several row tiles share.  Ids, weights and counts
must be exact; outputs within |gpu - ref| <= 2e-2 * max|ref| + 1e-3 in bf16,
1e-4 * max|ref| in fp32 against the oracle (which breaks ties the same way:
a stable sort of the probabilities).

A token whose input row holds NaN or Inf must leave every other token's
output bit for bit unchanged (its own row is non-finite).
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_amd as moe
from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def host(t):
    return None if t is None else t.float().cpu().numpy()


CASES = [
    random_case(64, 2048, 128, 8, 768, seed=31),                            # the decode layer's shape
    random_case(37, 128, 6, 2, 64, seed=32, norm_topk_prob=False),
    random_case(300, 256, 16, 4, 128, I_shared=64, seed=33),                 # 300-row segments
    random_case(5, 24, 6, 3, 40, dtype="f32", seed=34),
    random_case(9, 64, 7, 7, 64, seed=35),                                   # k = E
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_all_equal_probabilities_take_the_lowest_ids(cfg):
    t = make_inputs(cfg, DEV)
    rw = torch.zeros_like(t["router_w"])
    k, E, N = cfg.top_k, cfg.E, cfg.N
    ids, w, _ = moe.moe_route(t["x"], rw, k, cfg.norm_topk_prob)
    out = moe.moe_forward(t["x"], rw, t["w_gate_up"], t["w_down"], k, cfg.norm_topk_prob,
                          t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])
    lay = moe.moe_get_workspace_layout(moe.problem_from(t["x"], t["w_gate_up"], rw, k, cfg.norm_topk_prob,
                                                        t["shared_w_gate_up"]))
    gr = moe.moe_align(ids, E, lay["block_m"])
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == np.arange(k)[None, :]).all()
    h = {name: host(v) for name, v in t.items()}
    routing = O.route(h["x"], np.zeros_like(h["router_w"]), k, cfg.norm_topk_prob)
    assert (routing[0] == np.arange(k)[None, :]).all()
    assert np.array_equal(w.cpu().numpy(), routing[1])                      # 1/k or 1/E, bit for bit
    expect_counts = np.array([N] * k + [0] * (E - k))
    assert np.array_equal(gr.counts.cpu().numpy(), expect_counts)
    bm = lay["block_m"]
    assert int(gr.num_tiles.item()) == k * ((N + bm - 1) // bm)
    rows = list(range(N))                                                   # every token
    shared = None
    if cfg.I_shared:
        shared = {"w_gate_up": h["shared_w_gate_up"], "w_down": h["shared_w_down"], "gate": h["shared_gate"]}
    ref, _ = O.moe_forward(h["x"], np.zeros_like(h["router_w"]), h["w_gate_up"], h["w_down"], k,
                           cfg.norm_topk_prob, shared=shared, rows=rows, routing=routing)
    got = host(out)[rows]
    tol = O.tolerance(ref, cfg.dtype)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    assert err <= tol, f"max|gpu-ref| = {err:.4e} > tol {tol:.4e}"


# ------------------------------------------------------------- non-finite input

@pytest.mark.parametrize("cfg,bad", [
    (random_case(64, 2048, 128, 8, 768, seed=41), 17),                           # the ids products
    (random_case(700, 256, 16, 4, 128, I_shared=64, seed=42), 333),              # grouped tiles + shared expert
    (random_case(700, 256, 16, 4, 128, seed=43, norm_topk_prob=False), 0),       # no renormalisation
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
@pytest.mark.parametrize("value", [float("nan"), float("inf")])
def test_non_finite_token_is_contained(cfg, bad, value):
    """A token whose input row holds NaN or Inf gets a non-finite output row
    and changes no other token's output: every row of an expert tile is
    computed on its own, in the expert's fixed K order, so the other rows
    must be bit for bit those of the batch without the bad token's values
    (that token routed differently only moves rows between tiles)."""
    t = make_inputs(cfg, DEV)
    args = (t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob, t["shared_w_gate_up"],
            t["shared_w_down"], t["shared_gate"])
    clean = moe.moe_forward(t["x"], *args)
    x = t["x"].clone()
    x[bad, :: 3] = value
    dirty = moe.moe_forward(x, *args)
    torch.cuda.synchronize()
    keep = torch.ones(cfg.N, dtype=torch.bool, device=DEV)
    keep[bad] = False
    assert torch.equal(dirty[keep], clean[keep]), "a non-finite token changed other tokens' outputs"
    assert not torch.isfinite(dirty[bad]).any(), "the non-finite token's output row is finite"
