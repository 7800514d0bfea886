"""The small-batch products moe_gate_up_ids / moe_down_ids find each
expert's pairs from the top-k ids themselves and index act and y by pair.
Every row must equal the grouped products' row for the same pair (tile
height 16) bit for bit: same instructions, same K order.  The grouped
products are checked against the oracle in test_gpu_stages.py, so these
equalities carry that parity over.  Cases: one token, ragged sizes, the
decode layer, 1024 pairs over 512 experts (the largest batch taken), the
blocked weight layout, and an expert list of several 16-row passes (every
token routed to the same experts)."""
import pytest
import torch

import sparse_moe_ffn_amd as moe
from sparse_moe_ffn_amd.inputs import make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


CASES = [
    (random_case(1, 128, 6, 4, 64, seed=41), False),
    (random_case(37, 192, 16, 4, 128, seed=42), False),
    (random_case(64, 2048, 128, 8, 768, seed=43), False),
    (random_case(32, 128, 512, 32, 64, seed=44, norm_topk_prob=False), False),
    (random_case(64, 2048, 128, 8, 768, seed=45), True),                    # all tokens on experts 0..7
    (random_case(100, 256, 16, 8, 192, seed=46), True),                     # 7 passes of 16 rows
]


def pack(w):
    return moe.moe_pack_weights(w)


@pytest.mark.parametrize("cfg,ties", CASES, ids=lambda c: c.name if hasattr(c, "name") else str(c))
@pytest.mark.parametrize("layout", [moe.MOE_LAYOUT_ROW_MAJOR, moe.MOE_LAYOUT_BLOCKED])
def test_ids_products_equal_grouped_rows(cfg, ties, layout):
    t = make_inputs(cfg, DEV)
    rw = torch.zeros_like(t["router_w"]) if ties else t["router_w"]
    wgu, wd = t["w_gate_up"], t["w_down"]
    if layout == moe.MOE_LAYOUT_BLOCKED:
        wgu, wd = pack(wgu), pack(wd)
    ids, w, _ = moe.moe_route(t["x"], rw, cfg.top_k, cfg.norm_topk_prob)
    gr = moe.moe_align(ids, cfg.E, 16)
    act_g = moe.moe_gate_up(t["x"], wgu, gr, cfg.top_k, weight_layout=layout)
    y_g = moe.moe_down(act_g, wd, w, gr, cfg.N, cfg.top_k, weight_layout=layout)
    act_i = moe.moe_gate_up_ids(t["x"], wgu, ids, weight_layout=layout)
    y_i = moe.moe_down_ids(act_i, wd, ids, w, weight_layout=layout)
    torch.cuda.synchronize()
    P = cfg.N * cfg.top_k
    rows = int(gr.num_tiles.item()) * 16                 # rows the grouping wrote (the rest is capacity)
    sorted_pairs = gr.sorted_pairs[:rows].long().cpu()
    real = sorted_pairs < P                              # the others are the padding sentinel P
    assert int(real.sum()) == P and bool((sorted_pairs[~real] == P).all())
    rows_of_pair = torch.full((P,), -1, dtype=torch.long)
    rows_of_pair[sorted_pairs[real]] = torch.nonzero(real).reshape(-1)
    assert bool((rows_of_pair >= 0).all())               # every pair has exactly one row
    rows_of_pair = rows_of_pair.to(DEV)
    assert torch.equal(act_i.view(torch.int16), act_g[rows_of_pair].view(torch.int16))
    assert torch.equal(y_i.view(torch.int16), y_g.view(torch.int16))
    if ties:
        assert int(gr.counts.max().item()) == cfg.N                         # passes of 16 rows per expert


def test_forward_takes_the_ids_products_bitwise():
    """moe_forward on a batch that reaches most experts with under 9 pairs
    each uses the ids products; its output equals the grouped stages' (16-row
    tiles) bit for bit."""
    cfg = random_case(48, 256, 64, 8, 128, I_shared=64, seed=47)
    t = make_inputs(cfg, DEV)
    out = moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                          t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])
    ids, w, sc = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob, t["shared_gate"])
    gr = moe.moe_align(ids, cfg.E, 16)
    act = moe.moe_gate_up(t["x"], t["w_gate_up"], gr, cfg.top_k)
    y = moe.moe_down(act, t["w_down"], w, gr, cfg.N, cfg.top_k)
    _, sy = moe.moe_shared_expert(t["x"], t["shared_w_gate_up"], t["shared_w_down"], sc)
    ref = moe.moe_combine(y, cfg.N, cfg.top_k, sy)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_out_of_range_ids_match_no_expert():
    """Ids outside [0, E) (negative or >= E) match no expert: their pairs'
    rows stay as they were, every other row is the grouped result (moe_align
    drops the same pairs)."""
    cfg = random_case(64, 256, 32, 8, 128, seed=48)
    t = make_inputs(cfg, DEV)
    ids, w, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    bad = ids.clone()
    bad[3, 1] = -7
    bad[10, 0] = cfg.E
    bad[63, 7] = 1 << 30
    P = cfg.N * cfg.top_k
    dropped = torch.zeros(P, dtype=torch.bool)
    for n, j in ((3, 1), (10, 0), (63, 7)):
        dropped[n * cfg.top_k + j] = True
    gr = moe.moe_align(bad, cfg.E, 16)
    act_g = moe.moe_gate_up(t["x"], t["w_gate_up"], gr, cfg.top_k)
    y_g = moe.moe_down(act_g, t["w_down"], w, gr, cfg.N, cfg.top_k)
    act_i = torch.full((P, cfg.I), 7.0, dtype=t["x"].dtype, device=DEV)
    y_i = torch.full((P, cfg.H), 7.0, dtype=t["x"].dtype, device=DEV)
    moe.moe_gate_up_ids(t["x"], t["w_gate_up"], bad, act_i)
    moe.moe_down_ids(act_i, t["w_down"], bad, w, y_i)
    torch.cuda.synchronize()
    assert int(gr.counts.sum().item()) == P - 3
    rows = int(gr.num_tiles.item()) * 16
    sp = gr.sorted_pairs[:rows].long().cpu()
    real = sp < P
    keep = ~dropped
    rows_of_pair = torch.full((P,), -1, dtype=torch.long)
    rows_of_pair[sp[real]] = torch.nonzero(real).reshape(-1)
    assert bool((rows_of_pair[keep] >= 0).all()) and bool((rows_of_pair[dropped] == -1).all())
    kd = keep.to(DEV)
    assert torch.equal(act_i[kd].view(torch.int16), act_g[rows_of_pair[keep].to(DEV)].view(torch.int16))
    assert torch.equal(y_i[kd].view(torch.int16), y_g[kd].view(torch.int16))
    assert bool((act_i[~kd] == 7.0).all()) and bool((y_i[~kd] == 7.0).all())


def test_ids_forward_with_shared_expert_in_a_graph():
    """moe_forward on the ids path (with a shared expert) captured once and
    replayed with new inputs copied in, eager runs in between: every replay
    equals the eager result."""
    cfg = random_case(32, 256, 16, 4, 128, I_shared=64, seed=49)
    inputs = [make_inputs(random_case(32, 256, 16, 4, 128, I_shared=64, seed=s), DEV) for s in (49, 50, 51)]
    t = {k: (v.clone() if v is not None else None) for k, v in inputs[0].items()}
    p = moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], cfg.top_k, cfg.norm_topk_prob, t["shared_w_gate_up"])
    assert moe.moe_get_workspace_layout(p)["ids_products"] == 1
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(t["x"])

    def fwd(o):
        return moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                               t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"], out=o, workspace=ws)
    fwd(out)                                            # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(out)
    torch.cuda.synchronize()
    for rep in range(6):
        for name, v in inputs[rep % 3].items():
            if v is not None:
                t[name].copy_(v)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = fwd(torch.empty_like(out))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {rep}"
    del graph
