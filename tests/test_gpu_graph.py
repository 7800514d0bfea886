"""moe_forward and moe_forward_noalloc captured in a HIP graph on the grouped
paths (align in several chunks, 64- and 320-row tiles, the shared expert in
the same launches as the routed experts) and on the ids products with the
shared expert partly merged: each graph is captured once and
replayed on new inputs, with the program's own eager work and
synchronisations between the replays, and every replay must equal the eager
call bit for bit.  (The decode path, which skips the grouping, is replayed
in tests/test_gpu_dense_norm.py.)"""
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
    # N, H, E, k, I, I_shared, shared expert in the routed launches:
    # N*k > 4096 pairs (several align chunks), 128-row tiles
    (1000, 256, 72, 8, 128, 0, 0),
    # 320-row tiles, shared expert in the routed launches (both products)
    (4200, 256, 16, 2, 128, 1280, 3),
    # one align workgroup, 64-row tiles, shared expert in 16-row launches of its own
    (300, 192, 32, 4, 64, 128, 0),
    # the ids products (no grouping), shared tiles in the routed down launch only
    (80, 2048, 128, 8, 768, 2048, 2),
]


@pytest.mark.parametrize("N,H,E,k,I,Is,merged", CASES)
@pytest.mark.parametrize("noalloc", [False, True])
def test_forward_graph_replays_equal_eager(N, H, E, k, I, Is, merged, noalloc):
    cfg = random_case(N, H, E, k, I, I_shared=Is, dtype="bf16", seed=5)
    t = make_inputs(cfg, DEV)
    xs = [make_inputs(cfg.with_(seed=s), DEV)["x"] for s in (11, 12, 13)]
    blk = moe.MOE_LAYOUT_BLOCKED
    w = {n: (moe.moe_pack_weights(t[n]) if t[n] is not None else None)
         for n in ("w_gate_up", "w_down", "shared_w_gate_up", "shared_w_down")}
    p = moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], k, cfg.norm_topk_prob, t["shared_w_gate_up"], blk)
    assert moe.moe_get_workspace_layout(p)["shared_merged"] == merged
    if noalloc and moe.moe_workspace_size(p) > moe.MOE_NOALLOC_SCRATCH_BYTES:
        pytest.skip("beyond the allocation-free entry point's scratch")
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device=DEV)
    x_in = torch.empty_like(t["x"])
    out = torch.empty_like(t["x"])
    args = (t["router_w"], w["w_gate_up"], w["w_down"], k, cfg.norm_topk_prob, w["shared_w_gate_up"],
            w["shared_w_down"], t["shared_gate"])

    def call(x, o):
        if noalloc:
            return moe.moe_forward_noalloc(x, *args, out=o, weight_layout=blk)
        return moe.moe_forward(x, *args, out=o, workspace=ws, weight_layout=blk)

    x_in.copy_(xs[0])
    call(x_in, out)                                  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(x_in, out)
    torch.cuda.synchronize()
    ref = torch.empty_like(out)
    for rep in range(6):
        x_in.copy_(xs[rep % 3])
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref.zero_()                                  # eager work between the replays
        call(xs[rep % 3], ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {rep}: differs from the eager call"
    del graph
