"""Stage-level parity of the two grouped products on the GPU, for every tile
height the library supports.

Each case routes and aligns on the GPU, then checks
  gate/up:  act[r] = silu(x[t] . Wg[e]) * (x[t] . Wu[e]) for every real row r
            (pair p = sorted_pairs[r], token t = p // k, expert e of the tile),
  down:     y[p] = w[p] * (act[r] . Wd[e]) with the GPU's own act as input,
so each product is compared alone, against float64 on the same inputs.
Padding rows are not part of either result.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_amd as moe
from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BLOCK_MS = (16, 32, 64, 128, 320)

CASES = [
    random_case(300, 256, 8, 2, 192, dtype="bf16", seed=21),      # partial gate/up column block
    random_case(700, 320, 16, 4, 256, dtype="bf16", seed=22),     # partial down column block
    random_case(97, 2048, 32, 8, 768, dtype="bf16", seed=23),     # layer shapes, ragged expert loads
    random_case(1, 128, 6, 6, 64, dtype="bf16", seed=24),         # one token, k = E
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("bm", BLOCK_MS)
def test_grouped_products(cfg, bm):
    t = make_inputs(cfg, DEV)
    ids, w, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    gr = moe.moe_align(ids, cfg.E, bm)
    act = moe.moe_gate_up(t["x"], t["w_gate_up"], gr, cfg.top_k)
    y = moe.moe_down(act, t["w_down"], w, gr, cfg.N, cfg.top_k)
    torch.cuda.synchronize()

    P = cfg.N * cfg.top_k
    sorted_pairs = gr.sorted_pairs.cpu().numpy()
    tiles = int(gr.num_tiles.item())
    tile_expert = gr.tile_expert.cpu().numpy()[:tiles]
    rows = np.arange(tiles * bm)
    real = sorted_pairs[rows] < P
    rows = rows[real]
    pairs = sorted_pairs[rows]
    experts = tile_expert[rows // bm]
    assert np.array_equal(experts, ids.cpu().numpy().reshape(-1)[pairs]), "tile expert differs from the route"

    x = _host(t["x"])
    wgu = t["w_gate_up"].float().cpu().numpy()
    wd = t["w_down"].float().cpu().numpy()
    act_h = np.zeros((act.shape[0], cfg.I))                   # padding rows are never written
    act_h[rows] = _host(act.index_select(0, torch.as_tensor(rows, device=act.device)))
    y_h = _host(y)
    w_h = w.cpu().numpy().reshape(-1).astype(np.float64)
    ref_act = np.empty((rows.size, cfg.I))
    ref_y = np.empty((rows.size, cfg.H))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        g = x[pairs[sel] // cfg.top_k] @ wgu[e, :cfg.I].astype(np.float64).T
        u = x[pairs[sel] // cfg.top_k] @ wgu[e, cfg.I:].astype(np.float64).T
        ref_act[sel] = O.silu(g) * u
        ref_y[sel] = w_h[pairs[sel], None] * (act_h[rows[sel]] @ wd[e].astype(np.float64).T)
    got_act = act_h[rows]
    tol = O.tolerance(ref_act, "bf16")
    err = float(np.abs(got_act - ref_act).max())
    assert err <= tol, f"gate/up: max|gpu-ref| = {err:.3e} > {tol:.3e}"
    got_y = y_h[pairs]
    tol = O.tolerance(ref_y, "bf16")
    err = float(np.abs(got_y - ref_y).max())
    assert err <= tol, f"down: max|gpu-ref| = {err:.3e} > {tol:.3e}"
    assert sorted(pairs.tolist()) == list(range(P)), "every pair appears in exactly one real row"
