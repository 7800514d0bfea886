"""One GPU's share under expert parallelism, on one GPU.

With G GPUs and expert e on GPU e mod G, GPU g runs the grouped products
for its E/G experts over the (token, slot) pairs every GPU's router sent
it; the y rows go back to their tokens' GPUs for the slot-order combine.
Here the all-to-all is stood in for by torch indexing (no second GPU): each
shard is the library's own moe_align / moe_gate_up / moe_down over the
received rows (one row per pair, top_k = 1, local expert ids), checked row
by row against the oracle, and the G shards' rows, put back in pair order
and combined with moe_combine, must give the oracle's output of the whole
block."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_amd as moe
from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MARGIN = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def shard(t, ids, w, G, g, k, blocked):
    """The pairs GPU g receives (pair order), its rows of x and its experts."""
    flat_ids, flat_w = ids.reshape(-1), w.reshape(-1)
    sel = torch.nonzero(flat_ids % G == g).squeeze(1)
    x_recv = t["x"][torch.div(sel, k, rounding_mode="floor")].contiguous()
    ids_local = torch.div(flat_ids[sel], G, rounding_mode="floor").to(torch.int32).view(-1, 1).contiguous()
    w_recv = flat_w[sel].contiguous()
    wgu = t["w_gate_up"][g::G].contiguous()
    wd = t["w_down"][g::G].contiguous()
    if blocked:
        wgu, wd = moe.moe_pack_weights(wgu), moe.moe_pack_weights(wd)
    return sel, x_recv, ids_local, w_recv, wgu, wd


def run_shard(x_recv, ids_local, w_recv, wgu, wd, E_local, blocked):
    P, H = x_recv.shape
    I = wd.shape[2]
    lay = moe.moe_get_workspace_layout(moe.problem(P, H, E_local, 1, I))
    gr = moe.moe_align(ids_local, E_local, lay["block_m"])
    layout = moe.MOE_LAYOUT_BLOCKED if blocked else moe.MOE_LAYOUT_ROW_MAJOR
    act = moe.moe_gate_up(x_recv, wgu, gr, 1, weight_layout=layout)
    return moe.moe_down(act, wd, w_recv, gr, P, 1, weight_layout=layout), lay["block_m"]


@pytest.mark.parametrize("N,H,E,k,I,G,blocked", [(512, 256, 32, 4, 128, 8, False), (1000, 128, 64, 8, 192, 8, True),
                                                 (2048, 256, 128, 8, 128, 8, True), (300, 64, 12, 3, 64, 4, False)])
def test_ep_shards_match_oracle(N, H, E, k, I, G, blocked):
    cfg = random_case(N, H, E, k, I, dtype="bf16", seed=21)
    t = make_inputs(cfg, DEV)
    ids, w, _ = moe.moe_route(t["x"], t["router_w"], k, cfg.norm_topk_prob)
    h = {n: t[n].float().cpu().numpy() for n in ("x", "router_w", "w_gate_up", "w_down")}
    ids_ref, w_ref, _, margin = O.route(h["x"], h["router_w"], k, cfg.norm_topk_prob)
    keep = margin >= MARGIN
    assert np.array_equal(ids.cpu().numpy()[keep], ids_ref[keep])
    y_all = torch.empty((N * k, H), dtype=t["x"].dtype, device=DEV)
    seen = torch.zeros(N * k, dtype=torch.int32, device=DEV)
    for g in range(G):
        sel, x_recv, ids_local, w_recv, wgu, wd = shard(t, ids, w, G, g, k, blocked)
        if sel.numel() == 0:
            continue
        y, bm = run_shard(x_recv, ids_local, w_recv, wgu, wd, E // G, blocked)
        torch.cuda.synchronize()
        # every received row against the oracle: w * Expert_e(x[token]) in float64
        sel_h = sel.cpu().numpy()
        tok, slot = sel_h // k, sel_h % k
        rows = keep[tok]
        e_glob = ids_ref[tok, slot]
        ref = np.zeros((sel_h.size, H))
        for e in np.unique(e_glob[rows]):
            m = rows & (e_glob == e)
            wg, wu = h["w_gate_up"][e, :I], h["w_gate_up"][e, I:]
            ref[m] = w_ref[tok[m], slot[m]][:, None] * O.swiglu(h["x"][tok[m]], wg, wu, h["w_down"][e])
        got = y.float().cpu().numpy()
        tol = O.tolerance(ref[rows], "bf16")
        assert np.abs(got[rows] - ref[rows]).max() <= tol, f"shard {g} (block_m {bm})"
        y_all[sel] = y
        seen[sel] += 1
    assert bool((seen == 1).all()), "every pair goes to exactly one shard"
    out = moe.moe_combine(y_all, N, k)
    ref_out, _ = O.moe_forward(h["x"], h["router_w"], h["w_gate_up"], h["w_down"], k, cfg.norm_topk_prob)
    got = out.float().cpu().numpy()
    print(f"EP shards G={G}: {int((~keep).sum())} near-tie tokens left out")
    assert np.abs(got[keep] - ref_out[keep]).max() <= O.tolerance(ref_out[keep], "bf16")
