"""GPU parity of the rows around the block: the dense SwiGLU layer and the
residual add + RMSNorm in front of it, plus the decode block (norm + MoE)
captured in a HIP graph and replayed.

Outputs: |gpu - ref| <= 2e-2 * max|ref| + 1e-3 in bf16, <= 1e-4 * max|ref|
in fp32.  The new residual (a float32 sum rounded once to the dtype) is
compared bit for bit.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_amd as moe
from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import CONFIGS, DENSE_LAYERS, make_dense_inputs, make_inputs, make_norm_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MARGIN = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def host(t):
    return t.float().cpu().numpy()


def check(out, ref, dtype, what):
    tol = O.tolerance(ref, dtype)
    err = float(np.abs(out - ref).max()) if ref.size else 0.0
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max|gpu-ref| = {err:.4e} > tol {tol:.4e}"
    print(f"{what}: err {err:.3e} tol {tol:.3e}")


# ------------------------------------------------------------ dense SwiGLU

# The trailing comments give the gate/up row-tile height the library picks
# (the tallest that still fills half the CUs, 256 instead of 320 rows when
# that takes no more rounds of workgroups) and the down height where it
# differs (the tallest that gives 160 workgroups, else 32 rows while a launch
# of 32x128 tiles fits one round, else 64).  Every case ends in a ragged row
# tile.
DENSE_SMALL = [(1, 64, 64, "bf16"), (37, 128, 192, "bf16"),            # 16
               (200, 256, 128, "bf16"), (333, 192, 448, "bf16"),       # 16
               (200, 256, 1472, "bf16"), (4100, 128, 64, "bf16"),      # 32
               (600, 128, 2048, "bf16"), (4200, 256, 320, "bf16"),     # 64 (down 32)
               (2500, 1024, 512, "bf16"),                              # 64
               (1300, 1024, 2048, "bf16"),                             # 128 (down 32)
               (700, 128, 5440, "bf16"),                               # 256 (down 32), ragged column block
               (1900, 128, 5120, "bf16"),                              # 320 (256 rows: a second round)
               (1000, 2048, 512, "bf16"),                              # 32 (down 32x128: 1024 32x64 tiles)
               (1100, 2048, 1024, "bf16"),                             # 64 (down 64: 32x128 past a round)
               (5, 24, 40, "f32"), (70, 33, 17, "f32")]


@pytest.mark.parametrize("N,H,I,dtype", DENSE_SMALL)
def test_dense_mlp_small(N, H, I, dtype):
    t = make_dense_inputs(N, H, I, dtype=dtype, seed=N + I, std=0.05 if dtype == "f32" else 0.02, device=DEV)
    out = moe.moe_dense_mlp(t["x"], t["w_gate_up"], t["w_down"])
    torch.cuda.synchronize()
    ref = O.dense_mlp(host(t["x"]), host(t["w_gate_up"]), host(t["w_down"]))
    check(host(out), ref, dtype, f"dense N{N} H{H} I{I} {dtype}")


@pytest.mark.parametrize("N,H,I", [(3072, 4096, 6144),    # gate/up and down 320-row tiles
                                   (2900, 4096, 1664),    # 256 / 128
                                   (4096, 2048, 6144),    # 256 / 128
                                   (2048, 2048, 6144),    # 256 / 64
                                   (1536, 2048, 6144),    # 320 / 64 (256 rows: a second round)
                                   (1152, 2048, 6144),    # 256 / 64 (32x128 tiles past a round)
                                   (1024, 2048, 6144),    # 256 / 32 with 128 columns
                                   (512, 2048, 6144),     # 128 / 32
                                   (64, 2048, 6144),      # 32 / 32
                                   (16, 2048, 6144)])     # 16 / 16
def test_dense_tile_heights_bitwise(N, H, I):
    """Rows of a dense layer computed alone (16-row tiles for both products)
    equal the same rows inside the batch, whose tiles are taller, bit for
    bit: every tile height sums each element in one K order."""
    t = make_dense_inputs(N, H, I, seed=N + H, device=DEV)
    full = moe.moe_dense_mlp(t["x"], t["w_gate_up"], t["w_down"])
    for lo, hi in ((0, 3), (N - 2, N)):
        part = moe.moe_dense_mlp(t["x"][lo:hi].contiguous(), t["w_gate_up"], t["w_down"])
        torch.cuda.synchronize()
        assert torch.equal(part, full[lo:hi]), f"rows [{lo}, {hi}) differ from the batch of {N}"


@pytest.mark.slow
@pytest.mark.parametrize("name", ["dense_decode", "dense_prefill"])
def test_dense_mlp_full_size(name):
    L = DENSE_LAYERS[name]
    t = make_dense_inputs(L["N"], L["H"], L["I"], device=DEV)
    out = moe.moe_dense_mlp(t["x"], t["w_gate_up"], t["w_down"])
    out2 = moe.moe_dense_mlp(t["x"], t["w_gate_up"], t["w_down"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ref = O.dense_mlp(host(t["x"]), host(t["w_gate_up"]), host(t["w_down"]))      # every row
    check(host(out), ref, "bf16", name)
    one = moe.moe_dense_mlp(t["x"][5:6].contiguous(), t["w_gate_up"], t["w_down"])
    assert torch.equal(one[0], out[5]), "a row alone differs from the same row in the batch"


# ------------------------------------------------------ residual add + RMSNorm

@pytest.mark.parametrize("N,H,dtype,with_res", [
    (1, 64, "bf16", True), (64, 2048, "bf16", True), (64, 2048, "bf16", False), (4096, 2048, "bf16", True),
    (3, 16384, "bf16", True), (17, 200, "f32", True), (8, 64, "f32", False), (5, 2056, "bf16", True)])
def test_add_rmsnorm(N, H, dtype, with_res):
    t = make_norm_inputs(N, H, dtype=dtype, seed=H + N, device=DEV)
    res = t["residual"] if with_res else None
    normed, r = moe.moe_add_rmsnorm(t["x"], res, t["weight"], 1e-6)
    torch.cuda.synchronize()
    n_ref, r_ref = O.add_rmsnorm(host(t["x"]), None if res is None else host(res), host(t["weight"]), 1e-6, dtype)
    assert np.array_equal(host(r), r_ref), "new residual differs"
    check(host(normed), n_ref, dtype, f"rmsnorm N{N} H{H} {dtype}")


def test_add_rmsnorm_in_place_and_batch_invariant():
    t = make_norm_inputs(64, 2048, seed=9, device=DEV)
    n_ref, r_ref = moe.moe_add_rmsnorm(t["x"], t["residual"], t["weight"], 1e-6)
    res = t["residual"].clone()
    normed, r = moe.moe_add_rmsnorm(t["x"], res, t["weight"], 1e-6, residual_out=res)
    one, _ = moe.moe_add_rmsnorm(t["x"][9:10].contiguous(), t["residual"][9:10].contiguous(), t["weight"], 1e-6)
    torch.cuda.synchronize()
    assert r.data_ptr() == res.data_ptr()
    assert torch.equal(res, r_ref) and torch.equal(normed, n_ref)
    assert torch.equal(one[0], n_ref[9])


# --------------------------------------------- decode block in a HIP graph

def test_decode_block_graph_replays_match_eager_and_oracle():
    """Residual add + RMSNorm, then the MoE block, on the 64-token decode
    layer, captured once and replayed with new inputs copied in between."""
    cfg = CONFIGS["decode"]
    t = make_inputs(cfg, DEV)
    nrm = [make_norm_inputs(cfg.N, cfg.H, seed=s, device=DEV) for s in range(3)]
    weight = nrm[0]["weight"]
    x_in = torch.empty_like(nrm[0]["x"])
    res_in = torch.empty_like(nrm[0]["residual"])
    res_out = torch.empty_like(res_in)
    normed = torch.empty_like(x_in)
    out = torch.empty_like(x_in)
    p = moe.problem_from(normed, t["w_gate_up"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device=DEV)

    def block():
        moe.moe_add_rmsnorm(x_in, res_in, weight, 1e-6, residual_out=res_out, normed=normed)
        moe.moe_forward(normed, t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                        out=out, workspace=ws)

    x_in.copy_(nrm[0]["x"])
    res_in.copy_(nrm[0]["residual"])
    block()                                   # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block()
    torch.cuda.synchronize()
    h = {"router_w": host(t["router_w"]), "w_gate_up": host(t["w_gate_up"]), "w_down": host(t["w_down"])}
    for rep in range(6):
        src = nrm[rep % 3]
        x_in.copy_(src["x"])
        res_in.copy_(src["residual"])
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_res = out.clone(), res_out.clone()
        out.zero_()                          # eager work between replays
        block()
        torch.cuda.synchronize()
        assert torch.equal(got_out, out), f"replay {rep}: output differs from eager"
        assert torch.equal(got_res, res_out), f"replay {rep}: residual differs from eager"
        if rep < 3:
            n_ref, r_ref = O.add_rmsnorm(host(src["x"]), host(src["residual"]), host(weight), 1e-6, "bf16")
            assert np.array_equal(host(got_res), r_ref)
            xb = O.round_to(n_ref, "bf16")               # the block reads the normalised rows as bf16
            routing = O.route(xb, h["router_w"], cfg.top_k, cfg.norm_topk_prob)
            keep = routing[3] >= MARGIN
            rows = [r for r in range(cfg.N) if keep[r]]                # every token the margin rule keeps
            ref, _ = O.moe_forward(xb, h["router_w"], h["w_gate_up"], h["w_down"], cfg.top_k, cfg.norm_topk_prob,
                                   rows=rows, routing=routing)
            check(host(got_out)[rows], ref, "bf16", f"graph block replay {rep} ({len(rows)} rows)")
    del graph
