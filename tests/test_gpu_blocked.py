"""Expert weights in the blocked layout (moe_pack_weights): the packed
storage follows the documented index formula bit for bit, and every product
gives bit for bit the output of the row-major layout (same instructions,
same summation order; only the addresses of the weight loads differ)."""
import pytest
import torch

import sparse_moe_ffn_amd as moe
from sparse_moe_ffn_amd.inputs import CONFIGS, DENSE_LAYERS, make_dense_inputs, make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BLK = moe.MOE_LAYOUT_BLOCKED


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


@pytest.mark.parametrize("shape", [(3, 24, 192), (1, 8, 64), (2, 1536, 2048), (16, 64)])
def test_pack_follows_index_formula(shape):
    g = torch.Generator(device="cpu").manual_seed(sum(shape))
    bits = torch.randint(-32768, 32767, shape, generator=g, dtype=torch.int16)
    w = bits.view(torch.bfloat16).to(DEV)
    packed = moe.moe_pack_weights(w)
    torch.cuda.synchronize()
    b, r, c = (1,) + shape if len(shape) == 2 else shape
    # element (b, r, c) at b*R*C + (c/64)*R*64 + r*64 + c%64: 64-column panels, rows inside
    expect = bits.reshape(b, r, c // 64, 64).permute(0, 2, 1, 3).reshape(-1)
    assert torch.equal(packed.cpu().view(torch.int16).reshape(-1), expect)


def pack_all(t):
    return {k: (moe.moe_pack_weights(v) if k in ("w_gate_up", "w_down", "shared_w_gate_up", "shared_w_down")
                and v is not None else v) for k, v in t.items()}


def forward(t, cfg, layout):
    return moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                           t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"], weight_layout=layout)


# tile heights 16, 16, 128, 32, 64, 320 (the last also with partial column blocks)
CASES = [random_case(1, 128, 6, 6, 64), random_case(37, 192, 16, 4, 128, I_shared=64, seed=2),
         random_case(700, 320, 16, 4, 256, seed=4), random_case(97, 2048, 32, 8, 768),
         random_case(600, 128, 16, 2, 64, seed=5), random_case(2000, 320, 8, 2, 192, I_shared=64, seed=6)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_blocked_equals_row_major(cfg):
    t = make_inputs(cfg, DEV)
    ref = forward(t, cfg, moe.MOE_LAYOUT_ROW_MAJOR)
    out = forward(pack_all(t), cfg, BLK)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode", "prefill", "skew", "talker"])
def test_forward_blocked_equals_row_major_full_size(name):
    cfg = CONFIGS[name]
    t = make_inputs(cfg, DEV)
    ref = forward(t, cfg, moe.MOE_LAYOUT_ROW_MAJOR)
    tb = pack_all(t)
    del t
    out = forward(tb, cfg, BLK)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("N,H,I", [(5, 128, 64), (600, 256, 192), (4096, 2048, 6144)])
def test_dense_mlp_blocked_equals_row_major(N, H, I):
    t = make_dense_inputs(N, H, I, seed=7, device=DEV)
    ref = moe.moe_dense_mlp(t["x"], t["w_gate_up"], t["w_down"])
    out = moe.moe_dense_mlp(t["x"], moe.moe_pack_weights(t["w_gate_up"]), moe.moe_pack_weights(t["w_down"]),
                            weight_layout=BLK)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_staged_blocked_equals_forward():
    cfg = random_case(300, 256, 24, 6, 128, seed=9)
    t = make_inputs(cfg, DEV)
    tb = pack_all(t)
    out = forward(tb, cfg, BLK)
    lay = moe.moe_get_workspace_layout(moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], cfg.top_k,
                                                        cfg.norm_topk_prob))
    ids, w, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    gr = moe.moe_align(ids, cfg.E, lay["block_m"])
    act = moe.moe_gate_up(t["x"], tb["w_gate_up"], gr, cfg.top_k, weight_layout=BLK)
    y = moe.moe_down(act, tb["w_down"], w, gr, cfg.N, cfg.top_k, weight_layout=BLK)
    out2 = moe.moe_combine(y, cfg.N, cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
