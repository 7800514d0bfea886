"""moe_forward_noalloc (the allocation-free entry point) through the C ABI:
its output must equal moe_forward's bit for bit (same kernels on the same
inputs, only the workspace differs), on two calls in a row with the second
smaller, on the grouped and the small-batch schedules, with a shared expert
and in float32; a problem too large for the fixed scratch is rejected."""
import pytest
import torch

import sparse_moe_ffn_amd as moe
from sparse_moe_ffn_amd.binding import MOE_ENOSPC, MoEError
from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def args(t, cfg):
    return (t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
            t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])


def fits(cfg, t):
    p = moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], cfg.top_k, cfg.norm_topk_prob, t["shared_w_gate_up"])
    return moe.moe_workspace_size(p) <= moe.MOE_NOALLOC_SCRATCH_BYTES


# (first call, second smaller call): decode layer (small-batch products) then a
# ragged grouped batch; a grouped batch with a shared expert then one token;
# float32 tiny layer then fewer tokens.
PAIRS = [
    (CONFIGS["decode"], random_case(20, 2048, 128, 8, 768, seed=3)),
    (random_case(700, 256, 32, 4, 128, I_shared=64, seed=4), random_case(1, 256, 32, 4, 128, I_shared=64, seed=5)),
    (random_case(800, 2048, 128, 8, 768, seed=6), CONFIGS["decode"]),
    (CONFIGS["tiny"], random_case(3, 64, 6, 2, 128, dtype="f32", seed=7)),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=lambda c: c.name)
def test_noalloc_equals_forward_on_two_calls(first, second):
    for i, cfg in enumerate((first, second)):
        t = make_inputs(cfg, DEV)
        assert fits(cfg, t), f"{cfg.name} needs more scratch than the fixed array"
        print(f"call {i}: {cfg.name}", flush=True)
        out = torch.full_like(t["x"], float("nan"))
        moe.moe_forward_noalloc(*args(t, cfg), out=out)
        ref = moe.moe_forward(*args(t, cfg))
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {i} ({cfg.name}): differs from moe_forward"


def test_noalloc_blocked_weights():
    cfg = CONFIGS["decode"]
    t = make_inputs(cfg, DEV)
    wgu, wd = moe.moe_pack_weights(t["w_gate_up"]), moe.moe_pack_weights(t["w_down"])
    out = moe.moe_forward_noalloc(t["x"], t["router_w"], wgu, wd, cfg.top_k, cfg.norm_topk_prob,
                                  weight_layout=moe.MOE_LAYOUT_BLOCKED)
    ref = moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_rejects_problems_beyond_the_scratch():
    cfg = CONFIGS["prefill"]
    p = moe.problem(cfg.N, cfg.H, cfg.E, cfg.top_k, cfg.I)
    assert moe.moe_workspace_size(p) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((cfg.N, cfg.H), dtype=torch.bfloat16, device=DEV)
    rw = torch.zeros((cfg.E, cfg.H), dtype=torch.bfloat16, device=DEV)
    wgu = torch.zeros((cfg.E, 2 * cfg.I, cfg.H), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((cfg.E, cfg.H, cfg.I), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(MoEError) as ei:
        moe.moe_forward_noalloc(x, rw, wgu, wd, cfg.top_k, True)
    assert ei.value.code == MOE_ENOSPC and "scratch" in str(ei.value)
