"""moe_forward on two streams at once.  Without a caller workspace the
binding keeps one workspace per (device, stream), so two forwards that run
concurrently on different streams must not share intermediates: each
stream's outputs must equal the same calls made one after the other."""
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


def _forward(t, cfg):
    return moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                           t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])


def test_forward_on_two_streams_concurrently():
    # Two problems of the same shape (so the same workspace size) and one of
    # another shape, each with its own inputs.
    cases = [random_case(3000, 256, 64, 8, 128, dtype="bf16", seed=21),
             random_case(3000, 256, 64, 8, 128, dtype="bf16", seed=22),
             random_case(700, 192, 32, 4, 64, I_shared=128, dtype="bf16", seed=23)]
    inputs = [make_inputs(c, DEV) for c in cases]
    ref = [_forward(t, c) for t, c in zip(inputs, cases)]        # one after the other
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]  # default priority
    cur = torch.cuda.current_stream(DEV)
    for s in streams:
        s.wait_stream(cur)
    outs = []
    for rep in range(4):
        for i, (t, c) in enumerate(zip(inputs, cases)):
            s = streams[(i + rep) % 2]
            with torch.cuda.stream(s):
                outs.append((i, rep, _forward(t, c)))
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    for i, rep, o in outs:
        assert torch.equal(o, ref[i]), f"case {i}, round {rep}: differs from the call made alone"
