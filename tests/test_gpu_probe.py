"""The matrix-unit rate probe (measurement only): it runs through the C ABI,
returns the flop count of its launch, and its measured rate is physical --
not above the datasheet bf16 peak (which a loop the compiler removed would
exceed) and not absurdly low."""
import pytest
import torch

import sparse_moe_ffn_amd as moe
from sparse_moe_ffn_amd import binding as B

pytestmark = pytest.mark.gpu
DATASHEET_BF16_TFLOPS = 2516.6


def test_probe_rate_is_physical():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    g = torch.Generator(device="cuda:0").manual_seed(1)
    ops = torch.randn(1 << 16, generator=g, device="cuda:0").to(torch.bfloat16)
    sink = torch.empty(B.MOE_PROBE_SINK_FLOATS, dtype=torch.float32, device="cuda:0")
    iters = 2048
    flops = moe.moe_mfma_probe(ops, iters, sink)
    assert flops == B.MOE_PROBE_WORKGROUPS * 8 * 8 * iters * 2 * 16 * 16 * 32
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(5):
        e0.record()
        moe.moe_mfma_probe(ops, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    tflops = flops / (min(times) * 1e-3) / 1e12
    print(f"probe: {tflops:.0f} TFLOP/s ({tflops / DATASHEET_BF16_TFLOPS:.2f} of the datasheet bf16 peak)")
    assert 100.0 < tflops < 1.02 * DATASHEET_BF16_TFLOPS


def test_probe_rejects_bad_operands():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    with pytest.raises(ValueError):
        moe.moe_mfma_probe(torch.zeros(100, dtype=torch.bfloat16, device="cuda:0"), 10)
    with pytest.raises(ValueError):
        moe.moe_mfma_probe(torch.zeros(512, dtype=torch.float32, device="cuda:0"), 10)
