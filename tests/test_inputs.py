"""The seeded input generators (no GPU)."""
import math

import numpy as np
import torch

from sparse_moe_ffn_amd import inputs as I


def test_configs_shapes():
    c = I.CONFIGS
    assert (c["tiny"].N, c["tiny"].H, c["tiny"].E, c["tiny"].top_k, c["tiny"].I) == (8, 64, 6, 2, 128)
    assert c["tiny"].dtype == "f32" and c["tiny"].std == 0.05
    for name, n in (("decode", 64), ("prefill", 4096), ("skew", 16384), ("talker", 8192)):
        cf = c[name]
        assert (cf.N, cf.H, cf.E, cf.top_k, cf.I, cf.dtype) == (n, 2048, 128, 8, 768, "bf16")
    assert c["skew"].norm_topk_prob is False and c["talker"].I_shared == 2048
    assert math.isclose(c["prefill"].flops() / 1e9, 311.4, rel_tol=1e-3)
    assert math.isclose(c["talker"].flops() / 1e9, 829.0, rel_tol=2e-3)


def test_tiny_inputs_deterministic():
    a = I.make_inputs(I.CONFIGS["tiny"])
    b = I.make_inputs(I.CONFIGS["tiny"])
    for k in ("x", "router_w", "w_gate_up", "w_down"):
        assert a[k].dtype == torch.float32 and torch.equal(a[k], b[k])
    assert a["w_gate_up"].shape == (6, 256, 64) and a["w_down"].shape == (6, 64, 128)
    assert a["shared_gate"] is None
    assert abs(float(a["router_w"].std()) - 0.05) < 0.005


def test_shared_and_bf16_draws():
    cfg = I.random_case(5, 64, 4, 2, 64, I_shared=64, dtype="bf16", seed=3)
    t = I.make_inputs(cfg)
    assert t["x"].dtype == torch.bfloat16
    assert t["shared_w_gate_up"].shape == (128, 64) and t["shared_w_down"].shape == (64, 64)
    assert t["shared_gate"].shape == (64,)


def test_zipf_targets_water_filled():
    t = I.zipf_targets(120, 16384 * 8, 16384, 1.2)
    assert abs(t.sum() - 16384 * 8) < 1e-3
    assert t.max() <= 16384 and (t == 16384).sum() == 2
    assert np.all(np.diff(t) <= 1e-9)
    free = t[t < 16384]
    slope = np.polyfit(np.log(np.arange(3, 121)), np.log(free), 1)[0]
    assert abs(slope + 1.2) < 1e-6


def test_skew_model_fit():
    cfg = I.CONFIGS["skew"]
    sigma = cfg.std * math.sqrt(cfg.H - 1)
    live, targets = I._fit_live_biases(120, cfg.N, cfg.top_k, round(sigma, 6), cfg.skew_s)
    live = np.array(live)
    assert np.all(np.diff(live) <= 1e-9)                    # higher rank, higher bias
    z = np.linspace(-7, 7, 141)
    wz = np.exp(-0.5 * z * z)
    wz /= wz.sum()
    load = cfg.N * I._inclusion_prob(live, cfg.top_k, sigma, z, wz)
    assert abs(load.sum() - cfg.N * cfg.top_k) < 1.0       # k experts per token
    assert np.max(np.abs(np.log(load[2:] / np.array(targets)[2:]))) < 0.05
    perm = torch.randperm(cfg.E, generator=torch.Generator().manual_seed(0))
    b = I.skew_biases(cfg, perm)
    assert int((b == -64).sum()) == cfg.skew_dead
