"""Host-side arithmetic of bench.py (no GPU): the algorithmic work per
kernel and per stage, the per-stage roofline, the dominant kernel's roofline
and the expert-load report, against values worked out by hand from the
layer shapes."""
import numpy as np

import bench
from sparse_moe_ffn_amd.inputs import CONFIGS


def test_kernel_work_prefill_closed_form():
    cfg = CONFIGS["prefill"]                          # N=4096, H=2048, E=128, k=8, I=768, bf16
    counts = np.full(cfg.E, cfg.N * cfg.top_k // cfg.E)
    w = bench.kernel_work(cfg, counts)
    P = 4096 * 8
    assert w["gate_up"]["bytes"] == 128 * 2 * 768 * 2048 * 2 + 4096 * 2048 * 2 + P * 768 * 2
    assert w["down"]["bytes"] == 128 * 2048 * 768 * 2 + P * 768 * 2 + P * 2048 * 2
    assert w["gate_up"]["flops"] == 2.0 * P * 2048 * 1536
    assert w["down"]["flops"] == 2.0 * P * 768 * 2048
    # only hit experts' weights count
    counts[:10] = 0
    assert bench.kernel_work(cfg, counts)["down"]["bytes"] == 118 * 2048 * 768 * 2 + P * 768 * 2 + P * 2048 * 2


def test_stage_work_and_roofline():
    cfg = CONFIGS["talker"]                           # N=8192, shared expert I_s=2048
    counts = np.array([0, 1, 320, 321, 5000] + [0] * (cfg.E - 5))
    counts[5] = cfg.N * cfg.top_k - counts.sum()
    w = bench.stage_work(cfg, counts, 320, False)
    N, H, E, k, Is = cfg.N, cfg.H, cfg.E, cfg.top_k, cfg.I_shared
    assert w["route"]["bytes"] == N * H * 2 + (E + 1) * H * 2 + N * k * 8 + N * 4
    assert w["route"]["flops"] == 2.0 * N * H * (E + 1)
    padded = sum(-(-int(c) // 320) * 320 for c in counts)
    assert padded == 0 + 320 + 320 + 640 + 5120 + -(-int(counts[5]) // 320) * 320
    assert w["align"]["bytes"] == N * k * 8 + padded * 4
    assert w["shared"]["flops"] == 2.0 * N * H * 2 * Is + 2.0 * N * Is * H
    assert w["combine"]["bytes"] == N * k * H * 2 + 2 * N * H * 2
    assert set(w) == {"route", "align", "gate_up", "down", "shared", "combine"}
    # the ids path has no align stage
    assert "align" not in bench.stage_work(CONFIGS["decode"], np.full(128, 4), 16, True)
    res = {"stage_median_ms": {"combine": 0.05, "gate_up": 0.4}, "stage_work": w}
    r = bench.stage_roofline(res)
    assert r["combine"]["bound"] == "hbm"
    assert abs(r["combine"]["frac"] - w["combine"]["bytes"] / 8e12 / 0.05e-3) < 1e-4
    # gate/up of the talker: 2*P*H*2I flops against its bytes; the longer bound wins
    gu = w["gate_up"]
    t_hbm, t_mfma = gu["bytes"] / 8e12, gu["flops"] / 2516.6e12
    assert r["gate_up"]["bound"] == ("hbm" if t_hbm >= t_mfma else "mfma")
    assert abs(r["gate_up"]["frac"] - max(t_hbm, t_mfma) / 0.4e-3) < 1e-4


def test_roofline_for_decode_is_hbm_bound():
    cfg = CONFIGS["decode"]
    counts = np.full(cfg.E, 4)
    work = bench.kernel_work(cfg, counts)
    res = {"cfg": cfg, "stage_ms": {"gate_up": 0.12}, "work": work, "ids_path": True, "block_m": 16}
    r = bench.roofline_for(res)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - work["gate_up"]["bytes"] / 0.12e-3 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4


def test_load_report_recovers_a_zipf_slope():
    cfg = CONFIGS["skew"]
    rank = np.arange(1, 121)
    counts = np.concatenate([np.round(10000.0 * rank ** -1.2), np.zeros(8)])
    rep = bench.load_report(counts, cfg)
    assert rep["experts_with_no_pairs"] == 8 and rep["counts_min"] == 0 and rep["counts_max"] == 10000
    assert abs(rep["loglog_slope_live"] + 1.2) < 0.02
    assert rep["counts_desc"][0] == 10000 and len(rep["counts_desc"]) == 128
