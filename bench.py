#!/usr/bin/env python3
"""Throughput of the sparse MoE FFN block on one MI355X.

One step = one full pass of the block (router, align, gate/up, down,
[shared expert], combine) over one batch of seeded synthetic tokens already
resident in HBM, through the C ABI (``moe_forward``).  Expert weights are
packed once into the library's blocked layout before timing (a weight-load
step, ``moe_pack_weights``); the same step with row-major weights is timed
too and reported as ``ms_per_step_row_major``.

Prints ONE JSON line.  ``value`` is tokens/s of the main workload (default:
the 64-token decode layer, H=2048, E=128, top-8, I=768, bf16).  ``roofline``
is for the dominant kernel of that workload, timed with HIP events on the
stream the kernels run on, in a second loop that issues the same stages one
by one.  ``cpu_baseline`` times the CPU oracle on a bounded token sample.
``also`` holds the same figures for the other workloads given with --also
(by default the 4096-token prefill layer, the 16384-token skewed layer with
its expert-load report, the 8192-token talker layer with a shared expert, a
dense SwiGLU layer, the graph-replayed decode block and one GPU's
expert-parallel share of an 8 x 4096-token prefill batch), each timed over
the same number of steps as the main workload.  Every step time is given as
the wall-clock mean over the timed steps, run back to back, and as the
median / min / mean of per-step HIP events from a second loop of the same
steps.  ``mfma_peak_measured`` is the matrix-unit rate the library's probe
sustains in the same run, a second reference beside the datasheet peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak (datasheet, no sparsity)
METRIC = "MoE-layer tokens/s; % bf16 MFMA peak (prefill), % HBM BW (decode)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skew", "talker"])
    ap.add_argument("--also", default="prefill,skew,talker,dense_prefill,decode_block,ep8_share",
                    help="comma-separated extra workloads ('' for none): prefill, skew, talker, decode, "
                         "dense_prefill, dense_decode (dense SwiGLU layers), decode_block (residual add + "
                         "RMSNorm + the decode MoE layer, eager and replayed from a HIP graph), ep8_share "
                         "(one GPU's expert-parallel share of an 8 x 4096-token prefill batch)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle budget: whole passes over the main workload on all cores for about this "
                         "long, then a single-thread sample of a third of it (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def expert_hits(counts):
    return int((counts > 0).sum())


def kernel_work(cfg, counts):
    """Algorithmic bytes and flops per launch of each kernel.

    gate_up: weights of every hit expert (2I x H) once, each token's x row
    once, and one act row (I) per pair; flops 2*H*2I per pair.
    down: weights of every hit expert (H x I) once, one act row in and one y
    row (H) out per pair; flops 2*I*H per pair.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    P = cfg.N * cfg.top_k
    hit = expert_hits(counts)
    gu_bytes = hit * 2 * cfg.I * cfg.H * es + cfg.N * cfg.H * es + P * cfg.I * es
    dn_bytes = hit * cfg.H * cfg.I * es + P * cfg.I * es + P * cfg.H * es
    return {
        "gate_up": {"bytes": gu_bytes, "flops": 2.0 * P * cfg.H * 2 * cfg.I},
        "down": {"bytes": dn_bytes, "flops": 2.0 * P * cfg.I * cfg.H},
    }


def stage_work(cfg, counts, block_m, ids_path):
    """Algorithmic bytes and flops of every stage of one step (the staged
    calls of bench_workload), for the per-stage roofline.

    route: x and the router rows (plus the shared gate) read once, ids and
    weights (plus the shared scale) written; flops 2*H per logit.
    align: the N*k ids read, the stable order and the padded pair list
    written (int32).  gate_up, down: kernel_work.  shared: the shared
    expert's weights and x read once, its act written and read, its output
    row written; flops 2*H*2I_s + 2*I_s*H per token.  combine: the k rows of
    y per token (plus the shared row) read, the output row written.
    """
    es = 2 if cfg.dtype == "bf16" else 4
    N, H, E, k, Is = cfg.N, cfg.H, cfg.E, cfg.top_k, cfg.I_shared
    P = N * k
    cols = E + (1 if Is else 0)
    w = dict(kernel_work(cfg, counts))
    w["route"] = {"bytes": N * H * es + cols * H * es + P * 8 + (N * 4 if Is else 0), "flops": 2.0 * N * H * cols}
    if not ids_path:
        padded = int(sum(-(-int(c) // block_m) * block_m for c in counts))
        w["align"] = {"bytes": P * 4 + P * 4 + padded * 4, "flops": 0.0}
    if Is:
        w["shared"] = {"bytes": 3 * Is * H * es + N * H * es + 2 * N * Is * es + N * H * es,
                       "flops": 2.0 * N * H * 2 * Is + 2.0 * N * Is * H}
    w["combine"] = {"bytes": P * H * es + N * H * es + (N * H * es if Is else 0), "flops": 0.0}
    return w


def stage_roofline(res):
    """Each stage's median time against the roof that bounds it (the longer
    of bytes at the HBM peak and flops at the bf16 MFMA peak)."""
    out = {}
    for name, ms in res["stage_median_ms"].items():
        w = res["stage_work"].get(name)
        if w is None or ms <= 0:
            continue
        t = ms * 1e-3
        hbm_t = w["bytes"] / (HBM_PEAK_GBS * 1e9)
        mfma_t = w["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        bound = "hbm" if hbm_t >= mfma_t else "mfma"
        out[name] = {"ms": round(ms, 5), "bytes": int(w["bytes"]), "flops": w["flops"], "bound": bound,
                     "frac": round(max(hbm_t, mfma_t) / t, 4)}
    return out


def timed_steps(fn, steps, warmup, torch):
    """Run `warmup` untimed steps, then exactly `steps` timed ones back to
    back between two device synchronisations: the wall-clock mean per step
    (ms).  Then the same number of steps again with a HIP event recorded
    after each one on torch's current stream (the stream every call is
    enqueued on): the per-step durations (ms).  The events sit in a loop of
    their own because each record adds a few microseconds to a step."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return wall, per


def event_summary(per):
    n = len(per)
    med = per[n // 2] if n % 2 else 0.5 * (per[n // 2 - 1] + per[n // 2])
    return {"median": round(med, 5), "min": round(per[0], 5), "mean": round(sum(per) / n, 5)}


def load_report(counts, cfg):
    """Pairs per expert: min / max, experts with none, and the log-log slope
    of count against rank over the experts that have pairs (least squares),
    also over the ranks below the N-pair cap (where the Zipf target is not
    cut off)."""
    import numpy as np

    c = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    live = c[c > 0]
    rank = np.arange(1, live.size + 1, dtype=np.float64)

    def slope(v, r):
        return float(np.polyfit(np.log(r), np.log(v), 1)[0]) if v.size >= 2 else None

    below = live < cfg.N
    return {"counts_min": int(c.min()), "counts_max": int(c.max()), "experts_with_no_pairs": int((c == 0).sum()),
            "loglog_slope_live": round(slope(live, rank), 4),
            "loglog_slope_below_cap": round(slope(live[below], rank[below]), 4),
            "experts_at_cap": int((live >= cfg.N).sum()), "target_zipf_s": cfg.skew_s,
            "counts_desc": [int(v) for v in c]}


def bench_workload(name, steps, warmup, torch, moe):
    from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    t = make_inputs(cfg, dev)
    blk = moe.MOE_LAYOUT_BLOCKED
    tw = {k: (moe.moe_pack_weights(t[k]) if t[k] is not None else None)
          for k in ("w_gate_up", "w_down", "shared_w_gate_up", "shared_w_down")}
    args = (t["x"], t["router_w"], tw["w_gate_up"], tw["w_down"], cfg.top_k, cfg.norm_topk_prob,
            tw["shared_w_gate_up"], tw["shared_w_down"], t["shared_gate"])
    args_rm = (t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
               t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])
    p = moe.problem_from(t["x"], t["w_gate_up"], t["router_w"], cfg.top_k, cfg.norm_topk_prob,
                         t["shared_w_gate_up"], blk)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["x"])
    wall, per = timed_steps(lambda: moe.moe_forward(*args, out=out, workspace=ws, weight_layout=blk),
                            steps, warmup, torch)
    ms_row_major, per_rm = timed_steps(lambda: moe.moe_forward(*args_rm, out=out, workspace=ws), steps, warmup, torch)

    # Same stages issued one by one, HIP events between them, on the stream
    # the kernels run on (torch's current stream).
    lay = moe.moe_get_workspace_layout(p)
    bm = lay["block_m"]
    ids_path = lay["ids_products"] == 1                # small batch: no grouping, the products scan the ids
    stages = (["route"] + ([] if ids_path else ["align"]) + ["gate_up", "down"] + (["shared"] if cfg.I_shared else [])
              + ["combine"])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    ids = torch.empty((cfg.N, cfg.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((cfg.N, cfg.top_k), dtype=torch.float32, device=dev)
    sscale = torch.empty(cfg.N, dtype=torch.float32, device=dev) if cfg.I_shared else None
    route_scratch = torch.empty(max(1, moe.moe_route_scratch_size(p) // 4), dtype=torch.float32, device=dev)
    align_scratch = torch.empty(max(1, moe.moe_align_scratch_size(cfg.N * cfg.top_k, cfg.E) // 4),
                                dtype=torch.int32, device=dev)
    gr = moe.moe_align(ids.zero_(), cfg.E, bm, align_scratch)
    act = torch.empty((max(gr.max_rows, cfg.N * cfg.top_k), cfg.I), dtype=t["x"].dtype, device=dev)
    y = torch.empty((cfg.N * cfg.top_k, cfg.H), dtype=t["x"].dtype, device=dev)
    sact = torch.empty((cfg.N, cfg.I_shared), dtype=t["x"].dtype, device=dev) if cfg.I_shared else None
    sy = torch.empty((cfg.N, cfg.H), dtype=t["x"].dtype, device=dev) if cfg.I_shared else None

    def staged(e):
        e[0].record()
        moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob, t["shared_gate"], ids, wts, sscale,
                      route_scratch)
        e[1].record()
        i = 2
        g2 = None
        if ids_path:
            moe.moe_gate_up_ids(t["x"], tw["w_gate_up"], ids, act, weight_layout=blk)
            e[i].record()
            moe.moe_down_ids(act, tw["w_down"], ids, wts, y, weight_layout=blk)
            e[i + 1].record()
        else:
            g2 = moe.moe_align(ids, cfg.E, bm, align_scratch)
            e[i].record()
            i += 1
            moe.moe_gate_up(t["x"], tw["w_gate_up"], g2, cfg.top_k, act, weight_layout=blk)
            e[i].record()
            moe.moe_down(act, tw["w_down"], wts, g2, cfg.N, cfg.top_k, y, weight_layout=blk)
            e[i + 1].record()
        i += 2
        if cfg.I_shared:
            moe.moe_shared_expert(t["x"], tw["shared_w_gate_up"], tw["shared_w_down"], sscale, sact, sy,
                                  weight_layout=blk)
            e[i].record()
            i += 1
        moe.moe_combine(y, cfg.N, cfg.top_k, sy, out)
        e[i].record()
        return g2

    for _ in range(min(warmup, 5)):
        staged(ev[0])
    torch.cuda.synchronize()
    for s in range(steps):
        staged(ev[s])
    torch.cuda.synchronize()
    stage_ms = {name_: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
                for i, name_ in enumerate(stages)}
    stage_median_ms = {name_: event_summary(sorted(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)))["median"]
                       for i, name_ in enumerate(stages)}
    counts = moe.moe_align(ids, cfg.E, bm, align_scratch).counts.cpu().numpy()   # untimed: pairs per expert
    work = kernel_work(cfg, counts)
    swork = stage_work(cfg, counts, bm, ids_path)
    ms = wall
    res = {
        "cfg": cfg, "inputs": t, "ms_per_step": ms, "tokens_per_s": cfg.N / (ms * 1e-3),
        "step_event_ms": event_summary(per), "ms_per_step_row_major": ms_row_major,
        "step_event_ms_row_major": event_summary(per_rm),
        "tflops": cfg.flops() / (ms * 1e-3) / 1e12, "stage_ms": stage_ms, "stage_median_ms": stage_median_ms,
        "work": work, "stage_work": swork, "hit_experts": expert_hits(counts),
        "counts_min_max": [int(counts.min()), int(counts.max())],
        "block_m": bm, "ids_path": ids_path, "counts": counts, "steps": steps,
    }
    med = res["step_event_ms"]["median"]
    res["tflops_median"] = cfg.flops() / (med * 1e-3) / 1e12
    res["mfma_frac"] = res["tflops"] / MFMA_BF16_PEAK_TFLOPS
    res["mfma_frac_median"] = res["tflops_median"] / MFMA_BF16_PEAK_TFLOPS
    weight_bytes = res["hit_experts"] * 3 * cfg.I * cfg.H * 2 + cfg.I_shared * 3 * cfg.H * 2
    res["weight_hbm_frac"] = weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    return res


def prewarm(torch, moe, seconds=1.0):
    """Untimed: keep the GPU busy with decode-layer steps for about a second
    so its clocks have settled before any timed loop (a cold GPU runs the
    first hundreds of milliseconds slower)."""
    from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS["decode"]
    t = make_inputs(cfg, "cuda:0")
    out = torch.empty_like(t["x"])
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob, out=out)
        torch.cuda.synchronize()
    del t, out
    torch.cuda.empty_cache()


MEASURED_PEAK = {}          # filled by measure_mfma_peak() before the workloads run


def measure_mfma_peak(torch, moe, iters=4096, reps=9):
    """The matrix-unit rate this part sustains: the library's probe (back to
    back 16x16x32 bf16 matrix instructions on random register operands, 16
    waves per CU) timed with events on the stream it runs on; median of
    `reps` launches.  A second reference beside the datasheet peak."""
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(1)
    ops = torch.randn(1 << 20, generator=g, device=dev).to(torch.bfloat16)
    sink = torch.empty(moe.MOE_PROBE_SINK_FLOATS, dtype=torch.float32, device=dev)
    for _ in range(3):
        moe.moe_mfma_probe(ops, iters, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    flops = 0.0
    for e0, e1 in ev:
        e0.record()
        flops = moe.moe_mfma_probe(ops, iters, sink)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    tf = flops / (ms * 1e-3) / 1e12
    MEASURED_PEAK.update({"tflops": round(tf, 1), "frac_of_datasheet": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                          "launch_ms": round(ms, 4),
                          "kernel": "16x16x32 bf16 matrix instructions back to back on random register operands, "
                                    "512 workgroups x 8 waves, 8 independent accumulators per wave"})
    return dict(MEASURED_PEAK)


def of_measured(tflops):
    return round(tflops / MEASURED_PEAK["tflops"], 4) if MEASURED_PEAK else None


def bench_dense(name, steps, warmup, torch, moe):
    """A dense SwiGLU layer (moe_dense_mlp) of hidden 2048, I = 6144."""
    from sparse_moe_ffn_amd.inputs import DENSE_LAYERS, make_dense_inputs

    L = DENSE_LAYERS[name]
    t = make_dense_inputs(L["N"], L["H"], L["I"], device="cuda:0")
    act = torch.empty((L["N"], L["I"]), dtype=t["x"].dtype, device="cuda:0")
    out = torch.empty_like(t["x"])
    wgu, wd = moe.moe_pack_weights(t["w_gate_up"]), moe.moe_pack_weights(t["w_down"])
    ms, per = timed_steps(lambda: moe.moe_dense_mlp(t["x"], wgu, wd, act=act, out=out,
                                                    weight_layout=moe.MOE_LAYOUT_BLOCKED), steps, warmup, torch)
    flops = 6.0 * L["N"] * L["H"] * L["I"]
    wbytes = 3 * L["H"] * L["I"] * 2
    return {"workload": f"{name}: dense SwiGLU layer N={L['N']} H={L['H']} I={L['I']} bf16",
            "steps": steps, "tokens_per_s": round(L["N"] / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "step_event_ms": event_summary(per), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_frac_of_measured_peak": of_measured(flops / (ms * 1e-3) / 1e12),
            "weight_hbm_frac": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_ep_share(steps, warmup, torch, moe, gpus=8):
    """One GPU's share of the prefill layer under expert parallelism over
    `gpus` GPUs (expert e on GPU e mod gpus), run on this one GPU: the global
    batch is gpus x 4096 tokens, every GPU's router is run here (untimed) and
    torch indexing stands in for the dispatch all-to-all, so this GPU holds
    the x rows of the pairs routed to its E/gpus experts.  The timed step is
    what that GPU computes: moe_align over the received pairs (local expert
    ids, one row per pair), then the grouped gate/up and down products.  The
    y rows would then go back to their tokens' GPUs for the combine."""
    from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs

    base = CONFIGS["prefill"]
    cfg = base.with_(name="ep_global", N=base.N * gpus)
    t = make_inputs(cfg, "cuda:0")
    ids, w, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    flat_ids, flat_w = ids.reshape(-1), w.reshape(-1)
    sel = torch.nonzero(flat_ids % gpus == 0).squeeze(1)          # pairs sent to GPU 0, pair order
    P, E_loc = sel.numel(), cfg.E // gpus
    x_recv = t["x"][torch.div(sel, cfg.top_k, rounding_mode="floor")].contiguous()
    ids_local = torch.div(flat_ids[sel], gpus, rounding_mode="floor").to(torch.int32).view(-1, 1).contiguous()
    w_recv = flat_w[sel].contiguous()
    wgu = moe.moe_pack_weights(t["w_gate_up"][0::gpus].contiguous())
    wd = moe.moe_pack_weights(t["w_down"][0::gpus].contiguous())
    del t, ids, w, flat_ids, flat_w
    torch.cuda.empty_cache()
    bm = moe.moe_get_workspace_layout(moe.problem(P, cfg.H, E_loc, 1, cfg.I))["block_m"]
    blk = moe.MOE_LAYOUT_BLOCKED
    gr = moe.moe_align(ids_local, E_loc, bm)
    act = moe.moe_gate_up(x_recv, wgu, gr, 1, weight_layout=blk)
    y = moe.moe_down(act, wd, w_recv, gr, P, 1, weight_layout=blk)

    def step():
        g = moe.moe_align(ids_local, E_loc, bm)
        moe.moe_gate_up(x_recv, wgu, g, 1, act=act, weight_layout=blk)
        moe.moe_down(act, wd, w_recv, g, P, 1, y=y, weight_layout=blk)

    ms, per = timed_steps(step, steps, warmup, torch)
    counts = gr.counts.cpu()
    ev = event_summary(per)
    flops = 6.0 * P * cfg.H * cfg.I
    tf = flops / (ev["median"] * 1e-3) / 1e12
    wbytes = E_loc * 3 * cfg.H * cfg.I * 2
    return {"workload": f"ep{gpus}_share: GPU 0 of {gpus} (experts e mod {gpus} == 0) in the {cfg.N}-token prefill "
                        f"batch: {P} received pairs over {E_loc} local experts, H={cfg.H} I={cfg.I} bf16, "
                        "step = align + gate/up + down (route, all-to-all and combine not on this GPU's path)",
            "steps": steps, "pairs": P, "block_m": bm, "counts_min_max": [int(counts.min()), int(counts.max())],
            "ms_per_step": round(ms, 4), "step_event_ms": ev, "tflops_median": round(tf, 1),
            "mfma_frac_median": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "mfma_frac_of_measured_peak": of_measured(tf),
            "weight_bytes": wbytes}


def bench_decode_block(steps, warmup, torch, moe):
    """Residual add + RMSNorm, then the decode MoE layer, issued eagerly and
    replayed from one captured HIP graph."""
    from sparse_moe_ffn_amd.inputs import CONFIGS, make_inputs, make_norm_inputs

    cfg = CONFIGS["decode"]
    t = make_inputs(cfg, "cuda:0")
    n = make_norm_inputs(cfg.N, cfg.H, device="cuda:0")
    res_out, normed, out = (torch.empty_like(n["x"]) for _ in range(3))
    p = moe.problem_from(normed, t["w_gate_up"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device="cuda:0")
    wgu, wd = moe.moe_pack_weights(t["w_gate_up"]), moe.moe_pack_weights(t["w_down"])

    def block():
        moe.moe_add_rmsnorm(n["x"], n["residual"], n["weight"], 1e-6, residual_out=res_out, normed=normed)
        moe.moe_forward(normed, t["router_w"], wgu, wd, cfg.top_k, cfg.norm_topk_prob,
                        out=out, workspace=ws, weight_layout=moe.MOE_LAYOUT_BLOCKED)

    eager, per_e = timed_steps(block, steps, warmup, torch)
    block()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block()
    replay, per_g = timed_steps(graph.replay, steps, warmup, torch)
    del graph
    return {"workload": "decode_block: residual add + RMSNorm + the 64-token decode MoE layer",
            "steps": steps, "tokens_per_s": round(cfg.N / (replay * 1e-3), 1), "ms_per_step_graph": round(replay, 4),
            "step_event_ms_graph": event_summary(per_g), "ms_per_step_eager": round(eager, 4),
            "step_event_ms_eager": event_summary(per_e)}


GEMM_SOURCES = ("sparse_moe_ffn_amd/csrc/grouped_gemm.hip", "sparse_moe_ffn_amd/csrc/moe_common.h",
                "sparse_moe_ffn_amd/csrc/moe_launch.h")


def gemm_source_hash():
    """Hash of the GEMM sources with comments and blank space removed, so that
    an edit of a comment keeps the committed counters valid and any change of
    code voids them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary (profiles/traffic_gate_up_<workload>.txt), or None when there is
    none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != gemm_source_hash():
        return None
    return int(kv["traffic_bytes_per_launch"])


def roofline_for(res):
    """Roofline of the dominant kernel (gate/up).  Its bound is the roof that
    gives the longer lower bound on its time: algorithmic bytes at the HBM
    peak, or algorithmic flops at the dense bf16 MFMA peak.  Both fractions
    are reported; `frac` is the one of the binding roof."""
    cfg = res["cfg"]
    kern = "gate_up"
    dur_s = res["stage_ms"][kern] * 1e-3
    w = res["work"][kern]
    gbs = w["bytes"] / dur_s / 1e9
    tfs = w["flops"] / dur_s / 1e12
    tiles = "16-row passes over the top-k ids" if res["ids_path"] else f"block_m {res['block_m']}"
    common = {"kernel": f"grouped_gemm_bf16 gate_up (SwiGLU epilogue), {tiles}, blocked weights",
              "traffic": measured_traffic(cfg.name), "avg_launch_ms": round(res["stage_ms"][kern], 4),
              "algorithmic_bytes_per_launch": w["bytes"], "algorithmic_flops_per_launch": w["flops"],
              "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
              "mfma_frac_of_measured_peak": of_measured(tfs)}
    if w["bytes"] / (HBM_PEAK_GBS * 1e9) >= w["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12):
        return {**common, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return {**common, "bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(res, budget_s, torch):
    """The CPU oracle as it is (its per-token definition, numpy float64 expert
    math) on the main workload, run on the host cores: the routing of the
    whole batch, then the tokens split over one worker thread per core (at
    most 16, the host share of one GPU), each with one BLAS thread.  Whole
    passes over the batch until the budget is spent.  Then the same oracle on
    one thread over the first tokens of the batch for a third of the budget."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    from oracle import moe_oracle as O

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                                # no way to pin BLAS threads: one worker
        threadpool_limits = None
    cfg, t = res["cfg"], res["inputs"]
    h = {k: (v.float().cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    sh = None
    if cfg.I_shared:
        sh = {"w_gate_up": h["shared_w_gate_up"], "w_down": h["shared_w_down"], "gate": h["shared_gate"]}
    cores = len(os.sched_getaffinity(0))
    workers = min(cores, 16) if threadpool_limits else 1

    def forward(rows, routing):
        O.moe_forward(h["x"], h["router_w"], h["w_gate_up"], h["w_down"], cfg.top_k, cfg.norm_topk_prob,
                      shared=sh, rows=rows, routing=routing)

    def one_pass(pool):
        routing = O.route(h["x"], h["router_w"], cfg.top_k, cfg.norm_topk_prob)
        chunks = [list(range(i, cfg.N, workers)) for i in range(min(workers, cfg.N))]
        list(pool.map(lambda rows: forward(rows, routing), chunks))

    import contextlib
    limit = threadpool_limits(1) if threadpool_limits else contextlib.nullcontext()
    with limit, ThreadPoolExecutor(workers) as pool:
        t0 = time.perf_counter()
        passes = 0
        while passes == 0 or time.perf_counter() - t0 < budget_s:
            one_pass(pool)
            passes += 1
        el = time.perf_counter() - t0
        # single thread: routing of the whole batch, then tokens one by one
        t1 = time.perf_counter()
        routing = O.route(h["x"], h["router_w"], cfg.top_k, cfg.norm_topk_prob)
        n1 = 0
        while n1 < cfg.N and (n1 == 0 or time.perf_counter() - t1 < budget_s / 3):
            forward([n1], routing)
            n1 += 1
        el1 = time.perf_counter() - t1
    return {"value": round(passes * cfg.N / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "threads_used": workers, "cpu_model": _cpu_model(),
            "single_thread": {"value": round(n1 / el1, 3), "unit": "tokens/s", "tokens": n1, "seconds": round(el1, 2)},
            "sample": f"{passes} whole passes over the {cfg.N} tokens of the {cfg.name} layer in {el:.1f} s "
                      f"(routing of the batch, then the per-token definition in numpy float64, tokens split over "
                      f"{workers} threads with one BLAS thread each); single thread: the first {n1} tokens"}


def copy_calibration(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return n


def leg_summary(r):
    """The figures of one MoE workload for the `also` part of the line."""
    cfg = r["cfg"]
    out = {"workload": f"{cfg.name}: N={cfg.N} H={cfg.H} E={cfg.E} top-{cfg.top_k} I={cfg.I}"
                       + (f" shared I_s={cfg.I_shared}" if cfg.I_shared else "")
                       + f" norm_topk_prob={cfg.norm_topk_prob}",
           "steps": r["steps"], "tokens_per_s": round(r["tokens_per_s"], 1),
           "ms_per_step": round(r["ms_per_step"], 4), "step_event_ms": r["step_event_ms"],
           "ms_per_step_row_major": round(r["ms_per_step_row_major"], 4),
           "step_event_ms_row_major": r["step_event_ms_row_major"],
           "tflops": round(r["tflops"], 1), "mfma_frac": round(r["mfma_frac"], 4),
           "mfma_frac_median": round(r["mfma_frac_median"], 4),
           "mfma_frac_of_measured_peak": of_measured(r["tflops_median"]),
           "weight_hbm_frac": round(r["weight_hbm_frac"], 4),
           "stage_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
           "stage_median_ms": r["stage_median_ms"], "stage_roofline": stage_roofline(r), "roofline": roofline_for(r),
           "counts_min_max": r["counts_min_max"], "hit_experts": r["hit_experts"]}
    if cfg.skew:
        out["load"] = load_report(r["counts"], cfg)
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (the block has no multi-GPU path).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_moe_ffn_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    moe.load_library()
    prewarm(torch, moe)
    print("[bench] matrix-unit probe", file=sys.stderr, flush=True)
    measure_mfma_peak(torch, moe)
    print(f"[bench] workload {a.workload}: {a.warmup} warmup + {a.steps} timed steps", file=sys.stderr, flush=True)
    main_res = bench_workload(a.workload, a.steps, a.warmup, torch, moe)
    also = {}
    for w in [s for s in a.also.split(",") if s and s != a.workload]:
        print(f"[bench] workload {w}", file=sys.stderr, flush=True)
        if w.startswith("dense_"):
            also[w] = bench_dense(w, a.steps, a.warmup, torch, moe)
            torch.cuda.empty_cache()
            continue
        if w == "decode_block":
            also[w] = bench_decode_block(a.steps, a.warmup, torch, moe)
            torch.cuda.empty_cache()
            continue
        if w == "ep8_share":
            also[w] = bench_ep_share(a.steps, a.warmup, torch, moe)
            torch.cuda.empty_cache()
            continue
        r = bench_workload(w, a.steps, a.warmup, torch, moe)
        also[w] = leg_summary(r)
        del r
        torch.cuda.empty_cache()
    if a.copy_calibration:
        copy_calibration(torch)
    cpu = None
    if a.cpu_seconds > 0:
        print("[bench] cpu oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(main_res, a.cpu_seconds, torch)
    cfg = main_res["cfg"]
    line = {
        "metric": METRIC, "value": round(main_res["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(main_res["ms_per_step"], 5),
        "step_event_ms": main_res["step_event_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Qwen3-30B-A3B-shaped MoE layer", "tokens": cfg.N, "hidden": cfg.H,
                   "experts": cfg.E, "top_k": cfg.top_k, "inter": cfg.I, "shared_inter": cfg.I_shared,
                   "norm_topk_prob": cfg.norm_topk_prob, "seed": cfg.seed, "weight_layout": "blocked"},
        "ms_per_step_row_major": round(main_res["ms_per_step_row_major"], 5),
        "step_event_ms_row_major": main_res["step_event_ms_row_major"],
        "tflops": round(main_res["tflops"], 2), "mfma_frac": round(main_res["mfma_frac"], 4),
        "weight_hbm_frac": round(main_res["weight_hbm_frac"], 4),
        "stage_ms": {k: round(v, 4) for k, v in main_res["stage_ms"].items()},
        "stage_median_ms": main_res["stage_median_ms"],
        "stage_roofline": stage_roofline(main_res),
        "hit_experts": main_res["hit_experts"],
        "roofline": roofline_for(main_res), "cpu_baseline": cpu, "also": also,
        "mfma_peak_measured": dict(MEASURED_PEAK),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
