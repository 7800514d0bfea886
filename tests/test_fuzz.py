"""Property fuzz over small random shapes (hypothesis, derandomized so every
run draws the same examples).

CPU: the oracle's three formulations agree, and routing and grouping keep
their invariants (distinct ids, descending weights, sum of the kept weights
1 with renormalisation and below 1 without, a stable permutation whose
counts sum to N*k, padded tiles of one expert each).

GPU: the whole HIP path against the oracle on random shapes, including
N = 1, k = 1, k = E, experts that get no pairs, a shared expert, and row
counts that are not multiples of any tile height; and the dense SwiGLU
layer on random shapes in both weight layouts.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, example, given, settings
from hypothesis import strategies as st

from oracle import moe_oracle as O
from sparse_moe_ffn_amd.inputs import make_inputs, random_case

FUZZ = settings(derandomize=True, database=None, deadline=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _np(t):
    return None if t is None else t.float().numpy()


@st.composite
def tiny_shapes(draw):
    E = draw(st.integers(1, 7))
    return dict(N=draw(st.integers(1, 9)), H=draw(st.sampled_from([4, 8, 12])), E=E,
                k=draw(st.integers(1, E)), I=draw(st.integers(1, 6)), renorm=draw(st.booleans()),
                shared=draw(st.sampled_from([0, 3])), seed=draw(st.integers(0, 10_000)))


@FUZZ
@given(tiny_shapes())
def test_oracle_formulations_agree(s):
    cfg = random_case(s["N"], s["H"], s["E"], s["k"], s["I"], I_shared=s["shared"], dtype="f32",
                      norm_topk_prob=s["renorm"], seed=s["seed"])
    t = make_inputs(cfg, "cpu")
    h = {k: _np(v) for k, v in t.items() if not isinstance(v, (int, float))}
    sh = None
    if cfg.I_shared:
        sh = {"w_gate_up": h["shared_w_gate_up"], "w_down": h["shared_w_down"], "gate": h["shared_gate"]}
    args = (h["x"], h["router_w"], h["w_gate_up"], h["w_down"], cfg.top_k, cfg.norm_topk_prob)
    a, _ = O.moe_forward(*args, shared=sh)
    b, _, _ = O.moe_forward_grouped(*args, shared=sh)
    c = O.moe_forward_by_slot(*args, shared=sh)
    scale = max(1.0, float(np.abs(a).max()))
    assert np.abs(a - b).max() <= 1e-12 * scale
    assert np.abs(a - c).max() <= 1e-12 * scale


@FUZZ
@given(tiny_shapes(), st.sampled_from([1, 2, 3, 8]))
def test_routing_and_grouping_invariants(s, bm):
    cfg = random_case(s["N"], s["H"], s["E"], s["k"], s["I"], dtype="f32", norm_topk_prob=s["renorm"],
                      seed=s["seed"])
    t = make_inputs(cfg, "cpu")
    ids, w, probs, _ = O.route(_np(t["x"]), _np(t["router_w"]), cfg.top_k, cfg.norm_topk_prob)
    N, k, E = cfg.N, cfg.top_k, cfg.E
    assert ids.shape == (N, k) and w.shape == (N, k)
    assert ((ids >= 0) & (ids < E)).all()
    assert all(len(set(row)) == k for row in ids.tolist()), "an expert chosen twice for one token"
    assert (np.diff(w, axis=1) <= 0).all(), "weights not in descending order"
    sums = w.astype(np.float64).sum(axis=1)
    if cfg.norm_topk_prob:
        np.testing.assert_allclose(sums, 1.0, rtol=0, atol=1e-6)
    else:
        assert (sums <= 1.0 + 1e-6).all() and (sums >= k / E - 1e-6).all()
    flat_e, _, flat_tok = O.flatten_pairs(ids, w)
    order, counts, offsets = O.group_pairs(flat_e, E)
    assert counts.sum() == N * k and offsets[-1] == N * k
    assert sorted(order.tolist()) == list(range(N * k))
    for e in range(E):
        seg = order[offsets[e]:offsets[e + 1]]
        assert (flat_e[seg] == e).all() and (np.diff(seg) > 0).all(), "segment not stable"
    sp, te, tr, nt = O.pad_segments(order, counts, bm, N * k)
    sp = np.asarray(sp)
    assert len(sp) == nt * bm and len(te) == nt and sum(tr) == N * k
    for tt in range(nt):
        real = sp[tt * bm:(tt + 1) * bm]
        real = real[real < N * k]
        assert len(real) == tr[tt] and (flat_e[real] == te[tt]).all()


# ------------------------------------------------------------------- GPU

@st.composite
def gpu_shapes(draw):
    dtype = draw(st.sampled_from(["bf16", "bf16", "f32"]))
    E = draw(st.integers(1, 40))
    k = draw(st.integers(1, min(E, 8)))
    if dtype == "bf16":
        H = draw(st.sampled_from([64, 128, 192, 256]))
        I = draw(st.sampled_from([64, 128, 192]))
        Is = draw(st.sampled_from([0, 0, 64, 128]))
    else:
        H = draw(st.integers(1, 40))
        I = draw(st.integers(1, 24))
        Is = draw(st.sampled_from([0, 5]))
    N = draw(st.sampled_from([1, 2, 3, 17, 63, 64, 65, 300, 641]))
    return dict(N=N, H=H, E=E, k=k, I=I, Is=Is, dtype=dtype, renorm=draw(st.booleans()),
                seed=draw(st.integers(0, 10_000)))


@pytest.mark.gpu
@settings(FUZZ, max_examples=40)
@given(gpu_shapes())
def test_forward_fuzz(s):
    import torch

    import sparse_moe_ffn_amd as moe

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = random_case(s["N"], s["H"], s["E"], s["k"], s["I"], I_shared=s["Is"], dtype=s["dtype"],
                      norm_topk_prob=s["renorm"], seed=s["seed"])
    print(f"fuzz case {cfg.name} renorm={cfg.norm_topk_prob} seed={cfg.seed}", flush=True)
    t = make_inputs(cfg, "cuda:0")
    out = moe.moe_forward(t["x"], t["router_w"], t["w_gate_up"], t["w_down"], cfg.top_k, cfg.norm_topk_prob,
                          t["shared_w_gate_up"], t["shared_w_down"], t["shared_gate"])
    ids_gpu, w_gpu, _ = moe.moe_route(t["x"], t["router_w"], cfg.top_k, cfg.norm_topk_prob)
    torch.cuda.synchronize()
    h = {k: (v.float().cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    routing = O.route(h["x"], h["router_w"], cfg.top_k, cfg.norm_topk_prob)
    keep = routing[3] >= 1e-6
    ids_g = ids_gpu.cpu().numpy()
    assert (ids_g[keep] == routing[0][keep]).all(), "expert ids differ from the oracle"
    np.testing.assert_allclose(w_gpu.cpu().numpy()[keep], routing[1][keep], rtol=2e-5, atol=2e-6)
    sh = None
    if cfg.I_shared:
        sh = {"w_gate_up": h["shared_w_gate_up"], "w_down": h["shared_w_down"], "gate": h["shared_gate"]}
    ref, _ = O.moe_forward(h["x"], h["router_w"], h["w_gate_up"], h["w_down"], cfg.top_k, cfg.norm_topk_prob,
                           shared=sh, routing=routing)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    tol = O.tolerance(ref[keep], cfg.dtype)
    err = float(np.abs(got[keep] - ref[keep]).max()) if keep.any() else 0.0
    assert err <= tol, f"{cfg.name}: max|gpu-ref| = {err:.3e} > {tol:.3e}"


@st.composite
def dense_shapes(draw):
    H = draw(st.sampled_from([64, 128, 256]))
    I = 64 * draw(st.integers(1, 48))
    N = draw(st.sampled_from([1, 17, 100, 333, 700, 1500, 2100, 4100]))
    while N * H * I > 4e8 and N > 1:
        N //= 2
    return dict(N=N, H=H, I=I, seed=draw(st.integers(0, 10_000)), blocked=draw(st.booleans()))


@pytest.mark.gpu
@settings(FUZZ, max_examples=30)
@given(dense_shapes())
@example(dict(N=1500, H=64, I=6144, seed=1, blocked=True))       # 320-row tiles (256 would add a round)
@example(dict(N=4100, H=64, I=1280, seed=6, blocked=False))      # 256
@example(dict(N=2100, H=64, I=1024, seed=2, blocked=False))      # 128
@example(dict(N=700, H=128, I=1472, seed=3, blocked=True))       # 64, ragged column block
@example(dict(N=333, H=64, I=1024, seed=4, blocked=False))       # 32
@example(dict(N=17, H=256, I=64, seed=5, blocked=True))          # 16 (64-column gate/up, 32-column down)
def test_dense_mlp_fuzz(s):
    """The dense SwiGLU layer on random shapes in both weight layouts.  The
    row-tile height follows the batch and the intermediate width (16 to 320
    rows, the tallest that still fills the GPU); the explicit examples take
    each height once, with ragged last row tiles, and the draws add more."""
    import torch

    import sparse_moe_ffn_amd as moe
    from sparse_moe_ffn_amd.inputs import make_dense_inputs

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"dense fuzz case N={s['N']} H={s['H']} I={s['I']} seed={s['seed']} blocked={s['blocked']}", flush=True)
    t = make_dense_inputs(s["N"], s["H"], s["I"], seed=s["seed"], device="cuda:0")
    wgu, wd = t["w_gate_up"], t["w_down"]
    lay = moe.MOE_LAYOUT_ROW_MAJOR
    if s["blocked"]:
        wgu, wd, lay = moe.moe_pack_weights(wgu), moe.moe_pack_weights(wd), moe.MOE_LAYOUT_BLOCKED
    out = moe.moe_dense_mlp(t["x"], wgu, wd, weight_layout=lay)
    torch.cuda.synchronize()
    ref = O.dense_mlp(_np(t["x"].cpu()), _np(t["w_gate_up"].cpu()), _np(t["w_down"].cpu()))
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    tol = O.tolerance(ref, "bf16")
    err = float(np.abs(got - ref).max())
    assert err <= tol, f"dense N{s['N']} H{s['H']} I{s['I']}: max|gpu-ref| = {err:.3e} > {tol:.3e}"
