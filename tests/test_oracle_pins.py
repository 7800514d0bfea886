"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
library special cases and brute force.  Each mutation test plants a known
mistake in the oracle (on the CPU) and checks that some pin catches it."""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rnd(a, d):
    """Values rounded to the d decimals the pages print (in float64)."""
    return np.round(np.asarray(a, dtype=np.float64), d).tolist()


def scalar_weights(g):
    """Pack the scalar example into [E, 2I, H] / [E, H, I] (gate rows first)."""
    E = g["E"]
    w_gate_up = np.array([[[g["w_gate"][e]], [g["w_up"][e]]] for e in range(E)], dtype=np.float32)
    w_down = np.array([[[g["w_down"][e]]] for e in range(E)], dtype=np.float32)
    return np.array(g["router_w"], np.float32), w_gate_up, w_down


def rand_case(rng, N, H, E, k, I, Is=0, std=0.5):
    x = rng.standard_normal((N, H)).astype(np.float32)
    r = (rng.standard_normal((E, H)) * std).astype(np.float32)
    gu = (rng.standard_normal((E, 2 * I, H)) * std).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) * std).astype(np.float32)
    shared = None
    if Is:
        shared = {"w_gate_up": (rng.standard_normal((2 * Is, H)) * std).astype(np.float32),
                  "w_down": (rng.standard_normal((H, Is)) * std).astype(np.float32),
                  "gate": (rng.standard_normal((H,)) * std).astype(np.float32)}
    return x, r, gu, wd, shared


# ----------------------------------------------------------------- grouping

def test_grouping_walkthrough():
    g = golden("m03_grouping_walkthrough.json")
    ids = np.array(g["ids"])
    flat_e, _, flat_tok = O.flatten_pairs(ids, np.ones_like(ids, dtype=np.float32))
    assert flat_e.tolist() == g["flat_e"]
    assert flat_tok.tolist() == g["flat_tok"]
    order, counts, offsets = O.group_pairs(flat_e, g["E"])
    assert order.tolist() == g["order"]
    assert counts.tolist() == g["counts"]
    for e in range(g["E"]):
        seg = order[offsets[e]:offsets[e + 1]]
        assert seg.tolist() == g["segments"][str(e)]
        assert flat_tok[seg].tolist() == g["segment_tokens"][str(e)]


def test_grouping_pin_catches_repeat_mistake(monkeypatch):
    g = golden("m03_grouping_walkthrough.json")
    ids = np.array(g["ids"])

    def wrong_flatten(ids, weights):
        N, k = np.asarray(ids).shape
        return ids.reshape(-1), np.asarray(weights).reshape(-1), np.tile(np.arange(N), k)

    monkeypatch.setattr(O, "flatten_pairs", wrong_flatten)
    _, _, flat_tok = O.flatten_pairs(ids, np.ones_like(ids, dtype=np.float32))
    assert flat_tok.tolist() == g["flat_tok_wrong_repeat"]
    assert flat_tok.tolist() != g["flat_tok"]


@pytest.mark.parametrize("seed", range(6))
def test_group_invariants_and_stable_sort(seed):
    rng = np.random.default_rng(seed)
    N, k, E = int(rng.integers(1, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    k = min(k, E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(N)])
    flat_e, _, flat_tok = O.flatten_pairs(ids, np.zeros(ids.shape, np.float32))
    order, counts, offsets = O.group_pairs(flat_e, E)
    P = N * k
    assert sorted(order.tolist()) == list(range(P))                      # a permutation
    assert counts.sum() == P and offsets[-1] == P
    assert order.tolist() == sorted(range(P), key=lambda p: flat_e[p])  # Python's stable sort
    se = flat_e[order]
    assert np.all(np.diff(se) >= 0)
    for e in range(E):
        seg = order[offsets[e]:offsets[e + 1]]
        assert np.all(flat_e[seg] == e) and np.all(np.diff(seg) > 0)
        assert len(set(flat_tok[seg].tolist())) == len(seg)                # a token hits e once


def test_pad_segments_walkthrough():
    g = golden("m03_grouping_walkthrough.json")
    S = g["N"] * g["k"]
    sp, te, tr, nt = O.pad_segments(np.array(g["order"]), np.array(g["counts"]), 2, S)
    assert sp.tolist() == [1, S, 2, S, 0, 3, 4, S, 5, S]
    assert te.tolist() == [0, 1, 2, 2, 3]
    assert tr.tolist() == [1, 1, 2, 1, 1]
    assert nt == 5


@pytest.mark.parametrize("bm", [1, 3, 16])
def test_pad_segments_invariants(bm):
    rng = np.random.default_rng(bm)
    N, k, E = 37, 3, 10
    ids = np.stack([rng.permutation(E)[:k] for _ in range(N)])
    flat_e, _, _ = O.flatten_pairs(ids, np.zeros(ids.shape, np.float32))
    order, counts, _ = O.group_pairs(flat_e, E)
    S = N * k
    sp, te, tr, nt = O.pad_segments(order, counts, bm, S)
    assert sp.size == nt * bm
    assert nt == sum(-(-int(c) // bm) for c in counts)
    assert [p for p in sp.tolist() if p != S] == order.tolist()
    for t in range(nt):
        rows = sp[t * bm:(t + 1) * bm]
        real = rows[rows != S]
        assert real.size == tr[t] and np.all(flat_e[real] == te[t])
        assert np.all(rows[:tr[t]] != S) and np.all(rows[tr[t]:] == S)


# ------------------------------------------------------------------ routing

def test_route_example_both_modes():
    g = golden("m03_route_example.json")
    x = np.array(g["x"], np.float32)
    eye = np.eye(g["E"], g["H"], dtype=np.float32)
    d = g["decimals"]
    for renorm, key in ((True, "weights_renorm"), (False, "weights_no_renorm")):
        ids, w, probs, _ = O.route(x, eye, g["top_k"], renorm)
        assert rnd(probs, d) == g["probs"]
        assert ids.tolist() == g["ids"]
        assert rnd(w, d) == g[key]
    _, w, _, _ = O.route(x, eye, g["top_k"], False)
    assert round(float(w[0].astype(np.float64).sum()), d) == g["weight_sum_no_renorm_token0"]


def test_route_large_logits():
    """Logits in the hundreds and thousands: the probabilities are still the
    softmax of the logits (scipy's, in float64), which depends only on the
    differences between logits, so exp never overflows; router = eye(4) makes
    the logits equal to x ([M03] 题面速览: float32 softmax over all E)."""
    x = np.array([[1000.0, 999.0, 990.0, 0.0], [-500.0, 300.0, 299.5, 120.0], [88.0, 89.0, 90.0, 91.0]],
                 np.float32)
    eye = np.eye(4, dtype=np.float32)
    ids, w, probs, _ = O.route(x, eye, 2, False)
    ref = scipy.special.softmax(x.astype(np.float64), axis=1)
    assert np.isfinite(probs).all()
    np.testing.assert_allclose(probs, ref, rtol=1e-6, atol=1e-12)
    assert ids.tolist() == [[0, 1], [1, 2], [3, 2]]
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, 1), rtol=1e-6)
    _, w_on, _, _ = O.route(x, eye, 2, True)
    sel = np.take_along_axis(x.astype(np.float64), ids, 1)
    np.testing.assert_allclose(w_on, scipy.special.softmax(sel, axis=1), rtol=1e-6)


def test_route_pin_catches_topk_before_softmax(monkeypatch):
    g = golden("m03_route_example.json")
    x = np.array(g["x"], np.float32)
    eye = np.eye(g["E"], g["H"], dtype=np.float32)

    def topk_first(x, router_w, top_k, norm_topk_prob):
        logits = O.router_logits(x, router_w)
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
        sel = np.take_along_axis(logits, ids, 1)
        w = scipy.special.softmax(sel, axis=1).astype(np.float32)
        return ids, w, None, None

    monkeypatch.setattr(O, "route", topk_first)
    _, w, _, _ = O.route(x, eye, g["top_k"], False)
    assert rnd(w, g["decimals"]) != g["weights_no_renorm"]


def test_scalar_routing():
    g = golden("m03_scalar_block.json")
    r, _, _ = scalar_weights(g)
    x = np.array(g["x"], np.float32)
    assert O.router_logits(x, r).tolist() == g["logits"]
    ids, w, _, _ = O.route(x, r, g["top_k"], True)
    assert ids.tolist() == g["ids"]
    assert rnd(w, g["decimals"]) == g["weights"]


@pytest.mark.parametrize("seed", range(5))
def test_renorm_is_softmax_of_topk_logits(seed):
    rng = np.random.default_rng(100 + seed)
    x, r, _, _, _ = rand_case(rng, 12, 16, 9, 3, 4)
    ids, w, _, _ = O.route(x, r, 3, True)
    logits = O.router_logits(x, r)
    sel = np.take_along_axis(logits.astype(np.float64), ids, 1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("seed", range(5))
def test_weight_sum_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    E, k = 7, 3
    x, r, _, _, _ = rand_case(rng, 20, 8, E, k, 4)
    _, w_on, _, _ = O.route(x, r, k, True)
    np.testing.assert_allclose(w_on.sum(1), 1.0, atol=1e-6)
    _, w_off, probs, _ = O.route(x, r, k, False)
    s = w_off.sum(1)
    assert np.all(s < 1.0) and np.all(s >= k / E - 1e-6)
    assert np.all(np.diff(w_off, axis=1) <= 0)                            # descending slots
    np.testing.assert_allclose(probs.sum(1), 1.0, atol=1e-6)


def test_tie_break_lower_expert_id():
    x = np.random.default_rng(3).standard_normal((5, 6)).astype(np.float32)
    r = np.tile(np.random.default_rng(4).standard_normal((1, 6)).astype(np.float32), (8, 1))
    ids, w, _, margin = O.route(x, r, 3, False)
    assert ids.tolist() == [[0, 1, 2]] * 5
    np.testing.assert_allclose(w, 1.0 / 8, rtol=1e-6)
    assert np.all(margin == 0.0)


@pytest.mark.parametrize("seed", range(8))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    E = int(rng.integers(1, 8))
    k = int(rng.integers(1, E + 1))
    v = rng.standard_normal(E).astype(np.float32)
    if seed % 2:
        v[rng.integers(0, E)] = v[0]                                      # force a tie
    ids, vals = O.topk_desc(v, k)
    # brute force: the kept set has the largest sum; order by (-value, id)
    best = max(itertools.combinations(range(E), k), key=lambda c: (sum(float(v[i]) for i in c), [-i for i in c]))
    assert sorted(ids.tolist()) == sorted(best) or np.isclose(sum(v[list(best)]), vals.sum())
    assert ids.tolist() == sorted(range(E), key=lambda e: (-float(v[e]), e))[:k]


def test_margin_definition():
    p = np.array([0.4, 0.3, 0.2, 0.1], np.float32)
    assert np.isclose(O.topk_margin(p, 2), 0.1)
    assert np.isclose(O.topk_margin(np.array([0.5, 0.2, 0.2, 0.1], np.float32), 1), 0.3)
    assert O.topk_margin(np.array([0.5, 0.2, 0.2, 0.1], np.float32), 2) == 0.0
    assert O.topk_margin(np.array([1.0], np.float32), 1) == float("inf")


# ------------------------------------------------------------- expert math

def test_scalar_per_expert_table():
    g = golden("m03_scalar_block.json")
    _, gu, wd = scalar_weights(g)
    d = g["decimals"]
    for key, xv in (("x=2", 2.0), ("x=-1", -1.0)):
        ys = [float(O.swiglu(np.array([xv]), gu[e, :1], gu[e, 1:], wd[e])[0]) for e in range(g["E"])]
        assert rnd(ys, d) == g["per_expert_out"][key]


@pytest.mark.parametrize("form", ["definition", "grouped", "by_slot"])
def test_scalar_block_end_to_end(form):
    g = golden("m03_scalar_block.json")
    r, gu, wd = scalar_weights(g)
    x = np.array(g["x"], np.float32)
    if form == "definition":
        out, _ = O.moe_forward(x, r, gu, wd, g["top_k"], True)
    elif form == "grouped":
        out, _, _ = O.moe_forward_grouped(x, r, gu, wd, g["top_k"], True)
    else:
        out = O.moe_forward_by_slot(x, r, gu, wd, g["top_k"], True)
    assert rnd(out, g["decimals"]) == g["out"]


def test_scalar_block_pin_catches_assignment(monkeypatch):
    g = golden("m03_scalar_block.json")
    r, gu, wd = scalar_weights(g)
    x = np.array(g["x"], np.float32)

    def assign_instead_of_add(a, idx, vals):
        a[idx] = vals                                                      # the planted mistake

    # np.add.at is a C ufunc method and cannot be patched; plant the mistake
    # through the module-level numpy reference the oracle uses instead.
    class _NP:
        def __getattr__(self, name):
            return getattr(np, name)

    class _Add:
        at = staticmethod(assign_instead_of_add)

        def __call__(self, *a, **k):
            return np.add(*a, **k)

        def __getattr__(self, name):
            return getattr(np.add, name)

    fake = _NP()
    fake.add = _Add()
    monkeypatch.setattr(O, "np", fake)
    out, _, _ = O.moe_forward_grouped(x, r, gu, wd, g["top_k"], True)
    assert round(float(out[0, 0]), g["decimals"]) == g["out_token0_if_assigned"]
    assert rnd(out, g["decimals"]) != g["out"]


def test_scalar_shared_expert():
    g = golden("m03_scalar_block.json")
    r, gu, wd = scalar_weights(g)
    x = np.array(g["x"], np.float32)
    s = g["shared"]
    shared = {"w_gate_up": np.array(s["gate_proj"] + s["up_proj"], np.float32),
              "w_down": np.array(s["down_proj"], np.float32),
              "gate": np.array(s["gate"], np.float32).reshape(-1)}
    d = g["decimals"]
    assert float(O.sigmoid(0.0)) == s["gate_value"]
    se = [float(O.swiglu(x[n], shared["w_gate_up"][:1], shared["w_gate_up"][1:], shared["w_down"])[0])
          for n in range(2)]
    assert rnd(se, d) == s["shared_expert_out"]
    for form in ("definition", "grouped", "by_slot"):
        if form == "definition":
            out, _ = O.moe_forward(x, r, gu, wd, g["top_k"], True, shared=shared)
        elif form == "grouped":
            out, _, _ = O.moe_forward_grouped(x, r, gu, wd, g["top_k"], True, shared=shared)
        else:
            out = O.moe_forward_by_slot(x, r, gu, wd, g["top_k"], True, shared=shared)
        assert rnd(out, d) == s["out_with_shared"]


def test_shared_gate_is_one_scalar_per_token():
    rng = np.random.default_rng(7)
    x, r, gu, wd, shared = rand_case(rng, 6, 8, 5, 2, 4, Is=3)
    out_s, _ = O.moe_forward(x, r, gu, wd, 2, True, shared=shared)
    out_0, _ = O.moe_forward(x, r, gu, wd, 2, True, shared=None)
    gus = shared["w_gate_up"]
    for n in range(6):
        sh = O.swiglu(x[n], gus[:3], gus[3:], shared["w_down"])
        ratio = (out_s[n] - out_0[n]) / sh
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-9)
        np.testing.assert_allclose(ratio[0], 1 / (1 + np.exp(-float(np.dot(x[n].astype(np.float64), shared["gate"])))), rtol=1e-12)


def test_dense_special_case_matches_torch_swiglu():
    """E = k = 1 reduces the block to a dense SwiGLU MLP with weight 1."""
    rng = np.random.default_rng(11)
    x, r, gu, wd, _ = rand_case(rng, 9, 12, 1, 1, 20)
    for renorm in (True, False):
        out, (ids, w, _, _) = O.moe_forward(x, r, gu, wd, 1, renorm)
        assert np.all(ids == 0) and np.all(w == 1.0)
        xt = torch.from_numpy(x).double()
        gt = torch.from_numpy(gu[0]).double()
        ref = torch.nn.functional.linear(
            torch.nn.functional.silu(torch.nn.functional.linear(xt, gt[:20])) * torch.nn.functional.linear(xt, gt[20:]),
            torch.from_numpy(wd[0]).double())
        np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- whole block

@pytest.mark.parametrize("seed,shape", [(0, (7, 8, 6, 2, 5, 0)), (1, (11, 5, 4, 4, 3, 2)),
                                        (2, (4, 16, 9, 1, 7, 3)), (3, (13, 3, 3, 3, 2, 0))])
def test_three_formulations_agree(seed, shape):
    N, H, E, k, I, Is = shape
    rng = np.random.default_rng(400 + seed)
    x, r, gu, wd, shared = rand_case(rng, N, H, E, k, I, Is)
    for renorm in (True, False):
        a, _ = O.moe_forward(x, r, gu, wd, k, renorm, shared=shared)
        b, _, _ = O.moe_forward_grouped(x, r, gu, wd, k, renorm, shared=shared)
        c = O.moe_forward_by_slot(x, r, gu, wd, k, renorm, shared=shared)
        scale = np.abs(a).max()
        np.testing.assert_allclose(b, a, atol=1e-12 * scale)
        np.testing.assert_allclose(c, a, atol=1e-12 * scale)


def test_brute_force_dense_all_experts():
    """Every expert on every token, weighted by a dense [N, E] routing matrix
    that is zero outside the top-k, equals the block."""
    rng = np.random.default_rng(13)
    N, H, E, k, I = 6, 5, 5, 2, 3
    x, r, gu, wd, _ = rand_case(rng, N, H, E, k, I)
    out, (ids, w, _, _) = O.moe_forward(x, r, gu, wd, k, True)
    dense = np.zeros((N, E))
    for n in range(N):
        for j in range(k):
            dense[n, ids[n, j]] += w[n, j]
    allx = np.stack([O.swiglu(x, gu[e, :I], gu[e, I:], wd[e]) for e in range(E)], axis=1)  # [N,E,H]
    np.testing.assert_allclose(np.einsum("ne,neh->nh", dense, allx), out, rtol=1e-12, atol=1e-14)


def test_batch_invariance_bitwise():
    rng = np.random.default_rng(14)
    x, r, gu, wd, shared = rand_case(rng, 9, 8, 6, 2, 4, Is=3)
    full, _ = O.moe_forward(x, r, gu, wd, 2, True, shared=shared)
    for i in range(9):
        one, _ = O.moe_forward(x[i:i + 1], r, gu, wd, 2, True, shared=shared)
        assert np.array_equal(one[0], full[i])


def test_single_token_touches_k_experts():
    rng = np.random.default_rng(15)
    x, r, _, _, _ = rand_case(rng, 1, 8, 10, 4, 2)
    ids, w, _, _ = O.route(x, r, 4, True)
    flat_e, _, _ = O.flatten_pairs(ids, w)
    _, counts, _ = O.group_pairs(flat_e, 10)
    assert (counts > 0).sum() == 4 and counts.max() == 1


def test_shape_trace():
    g = golden("m03_shape_trace.json")
    N, H, E, I, k = g["N"], g["H"], g["E"], g["I"], g["top_k"]
    rng = np.random.default_rng(16)
    x, r, gu, wd, _ = rand_case(rng, N, H, E, k, I, Is=I)
    assert list(O.router_logits(x, r).shape) == g["logits"]
    ids, w, probs, _ = O.route(x, r, k, True)
    assert list(probs.shape) == g["probs"] and list(w.shape) == g["weights"] and list(ids.shape) == g["ids"]
    flat_e, flat_w, flat_tok = O.flatten_pairs(ids, w)
    assert [flat_e.size] == [flat_w.size] == [flat_tok.size] == g["flat"]
    order, counts, _ = O.group_pairs(flat_e, E)
    assert list(order.shape) == g["order"] and list(counts.shape) == g["counts"]
    assert counts.sum() == g["counts_sum"]
    out, _ = O.moe_forward(x, r, gu, wd, k, True)
    assert list(out.shape) == g["out"]


def test_tolerance_formula():
    ref = np.array([[0.5, -2.0]])
    assert O.tolerance(ref, "bf16") == pytest.approx(2e-2 * 2.0 + 1e-3)
    assert O.tolerance(ref, "f32") == pytest.approx(1e-4 * 2.0)


# ----------------------------------------------------- dense SwiGLU layer

def test_dense_mlp_matches_page_expert_table():
    """Each expert of the page's scalar example, run as a dense layer over the
    two tokens, gives the page's per-expert outputs."""
    g = golden("m03_scalar_block.json")
    _, gu, wd = scalar_weights(g)
    x = np.array([[2.0], [-1.0]])
    for e in range(g["E"]):
        y = O.dense_mlp(x, gu[e], wd[e])[:, 0]
        assert rnd(y, g["decimals"]) == [g["per_expert_out"]["x=2"][e], g["per_expert_out"]["x=-1"][e]]


def test_dense_mlp_matches_torch_and_one_expert_block():
    rng = np.random.default_rng(21)
    x, r, gu, wd, _ = rand_case(rng, 7, 16, 1, 1, 24)
    d = O.dense_mlp(x, gu[0], wd[0])
    xt, gt = torch.from_numpy(x).double(), torch.from_numpy(gu[0]).double()
    F = torch.nn.functional
    ref = F.linear(F.silu(F.linear(xt, gt[:24])) * F.linear(xt, gt[24:]), torch.from_numpy(wd[0]).double())
    np.testing.assert_allclose(d, ref.numpy(), rtol=1e-12, atol=1e-12)
    out, _ = O.moe_forward(x, r, gu, wd, 1, False)
    np.testing.assert_allclose(out, d, rtol=1e-12, atol=1e-12)


# --------------------------------------------------- residual add + RMSNorm

def test_round_to_bf16_nearest_even():
    # bf16 keeps 7 fraction bits: 1 + 2^-8 is halfway to 1 + 2^-7 and goes to
    # the even neighbour 1; 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and
    # 1 + 2^-6 (even).
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0], np.float32)
    np.testing.assert_array_equal(O.round_to(v, "bf16"), [1.0, 1 + 2.0 ** -6, -1.0, 3.0])
    np.testing.assert_array_equal(O.round_to(v, "f32"), v)


@pytest.mark.parametrize("eps", [1e-6, 1e-2, 0.5])
def test_rms_norm_matches_torch(eps):
    rng = np.random.default_rng(22)
    h = rng.standard_normal((6, 40)) * 3
    w = rng.standard_normal(40)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (40,), torch.from_numpy(w), eps)
    np.testing.assert_allclose(O.rms_norm(h, w, eps), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_rms_norm_closed_forms():
    H = 16
    ones = np.ones(H)
    for c in (2.0, -0.5, 1e-3):                  # constant row: c / sqrt(c^2 + eps)
        np.testing.assert_allclose(O.rms_norm(np.full(H, c), ones, 1e-6), c / np.sqrt(c * c + 1e-6), rtol=1e-14)
    rng = np.random.default_rng(23)
    h = rng.standard_normal((5, H))
    y = O.rms_norm(h, ones, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)     # unit RMS
    np.testing.assert_allclose(O.rms_norm(7.5 * h, ones, 0.0), y, rtol=1e-12)  # scale invariant
    np.testing.assert_allclose(O.rms_norm(h, 3 * ones, 0.0), 3 * y, rtol=1e-12)


def test_add_rmsnorm_residual_semantics():
    rng = np.random.default_rng(24)
    x = O.round_to(rng.standard_normal((4, 32)), "bf16")
    res = O.round_to(rng.standard_normal((4, 32)) * 4, "bf16")
    w = rng.standard_normal(32)
    # first layer: the input is the residual
    n0, r0 = O.add_rmsnorm(x, None, w, 1e-6, "bf16")
    np.testing.assert_array_equal(r0, x)
    # later layers: the residual carries the un-normalised float32 sum
    n1, r1 = O.add_rmsnorm(x, res, w, 1e-6, "bf16")
    s = torch.from_numpy(x) + torch.from_numpy(res)
    np.testing.assert_array_equal(r1, s.to(torch.bfloat16).float().numpy())
    for n, r in ((n0, r0), (n1, r1)):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(r).double(), (32,), torch.from_numpy(w), 1e-6)
        np.testing.assert_allclose(n, ref.numpy(), rtol=1e-12, atol=1e-12)
