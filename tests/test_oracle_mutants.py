"""Planted mistakes in the CPU oracle, each of which some pin must catch.

Every case below replaces one oracle function, on the CPU, with a copy that
makes one plausible mistake (a dropped term, a wrong sign or index, a
transposed operand, a wrong sort, rounding in the wrong place), runs every
pin of ``test_oracle_pins.py`` against the mutated oracle, and requires at
least one of them to fail.  The pins themselves check the oracle against
the pages' worked examples, closed forms, library routines and brute force;
this file shows that those checks are tight enough to notice each mistake.
"""
import functools

import numpy as np
import pytest

import test_oracle_pins as P
from oracle import moe_oracle as O

F32, F64 = np.float32, np.float64


def _pins():
    """Every pin of the oracle, as (name, zero-argument callable)."""
    pins = [
        ("grouping_walkthrough", P.test_grouping_walkthrough),
        ("pad_segments_walkthrough", P.test_pad_segments_walkthrough),
        ("route_example_both_modes", P.test_route_example_both_modes),
        ("route_large_logits", P.test_route_large_logits),
        ("scalar_routing", P.test_scalar_routing),
        ("tie_break_lower_expert_id", P.test_tie_break_lower_expert_id),
        ("margin_definition", P.test_margin_definition),
        ("scalar_per_expert_table", P.test_scalar_per_expert_table),
        ("scalar_shared_expert", P.test_scalar_shared_expert),
        ("shared_gate_is_one_scalar_per_token", P.test_shared_gate_is_one_scalar_per_token),
        ("dense_special_case_matches_torch_swiglu", P.test_dense_special_case_matches_torch_swiglu),
        ("brute_force_dense_all_experts", P.test_brute_force_dense_all_experts),
        ("batch_invariance_bitwise", P.test_batch_invariance_bitwise),
        ("single_token_touches_k_experts", P.test_single_token_touches_k_experts),
        ("shape_trace", P.test_shape_trace),
        ("dense_mlp_matches_page_expert_table", P.test_dense_mlp_matches_page_expert_table),
        ("dense_mlp_matches_torch_and_one_expert_block", P.test_dense_mlp_matches_torch_and_one_expert_block),
        ("round_to_bf16_nearest_even", P.test_round_to_bf16_nearest_even),
        ("rms_norm_closed_forms", P.test_rms_norm_closed_forms),
        ("add_rmsnorm_residual_semantics", P.test_add_rmsnorm_residual_semantics),
    ]
    pins += [(f"group_invariants[{s}]", functools.partial(P.test_group_invariants_and_stable_sort, s))
             for s in range(6)]
    pins += [(f"pad_segments_invariants[{b}]", functools.partial(P.test_pad_segments_invariants, b))
             for b in (1, 3, 16)]
    pins += [(f"renorm_is_softmax_of_topk_logits[{s}]", functools.partial(P.test_renorm_is_softmax_of_topk_logits, s))
             for s in range(5)]
    pins += [(f"weight_sum_invariants[{s}]", functools.partial(P.test_weight_sum_invariants, s)) for s in range(5)]
    pins += [(f"topk_brute_force[{s}]", functools.partial(P.test_topk_brute_force, s)) for s in range(8)]
    pins += [(f"scalar_block_end_to_end[{f}]", functools.partial(P.test_scalar_block_end_to_end, f))
             for f in ("definition", "grouped", "by_slot")]
    pins += [(f"rms_norm_matches_torch[{e}]", functools.partial(P.test_rms_norm_matches_torch, e))
             for e in (1e-6, 1e-2, 0.5)]
    return pins


def _failing_pins():
    failed = []
    for name, fn in _pins():
        try:
            fn()
        except Exception:            # an assertion, or the mutant's own error (a shape mismatch, a NaN check)
            failed.append(name)
    return failed


# ------------------------------------------------------------------ mutants
# Each takes pytest's monkeypatch and plants one mistake in the oracle module.

def _softmax_without_max(mp):
    def softmax_f32(logits):
        l = np.asarray(logits, dtype=F32)
        z = np.exp(l).astype(F32)                                   # dropped: "- max"
        s = np.add.accumulate(z, axis=-1, dtype=F32)[..., -1:]
        return (z / s).astype(F32)
    mp.setattr(O, "softmax_f32", softmax_f32)


def _topk_before_softmax(mp):
    orig = O.softmax_f32

    def route(x, router_w, top_k, norm_topk_prob):
        logits = O.router_logits(x, router_w)
        ids, sel = O.topk_desc(logits, top_k)                       # top-k of the logits first
        w = orig(sel)
        return ids, w, orig(logits), O.topk_margin(orig(logits), top_k)
    mp.setattr(O, "route", route)


def _route_with(mp, renorm_sum):
    """A copy of route whose renormalising sum is replaced by `renorm_sum(w)`."""
    def route(x, router_w, top_k, norm_topk_prob):
        logits = O.router_logits(x, router_w)
        probs = O.softmax_f32(logits)
        ids, w = O.topk_desc(probs, top_k)
        if norm_topk_prob:
            w = (w / renorm_sum(w, probs)).astype(F32)
        return ids, w.astype(F32), probs, O.topk_margin(probs, top_k)
    mp.setattr(O, "route", route)


def _renorm_drops_last_slot(mp):
    _route_with(mp, lambda w, p: w[:, :-1].sum(axis=1, keepdims=True) + (w[:, -1:] if w.shape[1] == 1 else 0))


def _renorm_over_all_experts(mp):
    _route_with(mp, lambda w, p: p.sum(axis=1, keepdims=True))


def _ties_to_higher_id(mp):
    def topk_desc(values, k):
        v = np.asarray(values, dtype=F32)
        E = v.shape[-1]
        rev = np.argsort(-v[..., ::-1], axis=-1, kind="stable")[..., :k]
        ids = (E - 1 - rev).astype(np.int64)
        return ids, np.take_along_axis(v, ids, axis=-1)
    mp.setattr(O, "topk_desc", topk_desc)


def _margin_without_kth_gap(mp):
    def topk_margin(probs, k):
        p = np.asarray(probs, dtype=F64)
        s = -np.sort(-p, axis=-1)
        last = min(k, p.shape[-1])                                  # ranks 0..k-1 only
        if last < 2:
            return np.full(p.shape[:-1], np.inf) if p.ndim > 1 else np.inf
        gaps = np.min(s[..., : last - 1] - s[..., 1:last], axis=-1)
        return gaps if p.ndim > 1 else float(gaps)
    mp.setattr(O, "topk_margin", topk_margin)


def _logits_rounded_to_bf16(mp):
    orig = O.router_logits
    mp.setattr(O, "router_logits", lambda x, r: O.round_to(orig(x, r), "bf16"))


def _repeat_instead_of_interleave(mp):
    def flatten_pairs(ids, weights):
        ids = np.asarray(ids)
        N, k = ids.shape
        return (ids.reshape(-1).astype(np.int64), np.asarray(weights).reshape(-1),
                np.tile(np.arange(N, dtype=np.int64), k))
    mp.setattr(O, "flatten_pairs", flatten_pairs)


def _unstable_order(mp):
    def group_pairs(flat_e, E):
        flat_e = np.asarray(flat_e, dtype=np.int64)
        order = np.lexsort((-np.arange(flat_e.size), flat_e)).astype(np.int64)   # descending p inside a segment
        counts = np.bincount(flat_e, minlength=E).astype(np.int64)
        offsets = np.zeros(E + 1, dtype=np.int64)
        offsets[1:] = np.cumsum(counts)
        return order, counts, offsets
    mp.setattr(O, "group_pairs", group_pairs)


def _offsets_inclusive(mp):
    orig = O.group_pairs

    def group_pairs(flat_e, E):
        order, counts, offsets = orig(flat_e, E)
        off = offsets.copy()
        off[:-1] = offsets[1:]                                      # inclusive instead of exclusive scan
        return order, counts, off
    mp.setattr(O, "group_pairs", group_pairs)


def _padding_sentinel_zero(mp):
    orig = O.pad_segments
    mp.setattr(O, "pad_segments", lambda order, counts, bm, sentinel: orig(order, counts, bm, 0))


def _silu_wrong_sign(mp):
    mp.setattr(O, "silu", lambda z: np.asarray(z, dtype=F64) / (1.0 + np.exp(np.asarray(z, dtype=F64))))


def _gate_up_rows_swapped(mp):
    orig = O.swiglu
    mp.setattr(O, "swiglu", lambda h, wg, wu, wd: orig(h, wu, wg, wd))


def _down_not_transposed(mp):
    def swiglu(h, w_gate, w_up, w_down):
        h = np.asarray(h, dtype=F64)
        g = h @ np.asarray(w_gate, dtype=F64).T
        u = h @ np.asarray(w_up, dtype=F64).T
        return (O.silu(g) * u) @ np.asarray(w_down, dtype=F64)     # missing .T
    mp.setattr(O, "swiglu", swiglu)


def _assignment_instead_of_add(mp):
    class _Add:
        @staticmethod
        def at(a, idx, vals):
            a[idx] = vals                                           # repeats overwrite

        def __call__(self, *a, **k):
            return np.add(*a, **k)

        def __getattr__(self, name):
            return getattr(np.add, name)

    class _NP:
        add = _Add()

        def __getattr__(self, name):
            return getattr(np, name)

    mp.setattr(O, "np", _NP())


def _shared_gate_sign(mp):
    def shared_term(x_row, shared):
        gu = np.asarray(shared["w_gate_up"], dtype=F64)
        Is = gu.shape[0] // 2
        gate = float(O.sigmoid(-np.dot(np.asarray(x_row, dtype=F64),
                                       np.asarray(shared["gate"], dtype=F64).reshape(-1))))
        return gate * O.swiglu(x_row, gu[:Is], gu[Is:], shared["w_down"])
    mp.setattr(O, "shared_term", shared_term)


def _shared_gate_per_element(mp):
    def shared_term(x_row, shared):
        gu = np.asarray(shared["w_gate_up"], dtype=F64)
        Is = gu.shape[0] // 2
        gate = O.sigmoid(np.asarray(x_row, dtype=F64) * np.asarray(shared["gate"], dtype=F64).reshape(-1))
        return gate * O.swiglu(x_row, gu[:Is], gu[Is:], shared["w_down"])   # a vector gate
    mp.setattr(O, "shared_term", shared_term)


def _rms_sum_not_mean(mp):
    def rms_norm(h, weight, eps):
        h = np.asarray(h, dtype=F64)
        ms = np.sum(h * h, axis=-1, keepdims=True)                 # sum instead of mean
        return h / np.sqrt(ms + eps) * np.asarray(weight, dtype=F64)
    mp.setattr(O, "rms_norm", rms_norm)


def _eps_outside_sqrt(mp):
    def rms_norm(h, weight, eps):
        h = np.asarray(h, dtype=F64)
        ms = np.mean(h * h, axis=-1, keepdims=True)
        return h / (np.sqrt(ms) + eps) * np.asarray(weight, dtype=F64)
    mp.setattr(O, "rms_norm", rms_norm)


def _residual_not_rounded(mp):
    def add_rmsnorm(x, residual, weight, eps, dtype):
        h = np.asarray(x, dtype=F32)
        if residual is not None:
            h = (h + np.asarray(residual, dtype=F32)).astype(F32)
        return O.rms_norm(h, weight, eps), h                        # stored residual left unrounded
    mp.setattr(O, "add_rmsnorm", add_rmsnorm)


def _norm_before_add(mp):
    def add_rmsnorm(x, residual, weight, eps, dtype):
        h = O.rms_norm(x, np.ones(np.asarray(x).shape[-1]), eps).astype(F32)   # normalised before the add
        if residual is not None:
            h = (h + np.asarray(residual, dtype=F32)).astype(F32)
        r = O.round_to(h, dtype)
        return O.rms_norm(r, weight, eps), r
    mp.setattr(O, "add_rmsnorm", add_rmsnorm)


def _round_half_up(mp):
    def round_to(a, dtype):
        a = np.asarray(a, dtype=F32)
        if dtype == "f32":
            return a
        bits = a.view(np.uint32).astype(np.uint64)
        bits = ((bits + 0x8000) & 0xFFFF0000).astype(np.uint32)   # ties away from zero, not to even
        return bits.view(F32)
    mp.setattr(O, "round_to", round_to)


MUTANTS = {
    "softmax without the max subtraction": _softmax_without_max,
    "top-k before softmax": _topk_before_softmax,
    "renorm sum drops the last slot": _renorm_drops_last_slot,
    "renorm over all experts": _renorm_over_all_experts,
    "ties to the higher expert id": _ties_to_higher_id,
    "margin without the k-th gap": _margin_without_kth_gap,
    "logits rounded to bf16": _logits_rounded_to_bf16,
    "repeat instead of repeat_interleave": _repeat_instead_of_interleave,
    "unstable order inside a segment": _unstable_order,
    "inclusive segment offsets": _offsets_inclusive,
    "padding sentinel 0": _padding_sentinel_zero,
    "SiLU with the wrong sign": _silu_wrong_sign,
    "gate and up rows swapped": _gate_up_rows_swapped,
    "down weight not transposed": _down_not_transposed,
    "assignment instead of index-add": _assignment_instead_of_add,
    "shared gate with the wrong sign": _shared_gate_sign,
    "shared gate per element": _shared_gate_per_element,
    "RMS with a sum instead of a mean": _rms_sum_not_mean,
    "eps outside the square root": _eps_outside_sqrt,
    "residual not rounded to the activation dtype": _residual_not_rounded,
    "norm before the residual add": _norm_before_add,
    "bf16 rounding ties away from zero": _round_half_up,
}


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    failed = _failing_pins()
    print(f"{name}: caught by {failed}")
    assert failed, f"no pin catches the planted mistake: {name}"
