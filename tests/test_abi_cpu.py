"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import sparse_moe_ffn_amd as moe
from sparse_moe_ffn_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_mi355x.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = moe.load_library()
    names = declared()
    assert "moe_forward" in names and "moe_route" in names and "moe_align" in names
    for n in names:
        assert hasattr(lib, n), n


def test_problem_validation_codes():
    P = moe.problem
    ok = P(4096, 2048, 128, 8, 768)
    assert moe.moe_workspace_size(ok) > 0
    for bad, code in ((P(4, 64, 4, 5, 64), B.MOE_EINVAL), (P(4, 64, 4, 0, 64), B.MOE_EINVAL),
                      (P(-1, 64, 4, 2, 64), B.MOE_EINVAL), (P(4, 100, 4, 2, 64), B.MOE_EUNSUPPORTED),
                      (P(4, 64, 4, 2, 96), B.MOE_EUNSUPPORTED), (P(4, 64, 600, 2, 64), B.MOE_EUNSUPPORTED),
                      (P(4, 64, 64, 33, 64), B.MOE_EUNSUPPORTED), (P(4, 64, 4, 2, 64, shared_inter=32), B.MOE_EUNSUPPORTED)):
        with pytest.raises(B.MoEError) as ei:
            moe.moe_workspace_size(bad)
        assert ei.value.code == code, (bad.top_k, ei.value)
    # fp32 takes any shape
    assert moe.moe_workspace_size(P(3, 1, 3, 2, 1, dtype=__import__("torch").float32)) > 0


def test_workspace_layout_is_ordered_and_aligned():
    for args in ((4096, 2048, 128, 8, 768), (64, 2048, 128, 8, 768), (8192, 2048, 128, 8, 768, 2048), (7, 64, 5, 3, 64)):
        L = moe.moe_get_workspace_layout(moe.problem(*args))
        offs = [L[k] for k in ("route_scratch", "topk_ids", "topk_w", "shared_scale", "counts", "offsets", "order", "sorted_pairs",
                               "tile_expert", "tile_rows", "num_tiles", "align_scratch", "act", "y", "shared_act",
                               "shared_y")]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert L["total_bytes"] >= offs[-1] and L["total_bytes"] % 256 == 0
        assert L["max_rows"] == L["max_tiles"] * L["block_m"]


def test_block_m_follows_rows_per_expert():
    """Grouped tiles: 16 rows below 2 pairs per expert, 32 up to 16, 64
    below 42, 128 below 124, else 320.  The ids products (most experts hit,
    under 9 pairs each, at most 1024 pairs) report their 16-row passes."""
    bm = lambda N, E=128: moe.moe_get_workspace_layout(moe.problem(N, 2048, E, 8, 768))["block_m"]
    Ns = (16, 64, 128, 136, 160, 256, 264, 384, 640, 720, 1024, 1900, 2048, 4096, 16384)
    assert tuple(bm(N) for N in Ns) == (16, 16, 16, 32, 32, 32, 64, 64, 64, 128, 128, 128, 320, 320, 320)
    assert (bm(90, 512), bm(129, 512)) == (16, 32)       # grouped at avg 1.4 and 2.02
    assert moe.moe_get_workspace_layout(moe.problem(1000, 256, 16, 8, 128, dtype=torch.float32))["block_m"] == 16


@pytest.mark.parametrize("pairs,E,bm", [(6, 5, 2), (512, 128, 16), (32768, 128, 128), (3, 10, 64), (0, 4, 16)])
def test_align_capacity_bounds_every_grouping(pairs, E, bm):
    rows, tiles = moe.moe_align_capacity(pairs, E, bm)
    assert rows == tiles * bm
    # the worst case: as many experts as possible with one pair past a tile boundary
    m = min(E, pairs)
    worst = 0
    if m:
        base, extra = divmod(pairs, m)
        worst = sum(-(-(base + (i < extra)) // bm) for i in range(m))
    assert tiles >= worst


def test_align_scratch_size():
    assert moe.moe_align_scratch_size(4096, 128) == 0
    assert moe.moe_align_scratch_size(4097, 128) == (2 * 128 + 128) * 4
    assert moe.moe_align_scratch_size(131072, 128) == (32 * 128 + 128) * 4


def test_forward_rejects_before_any_hip_call():
    lib = moe.load_library()
    p = moe.problem(16, 64, 4, 2, 64)
    fake = ctypes.c_void_p(1 << 20)
    rc = lib.moe_forward(ctypes.byref(p), fake, fake, fake, fake, None, None, None, fake, fake, 16, None)
    assert rc == B.MOE_ENOSPC and b"workspace" in lib.moe_last_error()
    rc = lib.moe_forward(ctypes.byref(p), None, fake, fake, fake, None, None, None, fake, fake, 1 << 30, None)
    assert rc == B.MOE_EINVAL
    rc = lib.moe_forward(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, fake, fake, 1 << 30, None)
    assert rc == B.MOE_EINVAL                               # shared weights without shared_inter
    rc = lib.moe_forward(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 2), fake, fake, fake, None, None, None,
                         fake, fake, 1 << 30, None)
    assert rc == B.MOE_EUNSUPPORTED                          # misaligned bf16
    rc = lib.moe_align(fake, 4, 2, 4, 0, fake, fake, fake, fake, fake, fake, fake, None, None)
    assert rc == B.MOE_EINVAL
    rc = lib.moe_align(fake, 5000, 2, 4, 16, fake, fake, fake, fake, fake, fake, fake, None, None)
    assert rc == B.MOE_EINVAL and b"scratch" in lib.moe_last_error()   # 10000 pairs need scratch
    rc = lib.moe_gate_up(ctypes.byref(p), fake, fake, fake, fake, fake, fake, 48, 4, fake, None)
    assert rc == B.MOE_EUNSUPPORTED                          # bf16 tile height must be 16/32/64/128
    # empty batch: valid, nothing to do
    p0 = moe.problem(0, 64, 4, 2, 64)
    assert lib.moe_forward(ctypes.byref(p0), None, None, None, None, None, None, None, None, None, 0, None) == 0


def test_dense_mlp_and_add_rmsnorm_reject_before_any_hip_call():
    lib = moe.load_library()
    fake = ctypes.c_void_p(1 << 20)
    p = moe.problem(16, 64, 1, 1, 96)                        # bf16 inter must be a multiple of 64
    assert lib.moe_dense_mlp(ctypes.byref(p), fake, fake, fake, fake, fake, None) == B.MOE_EUNSUPPORTED
    p = moe.problem(16, 64, 1, 1, 128)
    assert lib.moe_dense_mlp(ctypes.byref(p), fake, None, fake, fake, fake, None) == B.MOE_EINVAL
    assert lib.moe_dense_mlp(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 8), fake, fake, fake, fake,
                             None) == B.MOE_EUNSUPPORTED
    p0 = moe.problem(0, 64, 1, 1, 128)
    assert lib.moe_dense_mlp(ctypes.byref(p0), None, None, None, None, None, None) == 0
    f = lib.moe_add_rmsnorm
    other = ctypes.c_void_p(1 << 21)
    assert f(4, 60, B.MOE_BF16, fake, None, fake, fake, 1e-6, other, None) == B.MOE_EUNSUPPORTED   # H % 8
    assert f(4, 32768, B.MOE_BF16, fake, None, fake, fake, 1e-6, other, None) == B.MOE_EUNSUPPORTED
    assert f(4, 64, B.MOE_BF16, fake, None, fake, fake, 0.0, other, None) == B.MOE_EINVAL          # eps > 0
    assert f(4, 64, B.MOE_BF16, fake, None, fake, fake, float("nan"), other, None) == B.MOE_EINVAL
    assert f(4, 64, B.MOE_BF16, fake, None, fake, fake, 1e-6, fake, None) == B.MOE_EINVAL          # normed aliases
    assert f(4, 64, B.MOE_BF16, None, None, fake, fake, 1e-6, other, None) == B.MOE_EINVAL
    assert f(4, 64, 7, fake, None, fake, fake, 1e-6, other, None) == B.MOE_EUNSUPPORTED
    assert f(0, 64, B.MOE_BF16, None, None, None, None, 1e-6, None, None) == 0


def test_weight_layout_validation():
    import torch
    P = moe.problem
    assert moe.moe_workspace_size(P(64, 2048, 128, 8, 768, weight_layout=B.MOE_LAYOUT_BLOCKED)) > 0
    for bad, code in ((P(4, 64, 4, 2, 64, weight_layout=2), B.MOE_EINVAL),
                      (P(4, 64, 4, 2, 64, dtype=torch.float32, weight_layout=B.MOE_LAYOUT_BLOCKED),
                       B.MOE_EUNSUPPORTED)):
        with pytest.raises(B.MoEError) as ei:
            moe.moe_workspace_size(bad)
        assert ei.value.code == code
    p = P(4, 64, 4, 2, 64)
    p.reserved = 1
    with pytest.raises(B.MoEError) as ei:
        moe.moe_workspace_size(p)
    assert ei.value.code == B.MOE_EINVAL


def test_pack_weights_rejects_before_any_hip_call():
    lib = moe.load_library()
    buf = ctypes.create_string_buffer(1 << 16)
    a = ctypes.c_void_p((ctypes.addressof(buf) + 15) & ~15)
    b = ctypes.c_void_p(a.value + 8192)
    cases = [((1, 8, 64, B.MOE_F32, a, b), B.MOE_EUNSUPPORTED),      # fp32
             ((1, 12, 64, B.MOE_BF16, a, b), B.MOE_EUNSUPPORTED),    # rows % 8
             ((1, 8, 96, B.MOE_BF16, a, b), B.MOE_EUNSUPPORTED),     # cols % 64
             ((1, 8, 64, B.MOE_BF16, None, b), B.MOE_EINVAL),        # NULL
             ((2, 8, 64, B.MOE_BF16, a, ctypes.c_void_p(a.value + 1024)), B.MOE_EINVAL),   # overlap
             ((1, 8, 64, B.MOE_BF16, ctypes.c_void_p(a.value + 2), b), B.MOE_EUNSUPPORTED),  # alignment
             ((-1, 8, 64, B.MOE_BF16, a, b), B.MOE_EINVAL)]
    for args, code in cases:
        assert lib.moe_pack_weights(*args, None) == code, args
    assert lib.moe_pack_weights(0, 8, 64, B.MOE_BF16, None, None, None) == B.MOE_OK   # empty: nothing enqueued


def test_ids_products_reject_before_any_hip_call():
    """moe_gate_up_ids / moe_down_ids: bf16, 4 <= N*k <= 1024, N*k % 4 == 0,
    16-byte aligned ids; every rejection happens before a HIP call (no GPU here)."""
    import torch
    lib = moe.load_library()
    fake = ctypes.c_void_p(1 << 20)
    ok_p = moe.problem(64, 128, 16, 8, 64)
    for p, code in ((moe.problem(64, 128, 16, 8, 64, dtype=torch.float32), B.MOE_EUNSUPPORTED),
                    (moe.problem(129, 128, 16, 8, 64), B.MOE_EUNSUPPORTED),      # 1032 pairs
                    (moe.problem(3, 128, 16, 3, 64), B.MOE_EUNSUPPORTED),        # 9 pairs
                    (moe.problem(1, 128, 16, 2, 64), B.MOE_EUNSUPPORTED)):       # 2 pairs
        assert lib.moe_gate_up_ids(ctypes.byref(p), fake, fake, fake, fake, None) == code
        assert lib.moe_down_ids(ctypes.byref(p), fake, fake, fake, fake, fake, None) == code
    unaligned = ctypes.c_void_p((1 << 20) + 4)
    assert lib.moe_gate_up_ids(ctypes.byref(ok_p), fake, fake, unaligned, fake, None) == B.MOE_EUNSUPPORTED
    assert lib.moe_down_ids(ctypes.byref(ok_p), fake, fake, unaligned, fake, fake, None) == B.MOE_EUNSUPPORTED
    assert lib.moe_gate_up_ids(ctypes.byref(ok_p), fake, fake, None, fake, None) == B.MOE_EINVAL
    assert lib.moe_down_ids(ctypes.byref(ok_p), fake, fake, fake, None, fake, None) == B.MOE_EINVAL
    p0 = moe.problem(0, 128, 16, 8, 64)
    assert lib.moe_gate_up_ids(ctypes.byref(p0), None, None, None, None, None) == 0


def test_forward_schedule_choice():
    """moe_forward takes the ids products for bf16 batches with
    4 <= N*k <= 1024, N*k % 4 == 0, N*k >= 1.5 E (most experts hit) and
    N*k < 9 E (under 9 pairs per expert); otherwise the grouping."""
    import torch
    L = lambda *a, **kw: moe.moe_get_workspace_layout(moe.problem(*a, **kw))["ids_products"]
    assert [L(N, 2048, 128, 8, 768) for N in (1, 16, 23, 24, 64, 128, 129, 4096)] == [0, 0, 0, 1, 1, 1, 0, 0]
    assert L(64, 2048, 128, 8, 768, dtype=torch.float32) == 0
    assert L(5, 128, 4, 3, 64) == 0                     # 15 pairs: not a multiple of 4
    assert L(4, 128, 6, 2, 64) == 0                     # 8 pairs: 2 * 8 < 3 * 6
    assert L(6, 128, 6, 2, 64) == 1                     # 12 pairs: 2 * 12 >= 3 * 6
    assert L(100, 2048, 512, 8, 768) == 1               # 800 pairs over 512 experts
    assert L(120, 256, 64, 8, 64) == 0                  # 960 pairs: 15 per expert, grouped 32-row tiles


# ------------------------------------------------- binding shape checks (no GPU)
# Every binding checks each tensor's shape against the problem before it looks
# at devices or launches anything.  On the CPU, a call whose shapes are right
# stops at the device check ("must be on a GPU"); each wrong shape must stop
# earlier, naming the tensor.

import torch  # noqa: E402

_N, _H, _E, _K, _I, _IS = 6, 64, 4, 2, 128, 192


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _expect(fn, *names):
    """fn raises ValueError before the device check, naming one of `names`
    (a disagreement between two tensors may name either)."""
    with pytest.raises(ValueError) as ei:
        fn()
    msg = str(ei.value)
    assert any(n in msg for n in names) and "on a GPU" not in msg, msg


def _expect_device_error(fn):
    with pytest.raises(ValueError, match="must be on a GPU"):
        fn()


def _grouping(P, E=_E, bm=16):
    rows, tiles = moe.moe_align_capacity(P, E, bm)
    i = dict(dtype=torch.int32)
    return B.Grouping(_t(E, **i), _t(E + 1, **i), _t(P, **i), _t(rows, **i), _t(tiles, **i), _t(tiles, **i),
                      _t(1, **i), bm, rows, tiles, E, P)


def _forward_args():
    return dict(x=_t(_N, _H), router_w=_t(_E, _H), w_gate_up=_t(_E, 2 * _I, _H), w_down=_t(_E, _H, _I),
                top_k=_K, shared_w_gate_up=_t(2 * _IS, _H), shared_w_down=_t(_H, _IS), shared_gate=_t(_H),
                out=_t(_N, _H))


@pytest.mark.parametrize("name,bad", [
    ("x", _t(_N, _H + 64)), ("x", _t(_N * _H)), ("router_w", _t(_E + 1, _H)), ("w_gate_up", _t(_E, 2 * _I, _H + 64)),
    ("w_gate_up", _t(_E, 2 * _I + 1, _H)), ("w_down", _t(_E, _H, _I + 64)), ("w_down", _t(_E, _I, _H)),
    ("w_down", _t(_E + 1, _H, _I)), ("shared_w_gate_up", _t(2 * _IS, _H + 64)), ("shared_w_down", _t(_IS, _H)),
    ("shared_w_down", _t(_H, _IS + 64)), ("shared_gate", _t(_H + 1)), ("out", _t(_N + 1, _H))])
def test_forward_rejects_each_wrong_shape(name, bad):
    a = _forward_args()
    _expect_device_error(lambda: moe.moe_forward(**a))
    a[name] = bad
    _expect(lambda: moe.moe_forward(**a), name, "w_gate_up")


def test_forward_rejects_partial_shared_expert():
    a = _forward_args()
    a["shared_gate"] = None
    _expect(lambda: moe.moe_forward(**a), "shared")


def test_forward_rejects_short_workspace():
    a = _forward_args()
    p = moe.problem(_N, _H, _E, _K, _I, _IS)
    a["workspace"] = _t(moe.moe_workspace_size(p) - 1, dtype=torch.uint8)
    _expect(lambda: moe.moe_forward(**a), "workspace")


def test_route_rejects_wrong_shapes():
    i32, f32 = torch.int32, torch.float32
    ok = dict(x=_t(_N, _H), router_w=_t(_E, _H), top_k=_K, norm_topk_prob=True, shared_gate=_t(_H),
              topk_ids=_t(_N, _K, dtype=i32), topk_w=_t(_N, _K, dtype=f32), shared_scale=_t(_N, dtype=f32))
    _expect_device_error(lambda: moe.moe_route(**ok))
    for name, bad in (("router_w", _t(_E, _H + 64)), ("shared_gate", _t(_H - 1)), ("topk_ids", _t(_N, _K + 1, dtype=i32)),
                      ("topk_w", _t(_N + 1, _K, dtype=f32)), ("shared_scale", _t(_N + 1, dtype=f32)),
                      ("scratch", _t(1, dtype=f32))):
        a = dict(ok, **{name: bad})
        _expect(lambda: moe.moe_route(**a), name)


def test_align_rejects_wrong_shapes():
    _expect(lambda: moe.moe_align(_t(_N * _K, dtype=torch.int32), _E, 16), "topk_ids")
    big = 1200                                         # more than one 4096-pair chunk: needs scratch
    _expect(lambda: moe.moe_align(_t(big, 4, dtype=torch.int32), _E, 16, scratch=_t(1, dtype=torch.int32)),
            "scratch")


def test_gate_up_and_down_reject_wrong_shapes():
    g = _grouping(_N * _K)
    x, wgu, wd = _t(_N, _H), _t(_E, 2 * _I, _H), _t(_E, _H, _I)
    act, tw, y = _t(g.max_rows, _I), _t(_N, _K, dtype=torch.float32), _t(_N * _K, _H)
    _expect_device_error(lambda: moe.moe_gate_up(x, wgu, g, _K, act))
    _expect_device_error(lambda: moe.moe_down(act, wd, tw, g, _N, _K, y))
    _expect(lambda: moe.moe_gate_up(_t(_N, _H + 64), wgu, g, _K, act), "w_gate_up", "x")
    _expect(lambda: moe.moe_gate_up(x, wgu, g, _K, _t(g.max_rows - 1, _I)), "act")
    _expect(lambda: moe.moe_gate_up(x, wgu, g, _K, _t(g.max_rows, _I + 64)), "act")
    _expect(lambda: moe.moe_gate_up(x, wgu, _grouping(_N * _K + 2), _K, act), "grouping")
    _expect(lambda: moe.moe_gate_up(x, _t(_E + 1, 2 * _I, _H), g, _K, act), "grouping")
    _expect(lambda: moe.moe_down(_t(g.max_rows, _I + 64), wd, tw, g, _N, _K, y), "act")
    _expect(lambda: moe.moe_down(act, _t(_E, _H, _I + 64), tw, g, _N, _K, y), "act")
    _expect(lambda: moe.moe_down(act, wd, _t(_N, _K + 1, dtype=torch.float32), g, _N, _K, y), "topk_w")
    _expect(lambda: moe.moe_down(act, wd, tw, g, _N, _K, _t(_N * _K, _H + 64)), "y")
    _expect(lambda: moe.moe_down(act, wd, tw, g, _N + 1, _K, y), "grouping")


def test_ids_products_reject_wrong_shapes():
    x, wgu, wd = _t(_N, _H), _t(_E, 2 * _I, _H), _t(_E, _H, _I)
    ids, tw = _t(_N, _K, dtype=torch.int32), _t(_N, _K, dtype=torch.float32)
    act, y = _t(_N * _K, _I), _t(_N * _K, _H)
    _expect_device_error(lambda: moe.moe_gate_up_ids(x, wgu, ids, act))
    _expect_device_error(lambda: moe.moe_down_ids(act, wd, ids, tw, y))
    _expect(lambda: moe.moe_gate_up_ids(x, wgu, _t(_N + 1, _K, dtype=torch.int32), act), "topk_ids")
    _expect(lambda: moe.moe_gate_up_ids(x, wgu, ids, _t(_N * _K - 1, _I)), "act")
    _expect(lambda: moe.moe_gate_up_ids(x, _t(_E, 2 * _I, _H - 64), ids, act), "w_gate_up")
    _expect(lambda: moe.moe_down_ids(_t(_N * _K, _I + 64), wd, ids, tw, y), "act")
    _expect(lambda: moe.moe_down_ids(act, wd, ids, _t(_N * _K, dtype=torch.float32), y), "topk_w")
    _expect(lambda: moe.moe_down_ids(act, wd, ids, tw, _t(_N * _K, _H - 64)), "y")


def test_shared_combine_dense_norm_reject_wrong_shapes():
    x, sgu, sdn, sc = _t(_N, _H), _t(2 * _IS, _H), _t(_H, _IS), _t(_N, dtype=torch.float32)
    _expect_device_error(lambda: moe.moe_shared_expert(x, sgu, sdn, sc))
    _expect(lambda: moe.moe_shared_expert(x, sgu, _t(_IS, _H), sc), "shared_w_down")
    _expect(lambda: moe.moe_shared_expert(x, sgu, sdn, _t(_N + 1, dtype=torch.float32)), "shared_scale")
    _expect(lambda: moe.moe_shared_expert(x, sgu, sdn, sc, shared_act=_t(_N, _IS + 64)), "shared_act")
    _expect(lambda: moe.moe_shared_expert(x, sgu, sdn, sc, shared_y=_t(_N, _H + 64)), "shared_y")
    y = _t(_N * _K, _H)
    _expect_device_error(lambda: moe.moe_combine(y, _N, _K))
    _expect(lambda: moe.moe_combine(_t(_N * _K - 1, _H), _N, _K), "y")
    _expect(lambda: moe.moe_combine(y, _N, _K, shared_y=_t(_N, _H + 64)), "shared_y")
    _expect(lambda: moe.moe_combine(y, _N, _K, out=_t(_N + 1, _H)), "out")
    gu, dn = _t(2 * _I, _H), _t(_H, _I)
    _expect_device_error(lambda: moe.moe_dense_mlp(x, gu, dn))
    _expect(lambda: moe.moe_dense_mlp(x, gu, _t(_I, _H)), "w_down")
    _expect(lambda: moe.moe_dense_mlp(x, gu, dn, act=_t(_N, _I + 64)), "act")
    _expect(lambda: moe.moe_dense_mlp(x, gu, dn, out=_t(_N, _H + 64)), "out")
    w = _t(_H)
    _expect_device_error(lambda: moe.moe_add_rmsnorm(x, x, w))
    _expect(lambda: moe.moe_add_rmsnorm(x, _t(_N, _H + 64), w), "residual")
    _expect(lambda: moe.moe_add_rmsnorm(x, x, _t(_H + 8)), "weight")
    _expect(lambda: moe.moe_add_rmsnorm(x, x, w, normed=_t(_N + 1, _H)), "normed")


def test_forward_noalloc_rejects_before_any_hip_call():
    """The allocation-free entry point checks its arguments, and that the
    problem fits its fixed scratch, before any HIP call (so on a machine
    without a GPU too)."""
    lib = moe.load_library()
    fake = ctypes.c_void_p(1 << 20)
    big = moe.problem(4096, 2048, 128, 8, 768)
    assert moe.moe_workspace_size(big) > B.MOE_NOALLOC_SCRATCH_BYTES
    rc = lib.moe_forward_noalloc(ctypes.byref(big), fake, fake, fake, fake, None, None, None, fake, None)
    assert rc == B.MOE_ENOSPC and b"scratch" in lib.moe_last_error()
    small = moe.problem(64, 2048, 128, 8, 768)
    assert moe.moe_workspace_size(small) <= B.MOE_NOALLOC_SCRATCH_BYTES
    rc = lib.moe_forward_noalloc(ctypes.byref(small), None, fake, fake, fake, None, None, None, fake, None)
    assert rc == B.MOE_EINVAL
    rc = lib.moe_forward_noalloc(ctypes.byref(small), fake, fake, fake, fake, fake, None, None, fake, None)
    assert rc == B.MOE_EINVAL                               # shared weights without shared_inter
    p0 = moe.problem(0, 64, 4, 2, 64)
    assert lib.moe_forward_noalloc(ctypes.byref(p0), None, None, None, None, None, None, None, None, None) == 0


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == B.MOE_NOALLOC_SCRATCH_BYTES


def test_mfma_probe_rejects_before_any_hip_call():
    """The matrix-unit probe checks pointers, sizes and alignment before it
    launches anything."""
    lib = moe.load_library()
    fake = ctypes.c_void_p(1 << 20)
    flops = ctypes.c_double(-1.0)
    assert lib.moe_mfma_probe(None, 512, 10, fake, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(fake, 512, 10, None, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(fake, 512, 10, fake, None, None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(fake, 0, 10, fake, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(fake, 1000, 10, fake, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(fake, 512, 0, fake, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(fake, 512, (1 << 20) + 1, fake, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert lib.moe_mfma_probe(ctypes.c_void_p((1 << 20) + 2), 512, 10, fake, ctypes.byref(flops), None) == B.MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()
    assert flops.value == -1.0                              # nothing written on an error


def test_mfma_probe_constants_match_header():
    src = open(HEADER).read()
    assert re.search(r"#define MOE_PROBE_WORKGROUPS (\d+)", src).group(1) == str(B.MOE_PROBE_WORKGROUPS)
    assert "#define MOE_PROBE_SINK_FLOATS (MOE_PROBE_WORKGROUPS * 8 * 64)" in src
    assert B.MOE_PROBE_SINK_FLOATS == B.MOE_PROBE_WORKGROUPS * 8 * 64


def test_route_rejects_misaligned_scratch_before_any_hip_call():
    """The router writes its partial logits with 16-byte stores, so a bf16
    call with a scratch pointer that is not 16-byte aligned is refused before
    anything is launched."""
    lib = moe.load_library()
    p = moe.problem(64, 2048, 128, 8, 768)
    fake = ctypes.c_void_p(1 << 20)
    rc = lib.moe_route(ctypes.byref(p), fake, fake, None, fake, fake, None, ctypes.c_void_p((1 << 20) + 4), None)
    assert rc == B.MOE_EUNSUPPORTED and b"aligned" in lib.moe_last_error()


def test_shared_expert_tile_height_and_merge():
    """The layout reports the shared expert's tile height and which products
    moe_forward runs in one launch with the routed tiles (bit 0 gate/up,
    bit 1 down; host arithmetic)."""
    L = lambda *a, **kw: moe.moe_get_workspace_layout(moe.problem(*a, **kw))
    talker = L(8192, 2048, 128, 8, 768, 2048)          # routed 320, shared 320
    assert (talker["block_m"], talker["shared_block_m"], talker["shared_merged"]) == (320, 320, 3)
    # The ids products take the shared tiles where they fit the last round of
    # the routed launch: expected hit experts E (1 - (1 - 1/E)^P) times the
    # column blocks, rounds of 256 (gate/up) or 512 / 768 (down) workgroups.
    for N, bits in ((24, 3), (32, 3), (48, 0), (64, 0), (80, 2), (96, 2)):
        small = L(N, 2048, 128, 8, 768, 2048)
        assert (small["ids_products"], small["shared_block_m"], small["shared_merged"]) == (1, 16, bits), N
    assert L(53, 960, 92, 8, 64, 128)["shared_merged"] == 1
    plain = L(4096, 2048, 128, 8, 768)                 # no shared expert
    assert (plain["shared_block_m"], plain["shared_merged"]) == (0, 0)
    apart = L(700, 192, 300, 8, 64, 192)               # routed 64, shared 16
    assert (apart["block_m"], apart["shared_block_m"], apart["shared_merged"]) == (64, 16, 0)
    f32 = L(4100, 128, 8, 2, 64, 1280, dtype=torch.float32)
    assert f32["shared_merged"] == 0
