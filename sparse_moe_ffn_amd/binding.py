"""Python binding of the C ABI in ``include/moe_mi355x.h``.

Argument marshalling only: every function checks that its tensors are
contiguous, on one GPU and of the expected dtype, allocates missing outputs
with torch (device memory is torch's), passes raw pointers and torch's current
stream, and raises ``MoEError`` with the library's message on a non-zero
return.  All computation happens in the HIP kernels of
``libmoe_mi355x.so``; there is no fallback: if the library is missing, or
has no GPU to run on, calls fail.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_ENOSPC, MOE_EUNSUPPORTED, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_LAYOUT_ROW_MAJOR, MOE_LAYOUT_BLOCKED = 0, 1

_DTYPES = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


class MoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


class MoEProblem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("num_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("shared_inter", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MoEWorkspaceLayout(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int64), ("max_rows", ctypes.c_int64), ("max_tiles", ctypes.c_int64),
                ("ids_products", ctypes.c_int64), ("shared_block_m", ctypes.c_int64),
                ("shared_merged", ctypes.c_int64)] + [
        (n, ctypes.c_size_t) for n in ("route_scratch", "topk_ids", "topk_w", "shared_scale", "counts", "offsets",
                                       "order",
                                       "sorted_pairs", "tile_expert", "tile_rows", "num_tiles", "align_scratch",
                                       "act", "y",
                                       "shared_act", "shared_y", "total_bytes")]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def load_library() -> ctypes.CDLL:
    """The HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_ffn_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        PP = ctypes.POINTER(MoEProblem)
        sig = {
            "moe_workspace_size": [PP, ctypes.POINTER(ctypes.c_size_t)],
            "moe_get_workspace_layout": [PP, ctypes.POINTER(MoEWorkspaceLayout)],
            "moe_align_capacity": [_I64, _I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
            "moe_route": [PP, _P, _P, _P, _P, _P, _P, _P, _P],
            "moe_route_scratch_size": [PP, ctypes.POINTER(ctypes.c_size_t)],
            "moe_align": [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P],
            "moe_align_scratch_size": [_I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
            "moe_gate_up": [PP, _P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P],
            "moe_down": [PP, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P],
            "moe_gate_up_ids": [PP, _P, _P, _P, _P, _P],
            "moe_down_ids": [PP, _P, _P, _P, _P, _P, _P],
            "moe_shared_expert": [PP, _P, _P, _P, _P, _P, _P, _P],
            "moe_combine": [PP, _P, _P, _P, _P],
            "moe_forward": [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
            "moe_forward_noalloc": [PP, _P, _P, _P, _P, _P, _P, _P, _P, _P],
            "moe_dense_mlp": [PP, _P, _P, _P, _P, _P, _P],
            "moe_add_rmsnorm": [_I64, _I64, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_float, _P, _P],
            "moe_pack_weights": [_I64, _I64, _I64, ctypes.c_int32, _P, _P, _P],
            "moe_mfma_probe": [_P, _I64, _I64, _P, ctypes.POINTER(ctypes.c_double), _P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.moe_last_error.argtypes = []
        lib.moe_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoEError(rc, load_library().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(t: torch.Tensor, name: str, dtype=None, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _tensor(t, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    return t


def _shape(t, name: str, shape) -> torch.Tensor:
    """Raise ValueError unless `t` has exactly `shape`.  Every binding checks
    the shape of each tensor it passes, before any device check or launch: a
    mis-shaped tensor would size the kernels' reads and writes wrongly."""
    _tensor(t, name)
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(int(d) for d in shape)}, got {tuple(t.shape)}")
    return t


def _rank(t, name: str, ndim: int) -> torch.Tensor:
    _tensor(t, name)
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return t


def _numel_at_least(t, name: str, n: int) -> torch.Tensor:
    _tensor(t, name)
    if t.numel() < n:
        raise ValueError(f"{name} must hold at least {n} elements, got {t.numel()}")
    return t


def _rows_cols(t, name: str, min_rows: int, cols: int) -> torch.Tensor:
    """A 2-D tensor with exactly `cols` columns and at least `min_rows` rows
    (intermediate buffers may be larger than one call needs)."""
    _rank(t, name, 2)
    if t.shape[1] != cols or t.shape[0] < min_rows:
        raise ValueError(f"{name} must have shape (>= {min_rows}, {cols}), got {tuple(t.shape)}")
    return t


def problem(num_tokens, hidden, num_experts, top_k, inter, shared_inter=0, dtype=torch.bfloat16,
            norm_topk_prob=True, weight_layout=MOE_LAYOUT_ROW_MAJOR) -> MoEProblem:
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    return MoEProblem(int(num_tokens), int(hidden), int(num_experts), int(top_k), int(inter),
                      int(shared_inter), _DTYPES[dtype], int(bool(norm_topk_prob)), int(weight_layout), 0)


def problem_from(x, w_gate_up, router_w, top_k, norm_topk_prob, shared_w_gate_up=None,
                 weight_layout=MOE_LAYOUT_ROW_MAJOR) -> MoEProblem:
    N, H = _rank(x, "x", 2).shape
    E, two_i, H2 = _rank(w_gate_up, "w_gate_up", 3).shape
    if H2 != H or two_i % 2:
        raise ValueError(f"w_gate_up must have shape (E, 2I, {H}), got {tuple(w_gate_up.shape)}")
    _shape(router_w, "router_w", (E, H))
    if shared_w_gate_up is not None:
        Is2, H3 = _rank(shared_w_gate_up, "shared_w_gate_up", 2).shape
        if H3 != H or Is2 % 2:
            raise ValueError(f"shared_w_gate_up must have shape (2I_s, {H}), got {tuple(shared_w_gate_up.shape)}")
    Is = 0 if shared_w_gate_up is None else shared_w_gate_up.shape[0] // 2
    return problem(N, H, E, top_k, two_i // 2, Is, x.dtype, norm_topk_prob, weight_layout)


def moe_pack_weights(w, out=None):
    """`w` ([rows, cols] or [batch, rows, cols], bf16, row-major) in the
    blocked layout of moe_pack_weights: a tensor of the same shape whose
    storage holds the 64-column panels (index it only through the library)."""
    w = _gpu(w, "w", torch.bfloat16)
    if w.dim() not in (2, 3):
        raise ValueError("w must be [rows, cols] or [batch, rows, cols]")
    batch, rows, cols = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    if out is None:
        out = torch.empty_like(w)
    _gpu(out, "out", torch.bfloat16, w.device)
    if out.shape != w.shape:
        raise ValueError("out must have the shape of w")
    with torch.cuda.device(w.device):
        _check(load_library().moe_pack_weights(batch, rows, cols, MOE_BF16, _ptr(w), _ptr(out), _stream(w.device)))
    return out


def moe_workspace_size(p: MoEProblem) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_get_workspace_layout(p: MoEProblem) -> dict:
    L = MoEWorkspaceLayout()
    _check(load_library().moe_get_workspace_layout(ctypes.byref(p), ctypes.byref(L)))
    return {name: getattr(L, name) for name, _ in MoEWorkspaceLayout._fields_}


def moe_align_capacity(num_pairs: int, num_experts: int, block_m: int):
    r, t = _I64(), _I64()
    _check(load_library().moe_align_capacity(num_pairs, num_experts, block_m, ctypes.byref(r), ctypes.byref(t)))
    return r.value, t.value


def moe_route_scratch_size(p: MoEProblem) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_route_scratch_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def moe_route(x, router_w, top_k, norm_topk_prob, shared_gate=None, topk_ids=None, topk_w=None,
              shared_scale=None, scratch=None):
    """(topk_ids int32 [N,k], topk_w float32 [N,k], shared_scale float32 [N] or None)."""
    N, H = _rank(x, "x", 2).shape
    E = _rank(router_w, "router_w", 2).shape[0]
    _shape(router_w, "router_w", (E, H))
    if shared_gate is not None and _tensor(shared_gate, "shared_gate").numel() != H:
        raise ValueError(f"shared_gate must have {H} elements, got {shared_gate.numel()}")
    for t, n, shape in ((topk_ids, "topk_ids", (N, top_k)), (topk_w, "topk_w", (N, top_k)),
                        (shared_scale, "shared_scale", (N,))):
        if t is not None:
            _shape(t, n, shape)
    p = problem(N, H, E, top_k, 1, 0, x.dtype, norm_topk_prob)
    if scratch is not None:
        _numel_at_least(scratch, "scratch", -(-moe_route_scratch_size(p) // 4))
    x = _gpu(x, "x")
    dev = x.device
    router_w = _gpu(router_w, "router_w", x.dtype, dev)
    if shared_gate is not None:
        shared_gate = _gpu(shared_gate, "shared_gate", x.dtype, dev)
        if shared_scale is None:
            shared_scale = torch.empty(N, dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty((N, top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((N, top_k), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(max(1, moe_route_scratch_size(p) // 4), dtype=torch.float32, device=dev)
    _gpu(topk_ids, "topk_ids", torch.int32, dev)
    _gpu(topk_w, "topk_w", torch.float32, dev)
    if shared_scale is not None:
        _gpu(shared_scale, "shared_scale", torch.float32, dev)
    _gpu(scratch, "scratch", torch.float32, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_route(ctypes.byref(p), _ptr(x), _ptr(router_w), _ptr(shared_gate),
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(shared_scale), _ptr(scratch),
                                        _stream(dev)))
    return topk_ids, topk_w, shared_scale


@dataclass
class Grouping:
    counts: torch.Tensor
    offsets: torch.Tensor
    order: torch.Tensor
    sorted_pairs: torch.Tensor
    tile_expert: torch.Tensor
    tile_rows: torch.Tensor
    num_tiles: torch.Tensor
    block_m: int
    max_rows: int
    max_tiles: int
    num_experts: int
    num_pairs: int


def moe_align_scratch_size(num_pairs: int, num_experts: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_align_scratch_size(num_pairs, num_experts, ctypes.byref(n)))
    return n.value


def moe_align(topk_ids, num_experts: int, block_m: int, scratch=None) -> Grouping:
    N, k = _rank(topk_ids, "topk_ids", 2).shape
    P = N * k
    max_rows, max_tiles = moe_align_capacity(P, num_experts, block_m)
    need = moe_align_scratch_size(P, num_experts)
    if need and scratch is not None:
        _numel_at_least(scratch, "scratch", need // 4)
    topk_ids = _gpu(topk_ids, "topk_ids", torch.int32)
    dev = topk_ids.device
    i32 = dict(dtype=torch.int32, device=dev)
    g = Grouping(torch.empty(num_experts, **i32), torch.empty(num_experts + 1, **i32), torch.empty(P, **i32),
                 torch.empty(max_rows, **i32), torch.empty(max_tiles, **i32), torch.empty(max_tiles, **i32),
                 torch.empty(1, **i32), block_m, max_rows, max_tiles, num_experts, P)
    if scratch is None and need:
        scratch = torch.empty(need // 4, **i32)
    if need:
        _gpu(scratch, "scratch", torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_align(_ptr(topk_ids), N, k, num_experts, block_m, _ptr(g.counts),
                                        _ptr(g.offsets), _ptr(g.order), _ptr(g.sorted_pairs),
                                        _ptr(g.tile_expert), _ptr(g.tile_rows), _ptr(g.num_tiles),
                                        _ptr(scratch) if need else None, _stream(dev)))
    return g


def _check_grouping(grouping: Grouping, num_pairs: int, num_experts: int):
    """The grouping must be the one moe_align made for these pairs and experts:
    its tile table sizes the products' grids and its pair indices address
    their rows."""
    if grouping.num_pairs != num_pairs or grouping.num_experts != num_experts:
        raise ValueError(f"grouping was made for {grouping.num_pairs} pairs and {grouping.num_experts} experts, "
                         f"not {num_pairs} and {num_experts}")
    rows, tiles = moe_align_capacity(num_pairs, num_experts, grouping.block_m)
    if (grouping.max_rows, grouping.max_tiles) != (rows, tiles):
        raise ValueError("grouping capacity does not match its pairs, experts and block_m")
    for t, n, shape in ((grouping.sorted_pairs, "sorted_pairs", (rows,)), (grouping.tile_expert, "tile_expert", (tiles,)),
                        (grouping.tile_rows, "tile_rows", (tiles,)), (grouping.num_tiles, "num_tiles", (1,))):
        _shape(t, "grouping." + n, shape)


def moe_gate_up(x, w_gate_up, grouping: Grouping, top_k: int, act=None, weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """act [max_rows, I] in x.dtype (rows of sentinel pairs are not written)."""
    N, H = _rank(x, "x", 2).shape
    E, two_i, H2 = _rank(w_gate_up, "w_gate_up", 3).shape
    if H2 != H or two_i % 2:
        raise ValueError(f"w_gate_up must have shape (E, 2I, {H}), got {tuple(w_gate_up.shape)}")
    _check_grouping(grouping, N * top_k, E)
    if act is not None:
        _rows_cols(act, "act", grouping.max_rows, two_i // 2)
    x = _gpu(x, "x")
    dev = x.device
    w_gate_up = _gpu(w_gate_up, "w_gate_up", x.dtype, dev)
    p = problem(N, H, E, top_k, two_i // 2, 0, x.dtype, weight_layout=weight_layout)
    if act is None:
        act = torch.empty((grouping.max_rows, two_i // 2), dtype=x.dtype, device=dev)
    _gpu(act, "act", x.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_gate_up(ctypes.byref(p), _ptr(x), _ptr(w_gate_up), _ptr(grouping.sorted_pairs),
                                          _ptr(grouping.tile_expert), _ptr(grouping.tile_rows),
                                          _ptr(grouping.num_tiles), grouping.block_m, grouping.max_tiles,
                                          _ptr(act), _stream(dev)))
    return act


def moe_down(act, w_down, topk_w, grouping: Grouping, num_tokens: int, top_k: int, y=None,
             weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """y [N*k, H] in act.dtype: y[p] = topk_w[p] * (act[row of p] . w_down[e]^T)."""
    E, H, I = _rank(w_down, "w_down", 3).shape
    _check_grouping(grouping, num_tokens * top_k, E)
    _rows_cols(act, "act", grouping.max_rows, I)
    if _tensor(topk_w, "topk_w").numel() != num_tokens * top_k:
        raise ValueError(f"topk_w must have {num_tokens * top_k} elements, got {topk_w.numel()}")
    if y is not None:
        _shape(y, "y", (num_tokens * top_k, H))
    act = _gpu(act, "act")
    dev = act.device
    w_down = _gpu(w_down, "w_down", act.dtype, dev)
    topk_w = _gpu(topk_w, "topk_w", torch.float32, dev)
    p = problem(num_tokens, H, E, top_k, I, 0, act.dtype, weight_layout=weight_layout)
    if y is None:
        y = torch.empty((num_tokens * top_k, H), dtype=act.dtype, device=dev)
    _gpu(y, "y", act.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_down(ctypes.byref(p), _ptr(act), _ptr(w_down), _ptr(topk_w),
                                       _ptr(grouping.sorted_pairs), _ptr(grouping.tile_expert),
                                       _ptr(grouping.tile_rows), _ptr(grouping.num_tiles), grouping.block_m,
                                       grouping.max_tiles, _ptr(y), _stream(dev)))
    return y


def moe_gate_up_ids(x, w_gate_up, topk_ids, act=None, weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """act [N*k, I] in x.dtype, indexed by pair: act[p] = SwiGLU of x[p / k]
    through expert topk_ids[p] (no grouping needed; bf16, 4 <= N*k <= 1024)."""
    N, H = _rank(x, "x", 2).shape
    E, two_i, H2 = _rank(w_gate_up, "w_gate_up", 3).shape
    if H2 != H or two_i % 2:
        raise ValueError(f"w_gate_up must have shape (E, 2I, {H}), got {tuple(w_gate_up.shape)}")
    if _rank(topk_ids, "topk_ids", 2).shape[0] != N:
        raise ValueError(f"topk_ids must have shape ({N}, k), got {tuple(topk_ids.shape)}")
    k = topk_ids.shape[1]
    if act is not None:
        _rows_cols(act, "act", N * k, two_i // 2)
    x = _gpu(x, "x")
    dev = x.device
    w_gate_up = _gpu(w_gate_up, "w_gate_up", x.dtype, dev)
    topk_ids = _gpu(topk_ids, "topk_ids", torch.int32, dev)
    p = problem(N, H, E, k, two_i // 2, 0, x.dtype, weight_layout=weight_layout)
    if act is None:
        act = torch.empty((N * k, two_i // 2), dtype=x.dtype, device=dev)
    _gpu(act, "act", x.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_gate_up_ids(ctypes.byref(p), _ptr(x), _ptr(w_gate_up), _ptr(topk_ids), _ptr(act),
                                              _stream(dev)))
    return act


def moe_down_ids(act, w_down, topk_ids, topk_w, y=None, weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """y [N*k, H] in act.dtype: y[p] = topk_w[p] * (act[p] . w_down[topk_ids[p]]^T)."""
    E, H, I = _rank(w_down, "w_down", 3).shape
    N, k = _rank(topk_ids, "topk_ids", 2).shape
    _rows_cols(act, "act", N * k, I)
    _shape(topk_w, "topk_w", (N, k))
    if y is not None:
        _shape(y, "y", (N * k, H))
    act = _gpu(act, "act")
    dev = act.device
    w_down = _gpu(w_down, "w_down", act.dtype, dev)
    topk_ids = _gpu(topk_ids, "topk_ids", torch.int32, dev)
    topk_w = _gpu(topk_w, "topk_w", torch.float32, dev)
    p = problem(N, H, E, k, I, 0, act.dtype, weight_layout=weight_layout)
    if y is None:
        y = torch.empty((N * k, H), dtype=act.dtype, device=dev)
    _gpu(y, "y", act.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_down_ids(ctypes.byref(p), _ptr(act), _ptr(w_down), _ptr(topk_ids), _ptr(topk_w),
                                           _ptr(y), _stream(dev)))
    return y


def moe_shared_expert(x, shared_w_gate_up, shared_w_down, shared_scale, shared_act=None, shared_y=None,
                      weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """(shared_act [N, I_s], shared_y [N, H] = shared_scale[:, None] * SwiGLU_s(x))."""
    N, H = _rank(x, "x", 2).shape
    Is2, H2 = _rank(shared_w_gate_up, "shared_w_gate_up", 2).shape
    if H2 != H or Is2 % 2:
        raise ValueError(f"shared_w_gate_up must have shape (2I_s, {H}), got {tuple(shared_w_gate_up.shape)}")
    Is = Is2 // 2
    _shape(shared_w_down, "shared_w_down", (H, Is))
    _shape(shared_scale, "shared_scale", (N,))
    if shared_act is not None:
        _shape(shared_act, "shared_act", (N, Is))
    if shared_y is not None:
        _shape(shared_y, "shared_y", (N, H))
    x = _gpu(x, "x")
    dev = x.device
    shared_w_gate_up = _gpu(shared_w_gate_up, "shared_w_gate_up", x.dtype, dev)
    shared_w_down = _gpu(shared_w_down, "shared_w_down", x.dtype, dev)
    shared_scale = _gpu(shared_scale, "shared_scale", torch.float32, dev)
    p = problem(N, H, 1, 1, 1, Is, x.dtype, weight_layout=weight_layout)
    if shared_act is None:
        shared_act = torch.empty((N, Is), dtype=x.dtype, device=dev)
    if shared_y is None:
        shared_y = torch.empty((N, H), dtype=x.dtype, device=dev)
    _gpu(shared_act, "shared_act", x.dtype, dev)
    _gpu(shared_y, "shared_y", x.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_shared_expert(ctypes.byref(p), _ptr(x), _ptr(shared_w_gate_up),
                                                _ptr(shared_w_down), _ptr(shared_scale), _ptr(shared_act),
                                                _ptr(shared_y), _stream(dev)))
    return shared_act, shared_y


def moe_combine(y, num_tokens: int, top_k: int, shared_y=None, out=None):
    """out [N, H] = sum over the k slot rows of y (+ shared_y)."""
    H = _rank(y, "y", 2).shape[1]
    _shape(y, "y", (num_tokens * top_k, H))
    if shared_y is not None:
        _shape(shared_y, "shared_y", (num_tokens, H))
    if out is not None:
        _shape(out, "out", (num_tokens, H))
    y = _gpu(y, "y")
    dev = y.device
    if shared_y is not None:
        shared_y = _gpu(shared_y, "shared_y", y.dtype, dev)
    p = problem(num_tokens, H, top_k, top_k, 1, 0, y.dtype)
    if out is None:
        out = torch.empty((num_tokens, H), dtype=y.dtype, device=dev)
    _gpu(out, "out", y.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_combine(ctypes.byref(p), _ptr(y), _ptr(shared_y), _ptr(out), _stream(dev)))
    return out


def moe_dense_mlp(x, w_gate_up, w_down, act=None, out=None, weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """Dense SwiGLU layer: out [N, H] = (silu(x Wg^T) * (x Wu^T)) Wd^T, with
    w_gate_up [2I, H] (gate rows first) and w_down [H, I]; act [N, I] is the
    intermediate (allocated when not given)."""
    N, H = _rank(x, "x", 2).shape
    two_i, H2 = _rank(w_gate_up, "w_gate_up", 2).shape
    if H2 != H or two_i % 2:
        raise ValueError(f"w_gate_up must have shape (2I, {H}), got {tuple(w_gate_up.shape)}")
    I = two_i // 2
    _shape(w_down, "w_down", (H, I))
    if act is not None:
        _shape(act, "act", (N, I))
    if out is not None:
        _shape(out, "out", (N, H))
    x = _gpu(x, "x")
    dev = x.device
    w_gate_up = _gpu(w_gate_up, "w_gate_up", x.dtype, dev)
    w_down = _gpu(w_down, "w_down", x.dtype, dev)
    p = problem(N, H, 1, 1, I, 0, x.dtype, weight_layout=weight_layout)
    if act is None:
        act = torch.empty((N, I), dtype=x.dtype, device=dev)
    if out is None:
        out = torch.empty_like(x)
    _gpu(act, "act", x.dtype, dev)
    _gpu(out, "out", x.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_dense_mlp(ctypes.byref(p), _ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(act),
                                            _ptr(out), _stream(dev)))
    return out


def moe_add_rmsnorm(x, residual, weight, eps=1e-6, residual_out=None, normed=None):
    """(normed, residual_out): residual_out = x + residual (x when residual is
    None), normed = RMSNorm(residual_out) * weight.  residual_out may be
    `residual` itself (in place)."""
    N, H = _rank(x, "x", 2).shape
    for t, n in ((residual, "residual"), (residual_out, "residual_out"), (normed, "normed")):
        if t is not None:
            _shape(t, n, (N, H))
    if _tensor(weight, "weight").numel() != H:
        raise ValueError(f"weight must have {H} elements, got {weight.numel()}")
    x = _gpu(x, "x")
    dev = x.device
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if residual is not None:
        _gpu(residual, "residual", x.dtype, dev)
    weight = _gpu(weight, "weight", x.dtype, dev)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    if normed is None:
        normed = torch.empty_like(x)
    _gpu(residual_out, "residual_out", x.dtype, dev)
    _gpu(normed, "normed", x.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_add_rmsnorm(N, H, _DTYPES[x.dtype], _ptr(x), _ptr(residual), _ptr(residual_out),
                                              _ptr(weight), float(eps), _ptr(normed), _stream(dev)))
    return normed, residual_out


_workspaces = {}


def workspace_for(p: MoEProblem, device) -> torch.Tensor:
    """A cached uint8 workspace large enough for `p`, one per (device,
    current stream).  Calls on one stream run in order and can share it;
    calls on different streams may run at the same time, so each stream has
    its own.  The workspace is allocated on that stream, so when it grows,
    torch's allocator reuses the old block only for later work on the same
    stream."""
    need = moe_workspace_size(p)
    dev = torch.device(device)
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _check_forward_shapes(x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out):
    """Shapes of every tensor of the whole block, against x [N, H] and
    w_gate_up [E, 2I, H]; raises ValueError before any device use."""
    N, H = _rank(x, "x", 2).shape
    E, two_i, H2 = _rank(w_gate_up, "w_gate_up", 3).shape
    if H2 != H or two_i % 2:
        raise ValueError(f"w_gate_up must have shape (E, 2I, {H}), got {tuple(w_gate_up.shape)}")
    _shape(router_w, "router_w", (E, H))
    _shape(w_down, "w_down", (E, H, two_i // 2))
    given = [t is not None for t in (shared_w_gate_up, shared_w_down, shared_gate)]
    if any(given) and not all(given):
        raise ValueError("the shared expert needs shared_w_gate_up, shared_w_down and shared_gate together")
    if shared_w_gate_up is not None:
        Is2, H3 = _rank(shared_w_gate_up, "shared_w_gate_up", 2).shape
        if H3 != H or Is2 % 2:
            raise ValueError(f"shared_w_gate_up must have shape (2I_s, {H}), got {tuple(shared_w_gate_up.shape)}")
        _shape(shared_w_down, "shared_w_down", (H, Is2 // 2))
        if _tensor(shared_gate, "shared_gate").numel() != H:
            raise ValueError(f"shared_gate must have {H} elements, got {shared_gate.numel()}")
    if out is not None:
        _shape(out, "out", (N, H))


def moe_forward(x, router_w, w_gate_up, w_down, top_k, norm_topk_prob=True, shared_w_gate_up=None,
                shared_w_down=None, shared_gate=None, out=None, workspace=None, weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """The whole block: out [N, H] in x.dtype.  With weight_layout
    MOE_LAYOUT_BLOCKED the expert (and shared-expert) weights are the
    outputs of moe_pack_weights.  Without `workspace`, the cached workspace
    of the current stream is used (workspace_for)."""
    _check_forward_shapes(x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out)
    p = problem_from(x, w_gate_up, router_w, top_k, norm_topk_prob, shared_w_gate_up, weight_layout)
    if workspace is not None:
        _numel_at_least(workspace, "workspace", moe_workspace_size(p))
    x = _gpu(x, "x")
    dev = x.device
    for t, n in ((router_w, "router_w"), (w_gate_up, "w_gate_up"), (w_down, "w_down")):
        _gpu(t, n, x.dtype, dev)
    for t, n in ((shared_w_gate_up, "shared_w_gate_up"), (shared_w_down, "shared_w_down"),
                 (shared_gate, "shared_gate")):
        if t is not None:
            _gpu(t, n, x.dtype, dev)
    if out is None:
        out = torch.empty_like(x)
    _gpu(out, "out", x.dtype, dev)
    if workspace is None:
        workspace = workspace_for(p, dev)
    _gpu(workspace, "workspace", torch.uint8, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_forward(ctypes.byref(p), _ptr(x), _ptr(router_w), _ptr(w_gate_up), _ptr(w_down),
                                          _ptr(shared_w_gate_up), _ptr(shared_w_down), _ptr(shared_gate),
                                          _ptr(out), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20     # the fixed scratch behind moe_forward_noalloc (include/moe_mi355x.h)


def moe_forward_noalloc(x, router_w, w_gate_up, w_down, top_k, norm_topk_prob, shared_w_gate_up=None,
                        shared_w_down=None, shared_gate=None, out=None, weight_layout=MOE_LAYOUT_ROW_MAJOR):
    """The whole block through the allocation-free entry point: the library
    keeps every intermediate in its fixed per-GPU scratch array (problems
    whose workspace exceeds MOE_NOALLOC_SCRATCH_BYTES are rejected).  `out`
    is allocated here only when not given."""
    _check_forward_shapes(x, router_w, w_gate_up, w_down, shared_w_gate_up, shared_w_down, shared_gate, out)
    p = problem_from(x, w_gate_up, router_w, top_k, norm_topk_prob, shared_w_gate_up, weight_layout)
    x = _gpu(x, "x")
    dev = x.device
    for t, n in ((router_w, "router_w"), (w_gate_up, "w_gate_up"), (w_down, "w_down")):
        _gpu(t, n, x.dtype, dev)
    for t, n in ((shared_w_gate_up, "shared_w_gate_up"), (shared_w_down, "shared_w_down"),
                 (shared_gate, "shared_gate")):
        if t is not None:
            _gpu(t, n, x.dtype, dev)
    if out is None:
        out = torch.empty_like(x)
    _gpu(out, "out", x.dtype, dev)
    with torch.cuda.device(dev):
        _check(load_library().moe_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(router_w), _ptr(w_gate_up),
                                                  _ptr(w_down), _ptr(shared_w_gate_up), _ptr(shared_w_down),
                                                  _ptr(shared_gate), _ptr(out), _stream(dev)))
    return out


MOE_PROBE_WORKGROUPS = 512
MOE_PROBE_SINK_FLOATS = MOE_PROBE_WORKGROUPS * 8 * 64


def moe_mfma_probe(operands, iters, sink=None) -> float:
    """Enqueue the matrix-unit rate probe on the current stream and return
    the launch's matrix flops (time it with events on that stream).
    operands: bf16 GPU tensor, a positive multiple of 512 elements (random
    values); sink: float32 GPU tensor of MOE_PROBE_SINK_FLOATS (allocated
    when None)."""
    ops = _gpu(operands, "operands", torch.bfloat16)
    if ops.numel() < 512 or ops.numel() % 512:
        raise ValueError(f"operands must hold a positive multiple of 512 elements, got {ops.numel()}")
    if sink is None:
        sink = torch.empty(MOE_PROBE_SINK_FLOATS, dtype=torch.float32, device=ops.device)
    sink = _gpu(sink, "sink", torch.float32, ops.device)
    if sink.numel() < MOE_PROBE_SINK_FLOATS:
        raise ValueError(f"sink must hold {MOE_PROBE_SINK_FLOATS} floats, got {sink.numel()}")
    flops = ctypes.c_double(0.0)
    with torch.cuda.device(ops.device):
        _check(load_library().moe_mfma_probe(_ptr(ops), ops.numel(), int(iters), _ptr(sink), ctypes.byref(flops),
                                             _stream(ops.device)))
    return flops.value
