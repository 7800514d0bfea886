"""Sparse MoE FFN block (Qwen3-style) for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels in ``libmoe_mi355x.so``
(C ABI: ``include/moe_mi355x.h``); :mod:`.binding` marshals torch tensors to
it.  Build the library with ``python -m sparse_moe_ffn_amd.build``.
"""
from .binding import (MoEError, MoEProblem, Grouping, load_library, problem, problem_from,  # noqa: F401
                      moe_workspace_size, moe_get_workspace_layout, moe_align_capacity, moe_align_scratch_size,
                      moe_route_scratch_size,
                      moe_route,
                      moe_align, moe_gate_up, moe_down, moe_gate_up_ids, moe_down_ids, moe_shared_expert, moe_combine, moe_forward,
                      moe_dense_mlp, moe_add_rmsnorm, moe_pack_weights, moe_forward_noalloc, MOE_NOALLOC_SCRATCH_BYTES,
                      moe_mfma_probe, MOE_PROBE_SINK_FLOATS,
                      MOE_LAYOUT_ROW_MAJOR, MOE_LAYOUT_BLOCKED)
