"""Expert-parallel MoE layer on one EP rank's share, for MI355X (gfx950).

The layer runs in the HIP library ``libmoe.so`` (C ABI in include/moe.h);
``_lib`` is its ctypes binding and ``build`` compiles it with hipcc.
"""
from . import _lib  # noqa: F401
from ._lib import (MOE_LAYOUT_KN, MOE_LAYOUT_NK,  # noqa: F401
                   DeviceWeights, MoeError, Problem, Weights,
                   device_weights, make_problem, moe_check_problem,
                   moe_combine, moe_dispatch, moe_dispatch_workspace_size,
                   moe_eplb_hottest_map, moe_eplb_plan, moe_eplb_rank_map,
                   moe_eplb_record_load, moe_ffn_intermediate,
                   moe_ffn_workspace_size, moe_grouped_ffn,
                   moe_layer_forward, moe_layer_forward_noalloc,
                   moe_layer_workspace_size,
                   moe_prepack_weights, moe_quantize_fp8_blocks,
                   moe_route_topk, moe_workspace_size, status_string)
