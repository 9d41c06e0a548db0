"""MI355X (gfx950) MoE expert path: route -> dispatch -> grouped SwiGLU FFN -> combine.

The computation lives in hand-written HIP kernels behind the C ABI of
include/moe.h (libmoe_mi355x.so, built in-tree by `build.py`).  This package
only marshals torch tensors and streams into that library.
"""
from ._lib import LIB_PATH, MoEError, lib  # noqa: F401
from .layer import MoELayer  # noqa: F401
from .ops import (alloc_plan, alloc_workspace, moe_check_error, moe_combine, moe_dispatch,  # noqa: F401
                  moe_capacity, moe_expert_ffn, moe_ffn_down, moe_ffn_plan, moe_ffn_up, moe_max_rows, moe_pack_weights,
                  moe_route, moe_router_logits, moe_workspace_bytes, moe_quantize_fp8,
                  moe_expert_ffn_fp8, moe_ffn_up_fp8, moe_ffn_down_fp8, moe_forward_fused_fp8, moe_expert_ffn_list,
                  weight_table, moe_route_reroute, moe_route_reroute_noalloc, moe_ffn_up_train, moe_pack_weights_backward,
                  moe_combine_backward, moe_gate_backward, moe_ffn_down_backward,
                  moe_ffn_up_backward, moe_ffn_wgrad, moe_wgrad_workspace_bytes,
                  moe_router_backward, moe_router_backward_workspace_bytes, moe_set_fused_overlap,
                  moe_forward_fused_list, moe_expert_ffn_fp8_list, moe_ffn_up_fp8_list,
                  moe_ffn_down_fp8_list, moe_forward_fused_fp8_list)
