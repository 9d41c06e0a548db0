"""ctypes view of the C ABI in include/moe.h (libmoe_mi355x.so, built in-tree).

Loading fails loudly if the library has not been built: there is no CPU or
PyTorch fallback for any step of the path.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_INVALID_TOPK = 2
MOE_ERR_UNSUPPORTED = 3
MOE_ERR_MISALIGNED = 4
MOE_ERR_WORKSPACE = 5
MOE_ERR_HIP = 6

MOE_F32 = 0
MOE_BF16 = 1
MOE_OVERLAP_NEVER = 0
MOE_OVERLAP_AUTO = 1
MOE_OVERLAP_ALWAYS = 2
MOE_GATE_SOFTMAX_TOPK_RENORM = 0
MOE_GATE_SIGMOID_TOPK_NORM = 1
MOE_FFN_PLAN_NONE = 0
MOE_FFN_PLAN_F32 = 1
MOE_FFN_PLAN_STREAM = 2
MOE_FFN_PLAN_STREAM_WIDE_OPERANDS = 3
MOE_FFN_PLAN_WIDE = 4
MOE_FFN_PLAN_BIG_ALL = 5
MOE_FFN_PLAN_BIG_TAIL = 6
MOE_FFN_PLAN_BIG_RIDE = 7
MOE_MAX_K = 8
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20
MOE_MAX_E = 1024

_vp, _i, _i64, _sz, _i32p, _fp = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_void_p, C.c_void_p

# name -> (restype, argtypes); mirrors include/moe.h
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [_i]),
    "moe_last_hip_error": (_i, []),
    "moe_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "moe_max_rows": (_i64, [_i, _i, _i, _i]),
    "moe_capacity": (_i64, [_i, _i, _i, _i64, _i64]),
    "moe_pack_weights": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "moe_router_logits": (_i, [_vp, _fp, _i, _i, _i, _fp, _vp]),
    "moe_route": (_i, [_fp, _i, _i, _i, _i, _i32p, _fp, _vp]),
    "moe_route_reroute": (_i, [_fp, _i, _i, _i, _i, _i, _i32p, _fp, _vp, _sz, _vp]),
    "moe_route_reroute_noalloc": (_i, [_fp, _i, _i, _i, _i, _i, _i32p, _fp, _vp]),
    "moe_dispatch": (_i, [_i32p, _i, _i, _i, _i, _i, _i, _vp, _i, _i, _i32p, _i32p, _i32p, _i32p,
                          _i32p, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_ffn_up": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "moe_ffn_down": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "moe_ffn_plan": (_i, [_i, _i64, _i, _i, _i, _i, _i]),
    "moe_combine": (_i, [_vp, _i32p, _fp, _i, _i, _i, _i, _vp, _vp]),
    "moe_check_error": (_i, [_vp, _vp]),
    "moe_expert_ffn_list": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_ffn_up_list": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp]),
    "moe_ffn_down_list": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp]),
    "moe_quantize_fp8": (_i, [_vp, _i, _i, _i, _vp, _fp, _vp]),
    "moe_expert_ffn_fp8": (_i, [_vp, _i32p, _i, _i64, _i, _i, _vp, _fp, _vp, _fp, _vp, _vp, _vp]),
    "moe_ffn_up_fp8": (_i, [_vp, _i32p, _i, _i64, _i, _i, _vp, _fp, _vp, _vp]),
    "moe_ffn_down_fp8": (_i, [_vp, _i32p, _i, _i64, _i, _i, _vp, _fp, _vp, _vp]),
    "moe_expert_ffn_fp8_list": (_i, [_vp, _i32p, _i, _i64, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp]),
    "moe_ffn_up_fp8_list": (_i, [_vp, _i32p, _i, _i64, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_ffn_down_fp8_list": (_i, [_vp, _i32p, _i, _i64, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_ffn_up_train": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_pack_weights_backward": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "moe_combine_backward": (_i, [_vp, _vp, _i32p, _fp, _i, _i, _i, _i, _vp, _fp, _vp]),
    "moe_gate_backward": (_i, [_fp, _i32p, _fp, _i, _i, _i, _i, _fp, _vp]),
    "moe_ffn_down_backward": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_ffn_up_backward": (_i, [_vp, _i32p, _i, _i64, _i, _i, _i, _vp, _vp, _vp]),
    "moe_wgrad_workspace_bytes": (_sz, [_i64, _i, _i, _i, _i]),
    "moe_ffn_wgrad": (_i, [_vp, _vp, _vp, _vp, _i32p, _i, _i64, _i, _i, _i, _fp, _fp, _vp, _sz,
                           _vp]),
    "moe_router_backward_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_router_backward": (_i, [_vp, _fp, _fp, _i, _i, _i, _i, _vp, _fp, _vp, _sz, _vp]),
    "moe_forward_fused": (_i, [_fp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i32p,
                               _fp, _i32p, _i32p, _i32p, _i32p, _i32p, _vp, _vp, _vp, _vp, _sz,
                               _vp]),
    "moe_forward_fused_reroute": (_i, [_fp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                       _i32p, _fp, _i32p, _i32p, _i32p, _i32p, _i32p, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
    "moe_forward_fused_fp8": (_i, [_fp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _fp, _vp,
                                   _fp, _i32p, _fp, _i32p, _i32p, _i32p, _i32p, _i32p, _vp, _vp,
                                   _vp, _vp, _sz, _vp]),
    "moe_forward_fused_fp8_list": (_i, [_fp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                        _vp, _vp, _i32p, _fp, _i32p, _i32p, _i32p, _i32p, _i32p,
                                        _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_set_fused_overlap": (_i, [_i]),
    "moe_forward_fused_list": (_i, [_fp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp,
                                    _i32p, _fp, _i32p, _i32p, _i32p, _i32p, _i32p, _vp, _vp, _vp,
                                    _vp, _sz, _vp]),
}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def lib():
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m routing_dispatch_expert_moe_amd.build` "
                "(the MoE path has no CPU fallback)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, where)
