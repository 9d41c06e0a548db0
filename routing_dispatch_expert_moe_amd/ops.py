"""Thin PyTorch binding of the C ABI: same names as include/moe.h.

Each function checks tensor placement, dtype and contiguity, allocates the
outputs the caller did not pass (torch is the allocator), and calls the
library on torch's current HIP stream.  No step of the MoE path runs here:
every computation happens in the library's kernels.
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import Optional, Sequence, Tuple

import torch

from . import _lib as L
from ._lib import check, lib

GATES = {
    "softmax_topk_renorm": L.MOE_GATE_SOFTMAX_TOPK_RENORM,
    "sigmoid_topk_norm": L.MOE_GATE_SIGMOID_TOPK_NORM,
}


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return L.MOE_F32
    if t == torch.bfloat16:
        return L.MOE_BF16
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _gate_code(gate) -> int:
    return GATES[gate] if isinstance(gate, str) else int(gate)


def moe_workspace_bytes(T: int, E: int, k: int, E_loc: int) -> int:
    return int(lib().moe_workspace_bytes(T, E, k, E_loc))


def moe_capacity(T: int, k: int, E: int, capacity_factor) -> int:
    """Per-expert capacity for a capacity factor (None = no limit -> -1)."""
    if capacity_factor is None:
        return -1
    q = Fraction(str(capacity_factor))
    c = int(lib().moe_capacity(T, k, E, q.numerator, q.denominator))
    if c < -1:
        raise ValueError("invalid capacity arguments")
    return c


def moe_max_rows(T: int, k: int, E_loc: int, capacity: int) -> int:
    return int(lib().moe_max_rows(T, k, E_loc, capacity))


_PLAN_NAMES = {0: "none", 1: "f32", 2: "stream", 3: "stream (operands of 4 GiB or more)",
               4: "wide", 5: "big_all", 6: "big_tail", 7: "big_ride"}


def moe_ffn_plan(half: str, max_rows: int, E_loc: int, d: int, f: int, dtype: str = "bf16",
                 cu_count: int = 256) -> str:
    """Name of the kernel plan moe_ffn_up (half='up') or moe_ffn_down
    (half='down') uses for these sizes (host-only query, no GPU)."""
    code = int(lib().moe_ffn_plan({"up": 0, "down": 1}[half], max_rows, E_loc, d, f,
                                  {"f32": L.MOE_F32, "bf16": L.MOE_BF16}[dtype], cu_count))
    if code < 0:
        raise ValueError("invalid arguments for moe_ffn_plan")
    return _PLAN_NAMES[code]


def alloc_workspace(T: int, E: int, k: int, E_loc: int, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(T, E, k, E_loc)
    if n == 0:
        raise ValueError("invalid sizes for the workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_pack_weights(w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
                     w13_packed: Optional[torch.Tensor] = None,
                     w2_packed: Optional[torch.Tensor] = None, stream=None):
    """w1, w3 [E_loc, d, f], w2 [E_loc, f, d] -> (w13 [E_loc, 2f, d], w2p [E_loc, d, f])."""
    E_loc, d, f = w1.shape
    if w13_packed is None:
        w13_packed = torch.empty((E_loc, 2 * f, d), dtype=w1.dtype, device=w1.device)
    if w2_packed is None:
        w2_packed = torch.empty((E_loc, d, f), dtype=w1.dtype, device=w1.device)
    check(lib().moe_pack_weights(_ptr(w1), _ptr(w3), _ptr(w2), E_loc, d, f, _dtype_code(w1.dtype),
                                 _ptr(w13_packed), _ptr(w2_packed), _stream(stream)),
          "moe_pack_weights")
    return w13_packed, w2_packed


def moe_router_logits(x: torch.Tensor, w_gate: torch.Tensor,
                      logits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, d = x.shape
    E = w_gate.shape[1]
    if x.dtype != torch.bfloat16 or w_gate.dtype != torch.float32:
        raise TypeError("router logits take bf16 x and an fp32 gate matrix")
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    check(lib().moe_router_logits(_ptr(x), _ptr(w_gate), T, d, E, _ptr(logits), _stream(stream)),
          "moe_router_logits")
    return logits


def moe_route(logits: torch.Tensor, k: int, gate, topk_idx: Optional[torch.Tensor] = None,
              topk_w: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be fp32")
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    check(lib().moe_route(_ptr(logits), T, E, k, _gate_code(gate), _ptr(topk_idx), _ptr(topk_w),
                          _stream(stream)), "moe_route")
    return topk_idx, topk_w


@dataclasses.dataclass
class DispatchPlan:
    """The per-batch routing plan (reused by the combine)."""
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_pair: torch.Tensor
    pair_pos: torch.Tensor
    n_kept: torch.Tensor
    x_perm: Optional[torch.Tensor]
    max_rows: int



def moe_route_reroute(logits: torch.Tensor, k: int, gate, capacity: int, ws: torch.Tensor,
                      topk_idx: Optional[torch.Tensor] = None,
                      topk_w: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k routing with capacity-overflow rerouting (see include/moe.h)."""
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be fp32")
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    check(lib().moe_route_reroute(_ptr(logits), T, E, k, _gate_code(gate), capacity,
                                  _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_route_reroute")
    return topk_idx, topk_w


def moe_route_reroute_noalloc(logits: torch.Tensor, k: int, gate, capacity: int,
                              topk_idx: Optional[torch.Tensor] = None,
                              topk_w: Optional[torch.Tensor] = None,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """moe_route_reroute with the library's fixed device scratch instead of a
    workspace (the C entry point allocates nothing; see include/moe.h)."""
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be fp32")
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    check(lib().moe_route_reroute_noalloc(_ptr(logits), T, E, k, _gate_code(gate), capacity,
                                          _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
          "moe_route_reroute_noalloc")
    return topk_idx, topk_w


def alloc_plan(T: int, E: int, k: int, E_loc: int, capacity: int, d: int, dtype,
               device="cuda") -> DispatchPlan:
    rows = moe_max_rows(T, k, E_loc, capacity)
    i32 = dict(dtype=torch.int32, device=device)
    return DispatchPlan(counts=torch.empty(E, **i32), offsets=torch.empty(E_loc + 1, **i32),
                        sorted_pair=torch.empty(max(rows, 1), **i32),
                        pair_pos=torch.empty(max(T * k, 1), **i32), n_kept=torch.empty(4, **i32),
                        x_perm=torch.empty((max(rows, 1), d), dtype=dtype, device=device),
                        max_rows=rows)


def moe_dispatch(topk_idx: torch.Tensor, E: int, capacity: int, e_begin: int, e_end: int,
                 x: Optional[torch.Tensor], ws: torch.Tensor, plan: Optional[DispatchPlan] = None,
                 d: Optional[int] = None, dtype=None, stream=None) -> DispatchPlan:
    T, k = topk_idx.shape
    if x is not None:
        d, dtype = x.shape[1], x.dtype
    d = d or 8
    dtype = dtype or torch.bfloat16
    if plan is None:
        plan = alloc_plan(T, E, k, e_end - e_begin, capacity, d, dtype, topk_idx.device)
    check(lib().moe_dispatch(_ptr(topk_idx), T, E, k, capacity, e_begin, e_end, _ptr(x), d,
                             _dtype_code(dtype), _ptr(plan.counts), _ptr(plan.offsets),
                             _ptr(plan.sorted_pair), _ptr(plan.pair_pos), _ptr(plan.n_kept),
                             _ptr(plan.x_perm) if x is not None else None, _ptr(ws), ws.numel(),
                             _stream(stream)), "moe_dispatch")
    return plan


def moe_ffn_up(x_perm, offsets, E_loc, max_rows, w13_packed, h=None, ws=None, stream=None):
    d = x_perm.shape[1]
    f = w13_packed.shape[1] // 2
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_ffn_up(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                           _dtype_code(x_perm.dtype), _ptr(w13_packed), _ptr(h), _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)), "moe_ffn_up")
    return h


def moe_ffn_down(h, offsets, E_loc, max_rows, w2_packed, y_perm=None, ws=None, stream=None):
    f = h.shape[1]
    d = w2_packed.shape[1]
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=h.dtype, device=h.device)
    check(lib().moe_ffn_down(_ptr(h), _ptr(offsets), E_loc, max_rows, d, f, _dtype_code(h.dtype),
                             _ptr(w2_packed), _ptr(y_perm), _ptr(ws),
                             ws.numel() if ws is not None else 0, _stream(stream)), "moe_ffn_down")
    return y_perm


def moe_expert_ffn(x_perm, offsets, E_loc, max_rows, w13_packed, w2_packed, h=None, y_perm=None,
                   ws=None, stream=None):
    d = x_perm.shape[1]
    f = w13_packed.shape[1] // 2
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_expert_ffn(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                               _dtype_code(x_perm.dtype), _ptr(w13_packed), _ptr(w2_packed),
                               _ptr(h), _ptr(y_perm), _ptr(ws), ws.numel() if ws is not None else 0,
                               _stream(stream)), "moe_expert_ffn")
    return h, y_perm


def weight_table(weights: Sequence[torch.Tensor]) -> torch.Tensor:
    """Device table (int64) of the data pointers of per-expert weight buffers,
    for the *_list calls; the buffers must stay alive while calls use it."""
    if not weights:
        raise ValueError("empty weight list")
    dev = weights[0].device
    for w in weights:
        if w.device != dev or not w.is_contiguous():
            raise ValueError("weight buffers must be contiguous tensors on one device")
    return torch.tensor([w.data_ptr() for w in weights], dtype=torch.int64, device=dev)


def moe_expert_ffn_list(x_perm, offsets, E_loc, max_rows, w13_table, w2_table, d, f, h=None,
                        y_perm=None, stream=None):
    """moe_expert_ffn over per-expert weight buffers (tables from weight_table)."""
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_expert_ffn_list(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                                    _dtype_code(x_perm.dtype), _ptr(w13_table), _ptr(w2_table),
                                    _ptr(h), _ptr(y_perm), _stream(stream)), "moe_expert_ffn_list")
    return h, y_perm


def moe_quantize_fp8(w_packed: torch.Tensor, q: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None, stream=None):
    """Packed bf16 weights [E, rows, K] -> (E4M3 codes uint8 [E, rows, K],
    fp32 scales [E, rows/128, K/128]); see moe_quantize_fp8 in include/moe.h."""
    E, R, K = w_packed.shape
    if q is None:
        q = torch.empty((E, R, K), dtype=torch.uint8, device=w_packed.device)
    if scales is None:
        scales = torch.empty((E, max(R // 128, 1), max(K // 128, 1)), dtype=torch.float32,
                             device=w_packed.device)
    check(lib().moe_quantize_fp8(_ptr(w_packed), E, R, K, _ptr(q), _ptr(scales), _stream(stream)),
          "moe_quantize_fp8")
    return q, scales


def moe_ffn_up_fp8(x_perm, offsets, E_loc, max_rows, w13_q, w13_s, h=None, stream=None):
    d = x_perm.shape[1]
    f = w13_q.shape[1] // 2
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_ffn_up_fp8(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f, _ptr(w13_q),
                               _ptr(w13_s), _ptr(h), _stream(stream)), "moe_ffn_up_fp8")
    return h


def moe_ffn_down_fp8(h, offsets, E_loc, max_rows, w2_q, w2_s, y_perm=None, stream=None):
    f = h.shape[1]
    d = w2_q.shape[1]
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=h.dtype, device=h.device)
    check(lib().moe_ffn_down_fp8(_ptr(h), _ptr(offsets), E_loc, max_rows, d, f, _ptr(w2_q),
                                 _ptr(w2_s), _ptr(y_perm), _stream(stream)), "moe_ffn_down_fp8")
    return y_perm


def moe_expert_ffn_fp8(x_perm, offsets, E_loc, max_rows, w13_q, w13_s, w2_q, w2_s, h=None,
                       y_perm=None, stream=None):
    d = x_perm.shape[1]
    f = w13_q.shape[1] // 2
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_expert_ffn_fp8(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                                   _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), _ptr(h),
                                   _ptr(y_perm), _stream(stream)), "moe_expert_ffn_fp8")
    return h, y_perm


def moe_ffn_up_fp8_list(x_perm, offsets, E_loc, max_rows, q_table, s_table, f, h=None,
                        stream=None):
    """moe_ffn_up_fp8 over per-expert code and scale buffers (tables from
    weight_table; each buffer one expert of moe_quantize_fp8's outputs)."""
    d = x_perm.shape[1]
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_ffn_up_fp8_list(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                                    _ptr(q_table), _ptr(s_table), _ptr(h), _stream(stream)),
          "moe_ffn_up_fp8_list")
    return h


def moe_ffn_down_fp8_list(h, offsets, E_loc, max_rows, q_table, s_table, d, y_perm=None,
                          stream=None):
    """moe_ffn_down_fp8 over per-expert code and scale buffers."""
    f = h.shape[1]
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=h.dtype, device=h.device)
    check(lib().moe_ffn_down_fp8_list(_ptr(h), _ptr(offsets), E_loc, max_rows, d, f,
                                      _ptr(q_table), _ptr(s_table), _ptr(y_perm),
                                      _stream(stream)), "moe_ffn_down_fp8_list")
    return y_perm


def moe_expert_ffn_fp8_list(x_perm, offsets, E_loc, max_rows, w13_q_table, w13_s_table,
                            w2_q_table, w2_s_table, f, h=None, y_perm=None, stream=None):
    """moe_expert_ffn_fp8 over per-expert code and scale buffers."""
    d = x_perm.shape[1]
    if h is None:
        h = torch.empty((max(max_rows, 1), f), dtype=x_perm.dtype, device=x_perm.device)
    if y_perm is None:
        y_perm = torch.empty((max(max_rows, 1), d), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_expert_ffn_fp8_list(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                                        _ptr(w13_q_table), _ptr(w13_s_table), _ptr(w2_q_table),
                                        _ptr(w2_s_table), _ptr(h), _ptr(y_perm),
                                        _stream(stream)), "moe_expert_ffn_fp8_list")
    return h, y_perm


def moe_combine(y_perm, pair_pos, topk_w, y=None, stream=None, T=None, k=None):
    """y [T, d]; topk_w None: unit weights (then pass T and k)."""
    if topk_w is not None:
        T, k = topk_w.shape
    d = y_perm.shape[1]
    if y is None:
        y = torch.empty((T, d), dtype=y_perm.dtype, device=y_perm.device)
    check(lib().moe_combine(_ptr(y_perm), _ptr(pair_pos), _ptr(topk_w), T, k, d,
                            _dtype_code(y_perm.dtype), _ptr(y), _stream(stream)), "moe_combine")
    return y


def moe_check_error(ws, stream=None) -> int:
    """Synchronise and return the device-side status (0 = OK) without raising."""
    return int(lib().moe_check_error(_ptr(ws), _stream(stream)))


OVERLAP_MODES = {"never": L.MOE_OVERLAP_NEVER, "auto": L.MOE_OVERLAP_AUTO,
                 "always": L.MOE_OVERLAP_ALWAYS}


def moe_set_fused_overlap(mode: str = "auto"):
    """How the fused launch orders its two GEMM phases from now on in this
    process: "never" (a device-wide barrier), "auto" (per-expert waits where
    they measured faster) or "always" (per-expert waits wherever possible)."""
    check(lib().moe_set_fused_overlap(OVERLAP_MODES[mode]), "moe_set_fused_overlap")


def moe_forward_fused(logits, x, k, gate, capacity, e_begin, e_end, w13_packed, w2_packed, ws,
                      plan: DispatchPlan, topk_idx, topk_w, h, y_perm, y, stream=None,
                      reroute: bool = False):
    """The whole layer (route, dispatch, expert FFN, combine) in one persistent launch.

    Every output buffer is caller-provided (the layer preallocates them); they
    receive the same bits as the four separate calls, except that no permuted
    copy of x is written (the first GEMM reads x through the permutation)."""
    T, E = logits.shape
    d = x.shape[1]
    f = w13_packed.shape[1] // 2
    fn = lib().moe_forward_fused_reroute if reroute else lib().moe_forward_fused
    check(fn(_ptr(logits), _ptr(x), T, E, k, _gate_code(gate), capacity, e_begin, e_end, d, f,
             _dtype_code(x.dtype), _ptr(w13_packed), _ptr(w2_packed), _ptr(topk_idx), _ptr(topk_w),
             _ptr(plan.counts), _ptr(plan.offsets), _ptr(plan.sorted_pair), _ptr(plan.pair_pos),
             _ptr(plan.n_kept), _ptr(h), _ptr(y_perm), _ptr(y), _ptr(ws), ws.numel(),
             _stream(stream)),
          "moe_forward_fused_reroute" if reroute else "moe_forward_fused")
    return y


def moe_forward_fused_list(logits, x, k, gate, capacity, e_begin, e_end, w13_table, w2_table,
                           f, ws, plan: DispatchPlan, topk_idx, topk_w, h, y_perm, y,
                           stream=None):
    """moe_forward_fused over per-expert weight buffers (tables from
    weight_table; each buffer one expert of moe_pack_weights' layout)."""
    T, E = logits.shape
    d = x.shape[1]
    check(lib().moe_forward_fused_list(
        _ptr(logits), _ptr(x), T, E, k, _gate_code(gate), capacity, e_begin, e_end, d, f,
        _dtype_code(x.dtype), _ptr(w13_table), _ptr(w2_table), _ptr(topk_idx), _ptr(topk_w),
        _ptr(plan.counts), _ptr(plan.offsets), _ptr(plan.sorted_pair), _ptr(plan.pair_pos),
        _ptr(plan.n_kept), _ptr(h), _ptr(y_perm), _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_forward_fused_list")
    return y


def moe_forward_fused_fp8_list(logits, x, k, gate, capacity, e_begin, e_end, w13_q_table,
                               w13_s_table, w2_q_table, w2_s_table, f, ws, plan: DispatchPlan,
                               topk_idx, topk_w, h, y_perm, y, stream=None):
    """moe_forward_fused_fp8 over per-expert code and scale buffers (tables
    from weight_table; each buffer one expert of moe_quantize_fp8's outputs)."""
    T, E = logits.shape
    d = x.shape[1]
    check(lib().moe_forward_fused_fp8_list(
        _ptr(logits), _ptr(x), T, E, k, _gate_code(gate), capacity, e_begin, e_end, d, f,
        _ptr(w13_q_table), _ptr(w13_s_table), _ptr(w2_q_table), _ptr(w2_s_table), _ptr(topk_idx),
        _ptr(topk_w), _ptr(plan.counts), _ptr(plan.offsets), _ptr(plan.sorted_pair),
        _ptr(plan.pair_pos), _ptr(plan.n_kept), _ptr(h), _ptr(y_perm), _ptr(y), _ptr(ws),
        ws.numel(), _stream(stream)), "moe_forward_fused_fp8_list")
    return y


def moe_forward_fused_fp8(logits, x, k, gate, capacity, e_begin, e_end, w13_q, w13_s, w2_q, w2_s,
                          ws, plan: DispatchPlan, topk_idx, topk_w, h, y_perm, y, stream=None):
    """moe_forward_fused with FP8 expert weights (codes and block scales from
    moe_quantize_fp8); bf16 activations, caller-provided outputs."""
    T, E = logits.shape
    d = x.shape[1]
    f = w13_q.shape[1] // 2
    check(lib().moe_forward_fused_fp8(
        _ptr(logits), _ptr(x), T, E, k, _gate_code(gate), capacity, e_begin, e_end, d, f,
        _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), _ptr(topk_idx), _ptr(topk_w),
        _ptr(plan.counts), _ptr(plan.offsets), _ptr(plan.sorted_pair), _ptr(plan.pair_pos),
        _ptr(plan.n_kept), _ptr(h), _ptr(y_perm), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
        "moe_forward_fused_fp8")
    return y


# --------------------------------------------------------------------------
# backward pass
# --------------------------------------------------------------------------
def moe_ffn_up_train(x_perm, offsets, E_loc, max_rows, w13_packed, h=None, ab=None, stream=None):
    """moe_ffn_up that also keeps the pre-activations ab [rows, 2f] (a then g)."""
    d = x_perm.shape[1]
    f = w13_packed.shape[1] // 2
    rows = max(max_rows, 1)
    if h is None:
        h = torch.empty((rows, f), dtype=x_perm.dtype, device=x_perm.device)
    if ab is None:
        ab = torch.empty((rows, 2 * f), dtype=x_perm.dtype, device=x_perm.device)
    check(lib().moe_ffn_up_train(_ptr(x_perm), _ptr(offsets), E_loc, max_rows, d, f,
                                 _dtype_code(x_perm.dtype), _ptr(w13_packed), _ptr(h), _ptr(ab),
                                 _stream(stream)), "moe_ffn_up_train")
    return h, ab


def moe_pack_weights_backward(w1: torch.Tensor, w3: torch.Tensor,
                              w13_t: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """w1, w3 [E_loc, d, f] -> w13_t [E_loc, d, 2f] (row c = W1[c] then W3[c])."""
    E_loc, d, f = w1.shape
    if w13_t is None:
        w13_t = torch.empty((E_loc, d, 2 * f), dtype=w1.dtype, device=w1.device)
    check(lib().moe_pack_weights_backward(_ptr(w1), _ptr(w3), E_loc, d, f, _dtype_code(w1.dtype),
                                          _ptr(w13_t), _stream(stream)),
          "moe_pack_weights_backward")
    return w13_t


def moe_combine_backward(dy, y_perm, pair_pos, topk_w, do_perm=None, dgate=None, stream=None):
    """(do_perm [rows, d], dgate [T, k] fp32) from dy [T, d] through the forward's plan."""
    T, k = topk_w.shape
    d = dy.shape[1]
    if do_perm is None:
        do_perm = torch.empty((max(y_perm.shape[0], 1), d), dtype=dy.dtype, device=dy.device)
    if dgate is None:
        dgate = torch.empty((T, k), dtype=torch.float32, device=dy.device)
    check(lib().moe_combine_backward(_ptr(dy), _ptr(y_perm), _ptr(pair_pos), _ptr(topk_w), T, k, d,
                                     _dtype_code(dy.dtype), _ptr(do_perm), _ptr(dgate),
                                     _stream(stream)), "moe_combine_backward")
    return do_perm, dgate


def moe_gate_backward(logits, topk_idx, dgate, gate, dlogits=None, stream=None):
    """dlogits [T, E] fp32 (zero outside the chosen experts)."""
    T, E = logits.shape
    k = topk_idx.shape[1]
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=logits.device)
    check(lib().moe_gate_backward(_ptr(logits), _ptr(topk_idx), _ptr(dgate), T, E, k,
                                  _gate_code(gate), _ptr(dlogits), _stream(stream)),
          "moe_gate_backward")
    return dlogits


def moe_ffn_down_backward(do_perm, offsets, E_loc, max_rows, w2_t, ab, dh=None, dab=None,
                          stream=None):
    """(dh [rows, f], dab [rows, 2f]); w2_t = W2 in its logical layout [E_loc, f, d]."""
    d = do_perm.shape[1]
    f = w2_t.shape[1]
    rows = max(max_rows, 1)
    if dh is None:
        dh = torch.empty((rows, f), dtype=do_perm.dtype, device=do_perm.device)
    if dab is None:
        dab = torch.empty((rows, 2 * f), dtype=do_perm.dtype, device=do_perm.device)
    check(lib().moe_ffn_down_backward(_ptr(do_perm), _ptr(offsets), E_loc, max_rows, d, f,
                                      _dtype_code(do_perm.dtype), _ptr(w2_t), _ptr(ab), _ptr(dh),
                                      _ptr(dab), _stream(stream)), "moe_ffn_down_backward")
    return dh, dab


def moe_ffn_up_backward(dab, offsets, E_loc, max_rows, w13_t, dx_perm=None, stream=None):
    """dx_perm [rows, d] = dab . [W1 | W3]^T per expert segment."""
    d = w13_t.shape[1]
    f = dab.shape[1] // 2
    if dx_perm is None:
        dx_perm = torch.empty((max(max_rows, 1), d), dtype=dab.dtype, device=dab.device)
    check(lib().moe_ffn_up_backward(_ptr(dab), _ptr(offsets), E_loc, max_rows, d, f,
                                    _dtype_code(dab.dtype), _ptr(w13_t), _ptr(dx_perm),
                                    _stream(stream)), "moe_ffn_up_backward")
    return dx_perm


def moe_wgrad_workspace_bytes(max_rows: int, E_loc: int, d: int, f: int, dtype) -> int:
    return int(lib().moe_wgrad_workspace_bytes(max_rows, E_loc, d, f, _dtype_code(dtype)))


def moe_ffn_wgrad(x_perm, h, do_perm, dab, offsets, E_loc, max_rows, dw13=None, dw2=None, ws=None,
                  stream=None):
    """fp32 weight gradients in the packed layouts: dw13 [E_loc, 2f, d], dw2 [E_loc, d, f]."""
    d = x_perm.shape[1]
    f = h.shape[1]
    dev = x_perm.device
    if dw13 is None:
        dw13 = torch.empty((E_loc, 2 * f, d), dtype=torch.float32, device=dev)
    if dw2 is None:
        dw2 = torch.empty((E_loc, d, f), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(moe_wgrad_workspace_bytes(max_rows, E_loc, d, f, x_perm.dtype),
                         dtype=torch.uint8, device=dev)
    check(lib().moe_ffn_wgrad(_ptr(x_perm), _ptr(h), _ptr(do_perm), _ptr(dab), _ptr(offsets), E_loc,
                              max_rows, d, f, _dtype_code(x_perm.dtype), _ptr(dw13), _ptr(dw2),
                              _ptr(ws), ws.numel(), _stream(stream)), "moe_ffn_wgrad")
    return dw13, dw2


def moe_router_backward_workspace_bytes(T: int, d: int, E: int) -> int:
    return int(lib().moe_router_backward_workspace_bytes(T, d, E))


def moe_router_backward(x, w_gate, dlogits, dx, dw_gate=None, ws=None, stream=None):
    """dx += dlogits . W_g^T (in place), and dW_g [d, E] fp32 = x^T . dlogits."""
    T, d = x.shape
    E = w_gate.shape[1]
    if dw_gate is None:
        dw_gate = torch.empty((d, E), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(moe_router_backward_workspace_bytes(T, d, E), 16), dtype=torch.uint8,
                         device=x.device)
    check(lib().moe_router_backward(_ptr(x), _ptr(w_gate), _ptr(dlogits), T, d, E,
                                    _dtype_code(x.dtype), _ptr(dx), _ptr(dw_gate), _ptr(ws),
                                    ws.numel(), _stream(stream)), "moe_router_backward")
    return dx, dw_gate
