"""One MoE layer on one GPU through the C ABI, with every buffer preallocated.

forward() enqueues, on the current HIP stream:
  [moe_router_logits] -> moe_route -> moe_dispatch -> moe_ffn_up -> moe_ffn_down -> moe_combine
and never synchronises with the host (row counts stay on the device).
forward_fused() enqueues the same path as one moe_forward_fused launch.
For training, enable_training() adds the backward operands and buffers;
forward_train() keeps the SwiGLU pre-activations, and backward(dy) enqueues
  moe_combine_backward -> moe_gate_backward -> [moe_router_backward]
  moe_ffn_down_backward -> moe_ffn_up_backward -> moe_combine (unit weights)
  moe_ffn_wgrad
reusing the forward's plan and saved tensors.
With FP8 weights (uint8 E4M3 codes from moe_quantize_fp8 plus their block
scales) the FFN steps run moe_ffn_up_fp8 / moe_ffn_down_fp8 on bf16
activations; the fused launch takes bf16 or fp32 weights only.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import ops


class MoELayer:
    def __init__(self, w13_packed: torch.Tensor, w2_packed: torch.Tensor, *, E: int, k: int,
                 gate, T: int, capacity: int = -1, e_begin: int = 0, e_end: Optional[int] = None,
                 w13_scale: Optional[torch.Tensor] = None, w2_scale: Optional[torch.Tensor] = None,
                 reroute: bool = False):
        self.w13, self.w2 = w13_packed, w2_packed
        self.fp8 = w13_packed.dtype == torch.uint8
        if self.fp8 and (w13_scale is None or w2_scale is None):
            raise ValueError("FP8 weights need their block scales")
        self.w13_scale, self.w2_scale = w13_scale, w2_scale
        # route with capacity-overflow rerouting (moe_route_reroute) instead of plain top-k
        self.reroute = reroute
        self.E, self.k, self.gate, self.T = E, k, gate, T
        self.capacity = capacity
        self.e_begin = e_begin
        self.e_end = E if e_end is None else e_end
        self.E_loc = self.e_end - self.e_begin
        self.d = w13_packed.shape[2]
        self.f = w13_packed.shape[1] // 2
        self.dtype = torch.bfloat16 if self.fp8 else w13_packed.dtype
        dev = w13_packed.device
        if w13_packed.shape[0] != self.E_loc:
            raise ValueError("packed weights must hold exactly the local experts")
        self.ws = ops.alloc_workspace(T, E, k, self.E_loc, dev)
        self.plan = ops.alloc_plan(T, E, k, self.E_loc, capacity, self.d, self.dtype, dev)
        rows = max(self.plan.max_rows, 1)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.h = torch.empty((rows, self.f), dtype=self.dtype, device=dev)
        self.y_perm = torch.empty((rows, self.d), dtype=self.dtype, device=dev)
        self.y = torch.empty((T, self.d), dtype=self.dtype, device=dev)

    # individual steps (the benchmark brackets each with events)
    def router(self, x, w_gate):
        return ops.moe_router_logits(x, w_gate, self.logits)

    def route(self, logits):
        if self.reroute:
            return ops.moe_route_reroute(logits, self.k, self.gate, self.capacity, self.ws,
                                         self.topk_idx, self.topk_w)
        return ops.moe_route(logits, self.k, self.gate, self.topk_idx, self.topk_w)

    def dispatch(self, x):
        return ops.moe_dispatch(self.topk_idx, self.E, self.capacity, self.e_begin, self.e_end, x,
                                self.ws, self.plan)

    def ffn_up(self):
        if self.fp8:
            return ops.moe_ffn_up_fp8(self.plan.x_perm, self.plan.offsets, self.E_loc,
                                      self.plan.max_rows, self.w13, self.w13_scale, self.h)
        return ops.moe_ffn_up(self.plan.x_perm, self.plan.offsets, self.E_loc, self.plan.max_rows,
                              self.w13, self.h, self.ws)

    def ffn_down(self):
        if self.fp8:
            return ops.moe_ffn_down_fp8(self.h, self.plan.offsets, self.E_loc, self.plan.max_rows,
                                        self.w2, self.w2_scale, self.y_perm)
        return ops.moe_ffn_down(self.h, self.plan.offsets, self.E_loc, self.plan.max_rows, self.w2,
                                self.y_perm, self.ws)

    def combine(self):
        return ops.moe_combine(self.y_perm, self.plan.pair_pos, self.topk_w, self.y)

    def forward(self, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
                w_gate: Optional[torch.Tensor] = None) -> torch.Tensor:
        if x.shape[0] != self.T:
            raise ValueError(f"layer was sized for T={self.T}, got {x.shape[0]}")
        if logits is None:
            if w_gate is None:
                raise ValueError("need logits or a gate matrix")
            logits = self.router(x, w_gate)
        self.route(logits)
        self.dispatch(x)
        self.ffn_up()
        self.ffn_down()
        self.combine()
        return self.y

    def forward_fused(self, x: torch.Tensor, logits: torch.Tensor) -> torch.Tensor:
        """route -> dispatch -> expert FFN -> combine as one persistent launch."""
        if x.shape[0] != self.T:
            raise ValueError(f"layer was sized for T={self.T}, got {x.shape[0]}")
        if self.fp8:
            if self.reroute:
                raise NotImplementedError("the fused launch with FP8 weights routes without rerouting")
            return ops.moe_forward_fused_fp8(logits, x, self.k, self.gate, self.capacity,
                                             self.e_begin, self.e_end, self.w13, self.w13_scale,
                                             self.w2, self.w2_scale, self.ws, self.plan,
                                             self.topk_idx, self.topk_w, self.h, self.y_perm,
                                             self.y)
        return ops.moe_forward_fused(logits, x, self.k, self.gate, self.capacity, self.e_begin,
                                     self.e_end, self.w13, self.w2, self.ws, self.plan,
                                     self.topk_idx, self.topk_w, self.h, self.y_perm, self.y,
                                     reroute=self.reroute)

    # ---------------------------------------------------------------- training
    def enable_training(self, w13_t: torch.Tensor, w2_t: torch.Tensor) -> None:
        """w13_t [E_loc, d, 2f] (moe_pack_weights_backward), w2_t = W2 [E_loc, f, d]."""
        if self.fp8:
            raise NotImplementedError("training takes bf16 / fp32 weights")
        self.w13_t, self.w2_t = w13_t, w2_t
        dev, dt = self.w13.device, self.dtype
        rows = max(self.plan.max_rows, 1)
        self.ab = torch.empty((rows, 2 * self.f), dtype=dt, device=dev)
        self.do_perm = torch.empty((rows, self.d), dtype=dt, device=dev)
        self.dgate = torch.empty((self.T, self.k), dtype=torch.float32, device=dev)
        self.dlogits = torch.empty((self.T, self.E), dtype=torch.float32, device=dev)
        self.dh = torch.empty((rows, self.f), dtype=dt, device=dev)
        self.dab = torch.empty((rows, 2 * self.f), dtype=dt, device=dev)
        self.dx_perm = torch.empty((rows, self.d), dtype=dt, device=dev)
        self.dx = torch.empty((self.T, self.d), dtype=dt, device=dev)
        self.dw13 = torch.empty((self.E_loc, 2 * self.f, self.d), dtype=torch.float32, device=dev)
        self.dw2 = torch.empty((self.E_loc, self.d, self.f), dtype=torch.float32, device=dev)
        self.wgrad_ws = torch.empty(max(ops.moe_wgrad_workspace_bytes(self.plan.max_rows, self.E_loc,
                                                                      self.d, self.f, dt), 16),
                                    dtype=torch.uint8, device=dev)
        self.dw_gate = None
        self.router_ws = None

    def ffn_up_train(self):
        return ops.moe_ffn_up_train(self.plan.x_perm, self.plan.offsets, self.E_loc,
                                    self.plan.max_rows, self.w13, self.h, self.ab)

    def forward_train(self, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
                      w_gate: Optional[torch.Tensor] = None) -> torch.Tensor:
        if logits is None:
            if w_gate is None:
                raise ValueError("need logits or a gate matrix")
            logits = self.router(x, w_gate)
        self.route(logits)
        self.dispatch(x)
        self.ffn_up_train()
        self.ffn_down()
        self.combine()
        return self.y

    def combine_backward(self, dy):
        return ops.moe_combine_backward(dy, self.y_perm, self.plan.pair_pos, self.topk_w,
                                        self.do_perm, self.dgate)

    def gate_backward(self, logits):
        return ops.moe_gate_backward(logits, self.topk_idx, self.dgate, self.gate, self.dlogits)

    def ffn_down_backward(self):
        return ops.moe_ffn_down_backward(self.do_perm, self.plan.offsets, self.E_loc,
                                         self.plan.max_rows, self.w2_t, self.ab, self.dh, self.dab)

    def ffn_up_backward(self):
        return ops.moe_ffn_up_backward(self.dab, self.plan.offsets, self.E_loc, self.plan.max_rows,
                                       self.w13_t, self.dx_perm)

    def combine_dx(self):
        return ops.moe_combine(self.dx_perm, self.plan.pair_pos, None, self.dx, T=self.T, k=self.k)

    def router_backward(self, x, w_gate):
        if self.dw_gate is None:
            self.dw_gate = torch.empty((self.d, self.E), dtype=torch.float32, device=x.device)
            self.router_ws = torch.empty(max(ops.moe_router_backward_workspace_bytes(self.T, self.d,
                                                                                     self.E), 16),
                                         dtype=torch.uint8, device=x.device)
        return ops.moe_router_backward(x, w_gate, self.dlogits, self.dx, self.dw_gate,
                                       self.router_ws)

    def wgrad(self):
        return ops.moe_ffn_wgrad(self.plan.x_perm, self.h, self.do_perm, self.dab,
                                 self.plan.offsets, self.E_loc, self.plan.max_rows, self.dw13,
                                 self.dw2, self.wgrad_ws)

    def backward(self, dy: torch.Tensor, logits: torch.Tensor, x: Optional[torch.Tensor] = None,
                 w_gate: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
        """Gradients of the last forward_train: dx, dlogits, dw13, dw2 (packed
        layouts, fp32), and dw_gate when the router ran (pass x and w_gate)."""
        self.combine_backward(dy)
        self.gate_backward(logits)
        self.ffn_down_backward()
        self.ffn_up_backward()
        self.combine_dx()
        if w_gate is not None:
            self.router_backward(x, w_gate)
        self.wgrad()
        out = dict(dx=self.dx, dlogits=self.dlogits, dgate=self.dgate, dw13=self.dw13,
                   dw2=self.dw2)
        if w_gate is not None:
            out["dw_gate"] = self.dw_gate
        return out

    def outputs(self) -> Dict[str, torch.Tensor]:
        p = self.plan
        return dict(logits=self.logits, topk_idx=self.topk_idx, topk_w=self.topk_w,
                    counts=p.counts, offsets=p.offsets, sorted_pair=p.sorted_pair,
                    pair_pos=p.pair_pos, n_kept=p.n_kept, x_perm=p.x_perm, h=self.h,
                    y_perm=self.y_perm, y=self.y)
