"""Helpers for the GPU parity tests: move seeded workloads onto the GPU, run the
library through its C ABI, bring results back as numpy.  (No arithmetic of
the method lives here.)"""
from __future__ import annotations

import sys

import numpy as np
import torch

import routing_dispatch_expert_moe_amd as M
from oracle import moe_oracle as O

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def t_in(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Host array (fp32 values or bf16 bits) -> device tensor of the matching torch dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def t_out(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host numpy (bf16 as uint16 bits, others as is)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return O.widen(t_out(t), dtype)


def packed_weights(wl, chunk: int = 16, keep_host: bool = False):
    """Generate the workload's local experts, upload and pack them chunk by chunk.

    Returns (w13 [E_loc, 2f, d], w2p [E_loc, d, f], host) where host is the list
    of per-expert (W1, W3, W2) host arrays if keep_host else None.
    """
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    w13 = torch.empty((wl.E_loc, 2 * wl.f, wl.d), dtype=tdt, device=DEV)
    w2p = torch.empty((wl.E_loc, wl.d, wl.f), dtype=tdt, device=DEV)
    host = [] if keep_host else None
    for c0 in range(0, wl.E_loc, chunk):
        ids = list(range(wl.e_begin + c0, wl.e_begin + min(wl.E_loc, c0 + chunk)))
        a, b, c = wl.stacked_weights(ids)
        if keep_host:
            host.extend(zip(a, b, c))
        n = len(ids)
        M.moe_pack_weights(t_in(a, wl.dtype), t_in(b, wl.dtype), t_in(c, wl.dtype),
                           w13[c0:c0 + n], w2p[c0:c0 + n])
    torch.cuda.synchronize()
    return w13, w2p, host


def weights_fn(wl, host=None):
    """Float64 weights of local expert i for the oracle (from the host copy, else regenerated)."""
    def get(i):
        if host is not None:
            w1, w3, w2 = host[i]
        else:
            w1, w3, w2 = wl.expert_weights(wl.e_begin + i)
        return O.widen(w1, wl.dtype), O.widen(w3, wl.dtype), O.widen(w2, wl.dtype)
    return get


def capacity_of(wl) -> int:
    """The library's capacity for the workload, checked against the oracle's rule."""
    c = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    assert c == O.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    return c


def layer_for(wl, w13, w2p, capacity=None, reroute=False) -> M.MoELayer:
    C = capacity_of(wl) if capacity is None else capacity
    return M.MoELayer(w13, w2p, E=wl.E, k=wl.k, gate=wl.gate, T=wl.T, capacity=C,
                      e_begin=wl.e_begin, e_end=wl.e_end, reroute=reroute)


def fused_matches_unfused(wl, w13, w2p, layer, x, logits, capacity=None):
    """Run moe_forward_fused (or its rerouting form, as `layer` routes) into a
    second layer's buffers and check that every output carries the same bits as
    the separate calls in `layer`."""
    fl = layer_for(wl, w13, w2p, capacity=capacity, reroute=layer.reroute)
    fl.forward_fused(x, logits)
    assert M.moe_check_error(fl.ws) == 0
    a, b = layer.outputs(), fl.outputs()
    n = int(t_out(a["n_kept"])[0])
    assert int(t_out(b["n_kept"])[0]) == n
    for key in ("topk_idx", "topk_w", "counts", "offsets", "pair_pos", "y"):
        assert np.array_equal(t_out(a[key]), t_out(b[key])), key
    for key in ("sorted_pair", "h", "y_perm"):
        assert np.array_equal(t_out(a[key])[:n], t_out(b[key])[:n]), key
    # a second fused call on the same workspace (barrier words re-armed) is identical
    y1 = t_out(fl.y).copy()
    fl.forward_fused(x, logits)
    assert M.moe_check_error(fl.ws) == 0
    assert np.array_equal(t_out(fl.y), y1)
    barrier_order_matches(fl, x, logits, y1)
    return fl


def barrier_order_matches(fl, x, logits, y_ref):
    """The fused call with its GEMM phases separated by a device-wide barrier
    and with per-expert waits (both forced, whatever the automatic choice)
    gives the same bits, and so does a call whose workspace is one byte short
    of the readiness counters (always the barrier)."""
    try:
        for mode in ("never", "always"):
            M.moe_set_fused_overlap(mode)
            fl.forward_fused(x, logits)
            assert M.moe_check_error(fl.ws) == 0
            assert np.array_equal(t_out(fl.y), y_ref), mode
        full = fl.ws
        fl.ws = full[:full.numel() - 1]
        try:
            fl.forward_fused(x, logits)
            assert M.moe_check_error(full) == 0
            assert np.array_equal(t_out(fl.y), y_ref), "short workspace"
        finally:
            fl.ws = full
    finally:
        M.moe_set_fused_overlap("auto")
