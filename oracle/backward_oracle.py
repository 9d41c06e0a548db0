"""CPU oracle of the MoE layer's backward pass: exact gradients in float64.

TEST INFRASTRUCTURE ONLY.  Like moe_oracle, this module is the plain reference
the GPU library is checked against; only the test suite, the package smoke
check and the CPU-baseline leg of the benchmark may import it, and it shares
no code, table or helper with the library.

Source: NCCL EP page ("NCCL EP架构解析"), §3.2 (training adaptation): the
backward step reuses the routing handle made by the forward step; the output
gradient is dispatched to the experts through it, the experts run their
backward, and the input gradients are combined through the same handle.  The
page gives no formulas; what is computed is the derivative of the forward
layer as moe_oracle defines it.  Readings (each also listed in the design
notes):

  R27 The backward computes the exact gradient of y = layer(x, logits,
      weights) at the given point with the routing decisions held fixed: the
      top-k sets, the capacity drops and the local/remote split are piecewise
      constant in the inputs, so their derivative is zero; gradients flow
      through the gate values, the expert FFNs and the router product.
  R28 The forward's plan (sorted_pair, offsets, pair_pos) is reused: the
      output gradient of pair (t, j) with a local row r is w[t, j] * dy[t] at
      row r; pairs without a local row (dropped or remote) get no row, and
      their gate gradient is 0 on this rank (remote gate gradients come from
      the rank that holds the expert).
  R29 Gradients: dx[t] = sum over t's local rows of the FFN input gradient
      (+ the router term dlogits[t] . W_g^T when the router runs); per local
      expert dW1, dW3 [d, f] and dW2 [f, d] in the x.W orientation;
      dlogits [T, E] is zero outside each token's chosen experts; the router
      weight gradient is x^T . dlogits.

Pins: tests/test_oracle_backward.py (central finite differences of
moe_oracle's own forward building blocks with Richardson extrapolation,
closed forms: softmax shift invariance, identical experts, W2 = 0, linearity;
planted mistakes are caught).
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

from . import moe_oracle as O


def gate_backward(logits_f32: np.ndarray, topk_idx: np.ndarray, dgate: np.ndarray,
                  gate: str) -> np.ndarray:
    """dlogits [T, E] from the gate-weight gradient dgate [T, k].

    softmax over the chosen: dl_j = w_j (dg_j - sum_i w_i dg_i);
    sigmoid normalised: w_j = s_j / S, dl_j = s_j (1 - s_j) (dg_j - sum_i w_i dg_i) / S.
    Experts outside the chosen k get 0 (R27).
    """
    l64 = (np.asarray(logits_f32, np.float32) + np.float32(0.0)).astype(np.float64)
    idx = np.asarray(topk_idx, np.int64)
    sel = np.take_along_axis(l64, idx, axis=-1)
    dg = np.asarray(dgate, np.float64)
    w = O.gate_values(sel, gate)
    centred = dg - np.sum(w * dg, axis=1, keepdims=True)
    if gate == O.GATE_SOFTMAX:
        dsel = w * centred
    elif gate == O.GATE_SIGMOID:
        s = 1.0 / (1.0 + np.exp(-sel))
        dsel = s * (1.0 - s) * centred / np.sum(s, axis=1, keepdims=True)
    else:
        raise ValueError(gate)
    out = np.zeros_like(l64)
    np.put_along_axis(out, idx, dsel, axis=-1)
    return out


def combine_backward(dy64: np.ndarray, y_perm64: np.ndarray, pair_pos: np.ndarray,
                     topk_w: np.ndarray, n_rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """Backward of y[t] = sum_j w[t, j] y_perm[pair_pos[t, j]] (R28).

    Returns (do_perm [n_rows, d]: row r of pair (t, j) holds w[t, j] dy[t];
    dgate [T, k]: dy[t] . y_perm[row], 0 for pairs without a local row).
    """
    w = np.asarray(topk_w, np.float64)
    T, k = w.shape
    dy = np.asarray(dy64, np.float64)
    pp = np.asarray(pair_pos).reshape(T, k)
    do = np.zeros((n_rows, dy.shape[1]), np.float64)
    dgate = np.zeros((T, k), np.float64)
    for j in range(k):
        rows = pp[:, j]
        have = rows >= 0
        do[rows[have]] = w[have, j:j + 1] * dy[have]
        dgate[have, j] = np.sum(dy[have] * y_perm64[rows[have]], axis=1)
    return do, dgate


def swiglu_backward(a: np.ndarray, g: np.ndarray, dh: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """h = silu(a) * g: (da, dg) with silu'(a) = s (1 + a (1 - s)), s = sigmoid(a)."""
    s = 1.0 / (1.0 + np.exp(-a))
    da = dh * g * s * (1.0 + a * (1.0 - s))
    dg = dh * a * s
    return da, dg


def expert_ffn_backward(x_perm64: np.ndarray, offsets: np.ndarray,
                        weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]],
                        do_perm64: np.ndarray) -> Dict[str, object]:
    """Backward of each local expert's SwiGLU FFN over its row segment.

    Returns dx_perm [n, d] and per local expert i the gradients dW1[i], dW3[i]
    [d, f] and dW2[i] [f, d] (zero for an expert with no rows), plus the
    intermediates a, g, h, dh [n, f] (float64).
    """
    off = np.asarray(offsets, np.int64)
    n = int(off[-1])
    d = x_perm64.shape[1]
    dx = np.zeros((n, d), np.float64)
    dW1: List[np.ndarray] = []
    dW3: List[np.ndarray] = []
    dW2: List[np.ndarray] = []
    inter = {}
    for i in range(len(off) - 1):
        w1, w3, w2 = weights(i)
        r0, r1 = int(off[i]), int(off[i + 1])
        x = x_perm64[r0:r1]
        a = x @ w1
        g = x @ w3
        h = O.silu(a) * g
        do = do_perm64[r0:r1]
        dh = do @ w2.T
        da, dg = swiglu_backward(a, g, dh)
        dx[r0:r1] = da @ w1.T + dg @ w3.T
        dW1.append(x.T @ da)
        dW3.append(x.T @ dg)
        dW2.append(h.T @ do)
        for name, v in (("a", a), ("g", g), ("h", h), ("dh", dh)):
            inter.setdefault(name, []).append(v)
    out: Dict[str, object] = dict(dx_perm=dx, dW1=dW1, dW3=dW3, dW2=dW2)
    for name, parts in inter.items():
        out[name] = np.concatenate(parts, axis=0) if parts else np.zeros((0, 0))
    return out


def uncombine(dx_perm64: np.ndarray, pair_pos: np.ndarray, T: int, k: int) -> np.ndarray:
    """dx[t] = sum over t's pairs with a local row r of dx_perm[r] (the same
    rows the forward's permute copied x[t] into)."""
    pp = np.asarray(pair_pos).reshape(T, k)
    dx = np.zeros((T, dx_perm64.shape[1]), np.float64)
    for j in range(k):
        rows = pp[:, j]
        have = rows >= 0
        dx[have] += dx_perm64[rows[have]]
    return dx


def router_backward(x64: np.ndarray, w_gate64: np.ndarray,
                    dlogits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """logits = x . W_g: (dx = dlogits . W_g^T [T, d], dW_g = x^T . dlogits [d, E])."""
    return dlogits @ np.asarray(w_gate64, np.float64).T, np.asarray(x64, np.float64).T @ dlogits


def moe_layer_backward(x: np.ndarray, dtype: str, logits_f32: np.ndarray, k: int, gate: str,
                       weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]],
                       E: int, dy: np.ndarray, capacity: int = -1, e_begin: int = 0,
                       e_end: Optional[int] = None,
                       w_gate64: Optional[np.ndarray] = None) -> Dict[str, object]:
    """Forward (moe_oracle.moe_layer) then the backward of sum(dy * y), float64.

    dy holds values of `dtype` (fp32 values or bf16 bits, like x).  With
    w_gate64 the logits are taken as x . W_g's fp32 values by the caller and
    the router term is added to dx and dW_g returned (R29).
    """
    fwd = O.moe_layer(x, dtype, logits_f32, k, gate, weights, E, capacity, e_begin, e_end)
    x64 = O.widen(x, dtype)
    dy64 = O.widen(dy, dtype)
    T = x64.shape[0]
    n = int(np.asarray(fwd["offsets"])[-1])
    do, dgate = combine_backward(dy64, fwd["y_perm"], fwd["pair_pos"], fwd["topk_w"], n)
    x_perm64 = O.permute(x64, fwd["sorted_pair"], k)
    eb = expert_ffn_backward(x_perm64, fwd["offsets"], weights, do)
    dx = uncombine(eb["dx_perm"], fwd["pair_pos"], T, k)
    dlogits = gate_backward(logits_f32, fwd["topk_idx"], dgate, gate)
    out: Dict[str, object] = dict(fwd=fwd, do_perm=do, dgate=dgate, dlogits=dlogits,
                                  dx_experts=dx.copy(), dx=dx)
    out.update(eb)
    if w_gate64 is not None:
        dxr, dwg = router_backward(x64, w_gate64, dlogits)
        out["dx"] = dx + dxr
        out["dW_g"] = dwg
    return out
