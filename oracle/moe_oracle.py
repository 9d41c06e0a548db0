"""CPU oracle of the MoE expert path: route -> dispatch -> SwiGLU experts -> combine.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct
reference that the GPU library is checked against.  Only the test suite, the
package smoke check and the CPU-baseline leg of the benchmark may import it;
the library itself never does, and shares no code, table or helper with it.

Everything is NumPy in float64, computed from the exact input bits (fp32, or
bf16 bit patterns widened exactly).  Sources, cited by page and section:

  * MoE sparse-activation page ("大模型MoE稀疏激活原理与硬件适配实战"):
      §2.2 three-level decomposition (route, load experts, compute locally);
      §2.3 per-expert load formula (Batch x SeqLen x K) / E and its worked
           example, which fixes the capacity rule below;
      §3.1 table, router row: embedding -> logits -> top-k expert indices;
      §3.2 routing stages: fine ranking of the logits and taking the top k
           (stage 2) is what `route` computes; stages 1, 3, 4 are not part of
           this layer (see the readings);
      §4.1 co-activation check: a token never picks the same expert twice;
      §5.3 scenario 3: the router runs in fp32.
  * NCCL EP page ("NCCL EP架构解析"): §2.1 LL combine kernel, the weighted sum
    over the k chosen experts of each token's expert outputs; §2.2 layout
    table, the compact expert-major [sum T x H] dispatch layout.
  * DWDP page ("DWDP: 在NVL72上的高性能分布式权重数据并行"): key optimisations,
    the gather + grouped GEMM + SwiGLU operator and the grouped GEMM +
    finalize operator; W3 and W1 form one fused first-layer operand.
  * MegaMoE comparison page: §1 of the core differences, the fused kernel's
    steps (dispatch, two linear layers, SwiGLU, aggregation).

SwiGLU is y = W2 . (silu(W1 . x) * (W3 . x)), silu(a) = a * sigmoid(a), with
weights in the x.W orientation: W1, W3 are [d, f] and W2 is [f, d].

Readings where the pages are silent or garbled (each also listed in the
design notes):
  R1  Selection key: the fp32 logit itself.  Softmax and sigmoid are
      monotone, so selecting on logits equals selecting on the gate values in
      exact arithmetic, and selection stays an exact fp32 comparison.
  R2  Ties go to the lower expert index; chosen experts are listed best first.
  R3  -0.0 and +0.0 compare equal (IEEE), so the lower index wins.
  R4  Logits are finite (precondition, asserted).
  R5  Softmax gates renormalised over the k chosen equal a softmax over the k
      chosen logits (the full denominator cancels).
  R6  Sigmoid gates: sigmoid(l_j) / sum over chosen sigmoid(l_i); no extra
      scaling constant.
  R9  Capacity C = ceil(cf * T * k / E) per expert; with cf = 1 it is the
      load formula of §2.3.
  R10 An expert keeps its first C pairs in token order; later ones drop.
  R11 A dropped pair contributes 0; surviving gates are not renormalised.
  R12 Dispatch layout: compact, expert-major, over local experts only.
  R13 Inside an expert's segment rows ascend in token index.
  R14 Pairs routed to a non-local expert are "remote": kept for capacity
      accounting, absent from the local FFN and from the local combine.
  R26 Overflow rerouting (the page's stage 3, "replace the full top-1 with the
      top-3" for top-2): in token order, an expert's load is the number of
      earlier tokens whose final choice holds it; a token whose best expert
      has reached the capacity takes its (k+1)-th best instead of the best;
      the dispatch capacity rule applies afterwards.  (Stage 1's logit
      threshold and stage 4's random choice stay out: the first changes which
      experts exist with no rule for fewer than k survivors, the second is
      not deterministic.)

Parity pins live in tests/test_oracle_*.py (brute force, closed forms,
invariants, library special cases, the page's worked capacity example).
Every function here is pinned; none is "parity unpinned".
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Callable, Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

GATE_SOFTMAX = "softmax_topk_renorm"
GATE_SIGMOID = "sigmoid_topk_norm"

# pair_pos codes for pairs that have no local row
DROPPED = -1
REMOTE = -2


# --------------------------------------------------------------------------
# input widening (exact)
# --------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of fp32 values or of bf16 bit patterns (uint16)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to_f32(a: np.ndarray) -> np.ndarray:
    """Nearest fp32 of float64 values (numpy's cast rounds to nearest even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# A0: router logits  (sparse-activation page §3.1 router row; §5.3 fp32 router)
# --------------------------------------------------------------------------
def router_logits(x64: np.ndarray, w_gate64: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * W_g[i, e], exact-input float64 product."""
    return np.asarray(x64, np.float64) @ np.asarray(w_gate64, np.float64)


# --------------------------------------------------------------------------
# A1: top-k routing and gates (sparse-activation page §3.2 stage 2, §4.1)
# --------------------------------------------------------------------------
def route(logits_f32: np.ndarray, k: int, gate: str) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token and their gate weights.

    Returns topk_idx [T, k] int32 (best first, ties to the lower index) and
    topk_w [T, k] float64 (R1-R6).
    """
    l32 = np.asarray(logits_f32, dtype=np.float32)
    T, E = l32.shape
    if not (1 <= k <= E):
        raise ValueError(f"k={k} outside [1, E={E}]")
    if not np.all(np.isfinite(l32)):
        raise ValueError("logits must be finite")
    # R3: -0.0 + 0.0 == +0.0, so both zeros share one key
    l32 = l32 + np.float32(0.0)
    l64 = l32.astype(np.float64)
    # primary key: logit descending; secondary: expert index ascending (R2)
    idx_key = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx_key, -l64), axis=-1)[:, :k]
    topk_idx = order.astype(np.int32)
    sel = np.take_along_axis(l64, order, axis=-1)
    return topk_idx, gate_values(sel, gate)


def gate_values(sel: np.ndarray, gate: str) -> np.ndarray:
    """Gate weights [T, k] from the chosen logits [T, k] (best first), float64 (R5, R6)."""
    sel = np.asarray(sel, dtype=np.float64)
    if gate == GATE_SOFTMAX:
        # R5: softmax over the chosen k, shifted by the largest chosen logit
        z = np.exp(sel - sel[:, :1])
        return z / z.sum(axis=1, keepdims=True)
    if gate == GATE_SIGMOID:
        s = 1.0 / (1.0 + np.exp(-sel))
        return s / s.sum(axis=1, keepdims=True)
    raise ValueError(gate)


def route_reroute(logits_f32: np.ndarray, k: int, gate: str,
                  capacity: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k routing with overflow rerouting (sparse-activation page §3.2,
    stage 3: when the best expert is already at its capacity limit, the token
    takes the next expert after its k instead) (R26).

    Tokens are taken in index order.  The load of expert e at token t is the
    number of earlier tokens whose final choice contains e.  If the best
    expert's load has reached the capacity (capacity >= 0, k < E), the best
    expert is replaced by the (k+1)-th best; the other k - 1 stay.  The final k
    are listed best first and the gates are computed over them exactly as in
    `route`.  The capacity rule of `dispatch` still applies afterwards (a
    replacement expert that is itself full drops the pair).
    """
    l32 = np.asarray(logits_f32, dtype=np.float32)
    T, E = l32.shape
    if not (1 <= k <= E):
        raise ValueError(f"k={k} outside [1, E={E}]")
    if not np.all(np.isfinite(l32)):
        raise ValueError("logits must be finite")
    l32 = l32 + np.float32(0.0)
    l64 = l32.astype(np.float64)
    idx_key = np.broadcast_to(np.arange(E), (T, E))
    ranked = np.lexsort((idx_key, -l64), axis=-1)[:, :min(k + 1, E)]
    load = np.zeros(E, dtype=np.int64)
    topk_idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        chosen = list(ranked[t, :k])
        if capacity >= 0 and k < E and load[chosen[0]] >= capacity:
            chosen = chosen[1:] + [ranked[t, k]]
        for e in chosen:
            load[e] += 1
        topk_idx[t] = chosen
    sel = np.take_along_axis(l64, topk_idx.astype(np.int64), axis=-1)
    return topk_idx, gate_values(sel, gate)


# --------------------------------------------------------------------------
# A2: capacity and the dispatch plan
# --------------------------------------------------------------------------
def capacity(T: int, k: int, E: int, capacity_factor: Optional[float]) -> int:
    """Per-expert capacity C = ceil(cf * T * k / E); -1 means no limit.

    With cf = 1 this is the per-expert load (Batch x SeqLen x K) / E of the
    sparse-activation page §2.3 (R9).  Exact rational arithmetic.
    """
    if capacity_factor is None:
        return -1
    q = Fraction(str(capacity_factor)) * T * k / E
    return int(math.ceil(q))


def dispatch(topk_idx: np.ndarray, E: int, capacity: int = -1,
             e_begin: int = 0, e_end: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Counting-sort plan of (token, slot) pairs into expert-major rows.

    Pair p = t * k + j is (token t, slot j) with expert e = topk_idx[t, j].
      counts[e]      all pairs that chose e (before any capacity drop)
      pos(p)         number of earlier tokens t' < t that chose e (R10, R13)
      kept           capacity < 0 or pos < capacity
      offsets[i]     exclusive scan of kept counts over local experts
                     e_begin + i, length E_loc + 1 (R12)
      sorted_pair[row] = p for kept local pairs, row = offsets[e - e_begin] + pos
      pair_pos[p]    row, DROPPED (-1) if not kept, REMOTE (-2) if kept but
                     the expert is not local (R14)
      n_kept         offsets[-1]
    NCCL EP page §2.2 (compact expert-major layout); ThunderEP page §2.1/§2.2
    (pack all rows bound for one owner together; per-expert index lists).
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    if e_end is None:
        e_end = E
    if not (0 <= e_begin < e_end <= E):
        raise ValueError("bad local expert range")
    if idx.size and (idx.min() < 0 or idx.max() >= E):
        raise ValueError("expert index out of range")
    E_loc = e_end - e_begin
    # pos by a running per-expert counter walked in token order
    running = np.zeros(E, dtype=np.int64)
    pos = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            pos[t * k + j] = running[e]
            running[e] += 1
    counts = running.astype(np.int32)
    kept_per_e = counts.astype(np.int64) if capacity < 0 else np.minimum(counts, capacity)
    offsets = np.zeros(E_loc + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept_per_e[e_begin:e_end])
    n_kept = int(offsets[-1])
    sorted_pair = np.full(max(n_kept, 0), -1, dtype=np.int32)
    pair_pos = np.empty(T * k, dtype=np.int32)
    for p in range(T * k):
        e = int(idx.flat[p])
        kept = capacity < 0 or pos[p] < capacity
        if not kept:
            pair_pos[p] = DROPPED
        elif e_begin <= e < e_end:
            row = int(offsets[e - e_begin] + pos[p])
            sorted_pair[row] = p
            pair_pos[p] = row
        else:
            pair_pos[p] = REMOTE
    return dict(counts=counts, offsets=offsets.astype(np.int32), sorted_pair=sorted_pair,
                pair_pos=pair_pos, n_kept=n_kept, pos=pos.astype(np.int32))


# --------------------------------------------------------------------------
# A3: permutation into expert-major rows
# --------------------------------------------------------------------------
def permute(x: np.ndarray, sorted_pair: np.ndarray, k: int) -> np.ndarray:
    """x_perm[row] = x[sorted_pair[row] // k] (a plain row copy, any dtype)."""
    sp = np.asarray(sorted_pair, dtype=np.int64)
    return np.asarray(x)[sp // k]


# --------------------------------------------------------------------------
# A4 + A5: per-expert SwiGLU FFN
# --------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    """a * sigmoid(a) in float64."""
    return a / (1.0 + np.exp(-a))


def swiglu_hidden(x64: np.ndarray, w1: np.ndarray, w3: np.ndarray) -> np.ndarray:
    """h = silu(x W1) * (x W3) for rows x [n, d] (the first FFN half); float64."""
    a = x64 @ w1
    g = x64 @ w3
    return silu(a) * g


def swiglu_ffn(x64: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """(silu(x W1) * (x W3)) W2 for rows x [n, d]; weights float64, x.W orientation."""
    return swiglu_hidden(x64, w1, w3) @ w2


def expert_ffn(x_perm64: np.ndarray, offsets: np.ndarray,
               weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """y_perm rows of each local expert segment through that expert's FFN.

    weights(i) returns float64 (W1, W3, W2) of local expert i.
    """
    off = np.asarray(offsets, dtype=np.int64)
    n = int(off[-1])
    d = x_perm64.shape[1]
    y = np.zeros((n, d), dtype=np.float64)
    for i in range(len(off) - 1):
        r0, r1 = int(off[i]), int(off[i + 1])
        if r1 > r0:
            w1, w3, w2 = weights(i)
            y[r0:r1] = swiglu_ffn(x_perm64[r0:r1], w1, w3, w2)
    return y


# --------------------------------------------------------------------------
# A6: weighted combine (NCCL EP page §2.1, LL combine)
# --------------------------------------------------------------------------
def combine(y_perm64: np.ndarray, pair_pos: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """y[t] = sum_j w[t, j] * y_perm[pair_pos[t*k + j]] over pairs with a local row.

    Tokens with no local kept pair get a zero row (R11, R14).
    """
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = w.shape
    d = y_perm64.shape[1] if y_perm64.ndim == 2 else 0
    y = np.zeros((T, d), dtype=np.float64)
    pp = np.asarray(pair_pos).reshape(T, k)
    for j in range(k):
        rows = pp[:, j]
        have = rows >= 0
        y[have] += w[have, j:j + 1] * y_perm64[rows[have]]
    return y


# --------------------------------------------------------------------------
# whole layer, and the brute-force dense form
# --------------------------------------------------------------------------
def moe_layer(x: np.ndarray, dtype: str, logits_f32: np.ndarray, k: int, gate: str,
              weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]],
              E: int, capacity: int = -1, e_begin: int = 0,
              e_end: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Route -> dispatch -> permute -> expert FFN -> combine, all float64.

    x holds fp32 values or bf16 bits per `dtype`; weights(i) returns the
    float64 weights of local expert i.
    """
    idx, w = route(logits_f32, k, gate)
    plan = dispatch(idx, E, capacity, e_begin, e_end)
    x64 = widen(x, dtype)
    x_perm64 = permute(x64, plan["sorted_pair"], k)
    y_perm = expert_ffn(x_perm64, plan["offsets"], weights)
    y = combine(y_perm, plan["pair_pos"], w)
    out = dict(topk_idx=idx, topk_w=w, y_perm=y_perm, y=y, x_perm=permute(x, plan["sorted_pair"], k))
    out.update(plan)
    return out


def dense_masked_moe(x64: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray,
                     pair_pos: np.ndarray, e_begin: int,
                     weights: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]],
                     E_loc: int) -> np.ndarray:
    """Brute force: every local expert runs on every token; gates outside the
    token's kept local choices are zero.  y = sum_e G[:, e] * FFN_e(x).

    Uses no permutation, offsets or combine; pair_pos only tells which pairs
    survived capacity and are local (pair_pos >= 0).
    """
    T, k = topk_idx.shape
    G = np.zeros((T, E_loc), dtype=np.float64)
    pp = np.asarray(pair_pos).reshape(T, k)
    for t in range(T):
        for j in range(k):
            if pp[t, j] >= 0:
                G[t, int(topk_idx[t, j]) - e_begin] += topk_w[t, j]
    y = np.zeros((T, x64.shape[1]), dtype=np.float64)
    for i in range(E_loc):
        w1, w3, w2 = weights(i)
        y += G[:, i:i + 1] * swiglu_ffn(x64, w1, w3, w2)
    return y


def token_outputs(tokens: Sequence[int], x64_rows: np.ndarray, topk_idx: np.ndarray,
                  topk_w: np.ndarray, pair_pos: np.ndarray, e_begin: int,
                  weights_global: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]
                  ) -> np.ndarray:
    """y for a sample of tokens, one token at a time from the layer's definition:
    y[t] = sum over kept local slots j of w[t, j] * FFN_{e_j}(x[t]).

    x64_rows[i] is token tokens[i]'s input row; weights_global(e) returns the
    float64 weights of global expert e.  Experts are visited once each.
    """
    tokens = list(tokens)
    T, k = topk_idx.shape
    pp = np.asarray(pair_pos).reshape(T, k)
    need: Dict[int, list] = {}
    for i, t in enumerate(tokens):
        for j in range(k):
            if pp[t, j] >= 0:
                need.setdefault(int(topk_idx[t, j]), []).append((i, j))
    y = np.zeros((len(tokens), x64_rows.shape[1]), dtype=np.float64)
    for e in sorted(need):
        w1, w3, w2 = weights_global(e)
        rows = [i for i, _ in need[e]]
        o = swiglu_ffn(x64_rows[rows], w1, w3, w2)
        for r, (i, j) in enumerate(need[e]):
            y[i] += topk_w[tokens[i], j] * o[r]
    return y


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """The parity measure max|got - ref| / max|ref|, element by element over
    arrays of one shape (a shape mismatch raises instead of broadcasting).
    Empty arrays give 0; an all-zero reference gives the absolute error
    max|got|; a NaN anywhere gives NaN, which fails every tolerance."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"rel_err: shapes {got.shape} and {ref.shape} differ")
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return num
    return num / den
