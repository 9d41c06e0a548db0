"""Pins of the oracle's router (top-k selection and gates).

Each test fixes the oracle to something other than itself: a brute-force
sort written independently, closed forms, a textbook softmax, invariants.
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import make

SOFT, SIG = O.GATE_SOFTMAX, O.GATE_SIGMOID


def brute_topk(row, k):
    """Pick k times the largest remaining value, lowest index on ties (selection sort)."""
    vals = [float(v) for v in row]
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(vals):
            if e in taken:
                continue
            if best is None or v > vals[best]:
                best = e
        taken.append(best)
    return taken


@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (2, 2), (5, 3), (8, 2), (64, 8), (256, 8)])
def test_topk_matches_brute_force(E, k):
    rng = np.random.default_rng(E * 100 + k)
    # coarse values make many exact ties
    logits = rng.integers(-4, 5, size=(40, E)).astype(np.float32) * np.float32(0.5)
    idx, _ = O.route(logits, k, SOFT)
    for t in range(40):
        assert list(idx[t]) == brute_topk(logits[t], k)


def test_topk_brute_force_on_tiny_workload():
    wl = make("tiny_fp32")
    idx, _ = O.route(wl.logits, wl.k, SOFT)
    for t in range(wl.T):
        assert list(idx[t]) == brute_topk(wl.logits[t], wl.k)


@pytest.mark.parametrize("k", [2, 8])
@pytest.mark.parametrize("gate", [SOFT, SIG])
def test_all_equal_rows(k, gate):
    logits = np.full((3, 16), 0.37, dtype=np.float32)
    idx, w = O.route(logits, k, gate)
    assert (idx == np.arange(k)[None, :]).all()
    assert (w == 1.0 / k).all()   # 1/2 and 1/8 are exact


def test_signed_zero_ties_lower_index_wins():
    logits = np.array([[-0.0, 0.0, -1.0, -0.0],
                       [0.0, -0.0, -2.0, -3.0],
                       [-5.0, -0.0, 0.0, -0.0]], dtype=np.float32)
    idx, w = O.route(logits, 2, SOFT)
    assert idx.tolist() == [[0, 1], [0, 1], [1, 2]]
    assert np.allclose(w, 0.5, rtol=0, atol=0)


def test_dominant_logit_first():
    logits = np.zeros((4, 8), dtype=np.float32)
    for t, e in enumerate([7, 0, 3, 5]):
        logits[t, e] = 30.0
    idx, w = O.route(logits, 2, SOFT)
    assert idx[:, 0].tolist() == [7, 0, 3, 5]
    # second choice: all remaining are tied at 0 -> lowest remaining index
    assert idx[:, 1].tolist() == [0, 1, 0, 0]
    assert np.all(w[:, 0] > 0.999999)


def test_softmax_then_topk_then_renorm_equals_oracle():
    """Page reading: softmax over all E, keep the k largest probabilities, renormalise.
    The oracle instead takes a softmax over the k chosen logits; the two agree exactly
    in real arithmetic (the full denominator cancels)."""
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((50, 32)).astype(np.float32)
    for k in (1, 2, 4, 32):
        idx, w = O.route(logits, k, SOFT)
        l = logits.astype(np.float64)
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        pk = np.take_along_axis(p, idx.astype(np.int64), axis=1)
        ref = pk / pk.sum(axis=1, keepdims=True)
        assert np.max(np.abs(w - ref)) < 1e-14
        if k == 32:  # k == E: plain softmax, in the oracle's order
            assert np.max(np.abs(w - np.take_along_axis(p, idx.astype(np.int64), axis=1))) < 1e-14


def test_sigmoid_pair_closed_form():
    """k = 2 with logits +a and -a: sigmoid(a) + sigmoid(-a) = 1, so w = (sigmoid(a), sigmoid(-a))."""
    a = math.log(3.0)   # sigmoid(ln 3) = 3/4
    logits = np.array([[-a, a, -10.0, -10.0]], dtype=np.float32)
    idx, w = O.route(logits, 2, SIG)
    assert idx.tolist() == [[1, 0]]
    a32 = float(np.float32(a))
    s = 1.0 / (1.0 + math.exp(-a32))
    assert abs(w[0, 0] - s) < 1e-15 and abs(w[0, 1] - (1 - s)) < 1e-15
    assert abs(w[0, 0] - 0.75) < 1e-7


def test_sigmoid_gates_differ_from_softmax_gates():
    """Guards against swapping the two gate rules."""
    logits = np.array([[2.0, 1.0, 0.0]], dtype=np.float32)
    _, ws = O.route(logits, 2, SOFT)
    _, wg = O.route(logits, 2, SIG)
    # softmax over (2, 1): e/(e+1); sigmoid-norm: s(2)/(s(2)+s(1))
    assert abs(ws[0, 0] - math.e / (math.e + 1)) < 1e-15
    s2, s1 = 1 / (1 + math.exp(-2)), 1 / (1 + math.exp(-1))
    assert abs(wg[0, 0] - s2 / (s1 + s2)) < 1e-15


@pytest.mark.parametrize("name", ["tiny_fp32", "dsv3_decode", "dsv3_prefill_zipf", "ep_rank_share"])
def test_invariants_on_workloads(name):
    wl = make(name)
    idx, w = O.route(wl.logits, wl.k, wl.gate)
    T, k = idx.shape
    # distinct experts per token: the co-activation diagonal is zero (sparse-activation page §4.1)
    assert all(len(set(r)) == k for r in idx.tolist())
    assert idx.min() >= 0 and idx.max() < wl.E
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
    assert np.all(w > 0)
    # best first: chosen logits are non-increasing along j
    sel = np.take_along_axis(wl.logits, idx.astype(np.int64), axis=1)
    assert np.all(sel[:, :-1] >= sel[:, 1:])
    # every unchosen logit is <= the k-th chosen logit
    mask = np.ones_like(wl.logits, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
    kth = sel[:, -1:]
    assert np.all(np.where(mask, wl.logits, -np.inf) <= kth)


def test_rejects_nonfinite_and_bad_k():
    with pytest.raises(ValueError):
        O.route(np.array([[np.nan, 0.0]], dtype=np.float32), 1, SOFT)
    with pytest.raises(ValueError):
        O.route(np.zeros((1, 4), dtype=np.float32), 5, SOFT)


def test_router_logits_one_hot_rows_and_linearity():
    rng = np.random.default_rng(3)
    wg = rng.standard_normal((16, 8))
    x = np.eye(16)
    assert np.array_equal(O.router_logits(x, wg), wg)
    xa = rng.standard_normal((5, 16))
    xb = rng.standard_normal((5, 16))
    lhs = O.router_logits(2.0 * xa + xb, wg)
    rhs = 2.0 * O.router_logits(xa, wg) + O.router_logits(xb, wg)
    assert np.max(np.abs(lhs - rhs)) < 1e-12


# ---------------------------------------------------------------- overflow rerouting (R26)
def test_reroute_without_pressure_is_plain_routing():
    rng = np.random.default_rng(11)
    for T, E, k in [(50, 8, 2), (40, 16, 4), (30, 4, 4)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        for cap in (-1, T):                      # no limit, or a limit nobody reaches
            idx, w = O.route_reroute(logits, k, O.GATE_SOFTMAX, cap)
            ridx, rw = O.route(logits, k, O.GATE_SOFTMAX)
            assert np.array_equal(idx, ridx) and np.allclose(w, rw, rtol=0, atol=0)


def test_reroute_hand_examples():
    # k = 1, every token prefers 0 > 1 > 2, capacity 2: the third and fourth go to 1
    l = np.tile(np.array([[2.0, 1.0, 0.0]], np.float32), (4, 1))
    idx, w = O.route_reroute(l, 1, O.GATE_SOFTMAX, 2)
    assert idx[:, 0].tolist() == [0, 0, 1, 1] and np.all(w == 1.0)
    # k = 2, capacity 1 (worked by hand):
    #   t0 ranks 0,1,2 -> {0,1}; t1 ranks 0,2,3, 0 is full -> {2,3};
    #   t2 ranks 1,2,3, 1 is full -> {2,3}; t3 ranks 2,3,0, 2 is full -> {3,0}
    l = np.array([[3, 2, 1, 0], [3, 0, 2, 1], [0, 3, 2, 1], [1, 0, 3, 2]], np.float32)
    idx, w = O.route_reroute(l, 2, O.GATE_SOFTMAX, 1)
    assert idx.tolist() == [[0, 1], [2, 3], [2, 3], [3, 0]]
    e = np.exp(-1.0)
    assert np.allclose(w[0], [1 / (1 + e), e / (1 + e)], rtol=1e-15)
    # sigmoid gates over the final pair of t3 (logits 2 and 1)
    idx, w = O.route_reroute(l, 2, O.GATE_SIGMOID, 1)
    s2, s1 = 1 / (1 + np.exp(-2.0)), 1 / (1 + np.exp(-1.0))
    assert np.allclose(w[3], [s2 / (s1 + s2), s1 / (s1 + s2)], rtol=1e-15)


def _reroute_brute(logits, k, cap):
    """The definition with every load recounted from the earlier tokens' final sets."""
    T, E = logits.shape
    final = []
    for t in range(T):
        ranked = sorted(range(E), key=lambda e: (-float(logits[t, e] + np.float32(0)), e))
        chosen = ranked[:k]
        if cap >= 0 and k < E:
            load = sum(1 for s in final if chosen[0] in s)
            if load >= cap:
                chosen = ranked[1:k] + [ranked[k]]
        final.append(chosen)
    return np.array(final, np.int32)


def test_reroute_matches_brute_force_and_invariants():
    rng = np.random.default_rng(12)
    for T, E, k, cap in [(60, 8, 2, 5), (80, 16, 4, 9), (40, 6, 1, 3), (50, 5, 5, 2),
                         (64, 12, 3, 0)]:
        logits = (rng.integers(-3, 4, (T, E)) * 0.5).astype(np.float32)   # many ties
        logits += rng.standard_normal(E).astype(np.float32)               # per-expert skew
        idx, w = O.route_reroute(logits, k, O.GATE_SOFTMAX, cap)
        assert np.array_equal(idx, _reroute_brute(logits, k, cap))
        ridx, _ = O.route(logits, min(k + 1, E), O.GATE_SOFTMAX)
        for t in range(T):
            assert len(set(idx[t])) == k and set(idx[t]) <= set(ridx[t])
            assert set(ridx[t, 1:k]) <= set(idx[t])                        # ranks 2..k always stay
        assert np.allclose(w.sum(axis=1), 1.0)
