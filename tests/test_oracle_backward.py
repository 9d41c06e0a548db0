"""Pins of the backward oracle (oracle/backward_oracle.py): central finite
differences of moe_oracle's own forward building blocks (routing decisions
held fixed, Richardson-extrapolated), closed forms, and planted mistakes."""
import numpy as np
import pytest

from oracle import backward_oracle as B
from oracle import moe_oracle as O


def _case(seed, T=14, d=8, f=6, E=5, k=2, gate=O.GATE_SOFTMAX, capacity=4, e_begin=1, e_end=4,
          identical=False, w2_zero=False, router=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    E_loc = e_end - e_begin
    ws = []
    for i in range(E_loc):
        r = np.random.default_rng(100 + (0 if identical else i))
        w1 = r.standard_normal((d, f)) / np.sqrt(d)
        w3 = r.standard_normal((d, f)) / np.sqrt(d)
        w2 = np.zeros((f, d)) if w2_zero else r.standard_normal((f, d)) / np.sqrt(f)
        ws.append((w1, w3, w2))
    wg = None
    if router:
        wg = rng.standard_normal((d, E)) * 0.5
        logits = (x.astype(np.float64) @ wg).astype(np.float32)
    else:
        # well-separated logits: a step of 1e-3 never changes a top-k set
        logits = np.stack([rng.permutation(E) for _ in range(T)]).astype(np.float32) * 0.5
        logits += rng.uniform(-0.1, 0.1, (T, E)).astype(np.float32)
    return dict(x=x, dy=dy, ws=ws, logits=logits, k=k, gate=gate, E=E, capacity=capacity,
                e_begin=e_begin, e_end=e_end, wg=wg)


def _backward(c):
    return B.moe_layer_backward(c["x"], "f32", c["logits"], c["k"], c["gate"], lambda i: c["ws"][i],
                                c["E"], c["dy"], c["capacity"], c["e_begin"], c["e_end"],
                                w_gate64=c["wg"])


def _loss_fn(c, res):
    """sum(dy * y) as a function of float64 (x, weights, logits or W_g), with the
    forward's routing decisions and plan fixed, built from moe_oracle's steps."""
    fwd = res["fwd"]
    idx = np.asarray(fwd["topk_idx"], np.int64)
    k = c["k"]
    dy = c["dy"].astype(np.float64)

    def loss(x64, ws, logits64):
        sel = np.take_along_axis(logits64, idx, axis=-1)
        w = O.gate_values(sel, c["gate"])
        xp = O.permute(x64, fwd["sorted_pair"], k)
        yp = O.expert_ffn(xp, fwd["offsets"], lambda i: ws[i])
        return float(np.sum(dy * O.combine(yp, fwd["pair_pos"], w)))
    return loss


def _fd(f, p, idx, h=1e-3):
    """Richardson-extrapolated central difference of f at p[idx]."""
    def d(step):
        a = p.copy()
        b = p.copy()
        a[idx] += step
        b[idx] -= step
        return (f(a) - f(b)) / (2 * step)
    return (4 * d(h / 2) - d(h)) / 3


def _check_fd(c, res, n=5, tol=1e-7):
    """Compare every analytic gradient family at n random coordinates; returns
    the worst relative mismatch."""
    loss = _loss_fn(c, res)
    rng = np.random.default_rng(7)
    x64 = c["x"].astype(np.float64)
    ws = [tuple(np.array(m, np.float64) for m in t) for t in c["ws"]]
    l64 = c["logits"].astype(np.float64)
    worst = 0.0

    def cmp(num, ana, scale):
        nonlocal worst
        worst = max(worst, abs(num - ana) / scale)

    scale = max(1.0, float(np.abs(res["dx"]).max()))
    for _ in range(n):
        i = tuple(rng.integers(0, s) for s in x64.shape)
        cmp(_fd(lambda p: loss(p, ws, l64) if c["wg"] is None else loss(p, ws, p @ c["wg"]), x64, i),
            res["dx"][i] if c["wg"] is not None else res["dx_experts"][i], scale)
    for e in range(len(ws)):
        for m, name in enumerate(("dW1", "dW3", "dW2")):
            g = res[name][e]
            s = max(1.0, float(np.abs(g).max()))
            for _ in range(n):
                i = tuple(rng.integers(0, sz) for sz in ws[e][m].shape)

                def f(p, e=e, m=m):
                    w2 = list(ws)
                    t = list(w2[e])
                    t[m] = p
                    w2[e] = tuple(t)
                    return loss(x64, w2, l64 if c["wg"] is None else x64 @ c["wg"])
                cmp(_fd(f, ws[e][m], i), g[i], s)
    if c["wg"] is None:
        s = max(1.0, float(np.abs(res["dlogits"]).max()))
        for _ in range(3 * n):
            i = tuple(rng.integers(0, sz) for sz in l64.shape)
            cmp(_fd(lambda p: loss(x64, ws, p), l64, i), res["dlogits"][i], s)
    else:
        s = max(1.0, float(np.abs(res["dW_g"]).max()))
        for _ in range(3 * n):
            i = tuple(rng.integers(0, sz) for sz in c["wg"].shape)
            cmp(_fd(lambda p: loss(x64, ws, x64 @ p), c["wg"], i), res["dW_g"][i], s)
    return worst


@pytest.mark.parametrize("gate", [O.GATE_SOFTMAX, O.GATE_SIGMOID])
@pytest.mark.parametrize("capacity,e_range", [(-1, (0, 5)), (4, (1, 4)), (2, (0, 3))])
def test_finite_differences(gate, capacity, e_range):
    c = _case(1, gate=gate, capacity=capacity, e_begin=e_range[0], e_end=e_range[1])
    res = _backward(c)
    if capacity >= 0:
        assert np.any(np.asarray(res["fwd"]["pair_pos"]) == -1)   # some pairs dropped
    assert _check_fd(c, res) < 1e-7


@pytest.mark.parametrize("gate", [O.GATE_SOFTMAX, O.GATE_SIGMOID])
def test_finite_differences_with_router(gate):
    # logits = x . W_g: dx gains the router term, and dW_g = x^T dlogits; the
    # routing decisions come from the fp32-rounded logits, the differences from
    # exact ones, so the bar allows for that rounding
    c = _case(2, gate=gate, capacity=-1, e_begin=0, e_end=5, router=True)
    res = _backward(c)
    assert _check_fd(c, res) < 1e-5


def test_wider_k_and_dims():
    c = _case(3, T=10, d=16, f=12, E=6, k=3, capacity=3, e_begin=2, e_end=6)
    assert _check_fd(c, _backward(c), n=3) < 1e-7


def test_softmax_gate_gradient_is_shift_invariant():
    c = _case(4, capacity=-1, e_begin=0, e_end=5)
    res = _backward(c)
    assert np.abs(res["dlogits"].sum(axis=1)).max() < 1e-12 * max(1.0, np.abs(res["dlogits"]).max())
    # a constant gate gradient has no effect through softmax
    T, k = res["dgate"].shape
    dl = B.gate_backward(c["logits"], res["fwd"]["topk_idx"], np.full((T, k), 3.5), O.GATE_SOFTMAX)
    assert np.abs(dl).max() < 1e-14


def test_identical_experts_reduce_to_one_ffn():
    # every expert the same, softmax gates, nothing dropped: y = FFN(x), so the
    # gates get no gradient, dx is the single FFN's input gradient and the
    # experts' weight gradients add up to the single FFN's
    c = _case(5, capacity=-1, e_begin=0, e_end=5, identical=True)
    res = _backward(c)
    assert np.abs(res["dlogits"]).max() < 1e-12
    one = dict(c, ws=c["ws"][:1], E=1, k=1, e_begin=0, e_end=1,
               logits=np.zeros((c["x"].shape[0], 1), np.float32))
    r1 = _backward(one)
    assert np.abs(res["dx"] - r1["dx"]).max() < 1e-12 * np.abs(r1["dx"]).max()
    for name in ("dW1", "dW3", "dW2"):
        tot = sum(res[name])
        assert np.abs(tot - r1[name][0]).max() < 1e-12 * np.abs(r1[name][0]).max()


def test_zero_down_projection():
    c = _case(6, w2_zero=True)
    res = _backward(c)
    assert not np.any(res["dx"]) and not np.any(res["dlogits"])
    for i in range(len(c["ws"])):
        assert not np.any(res["dW1"][i]) and not np.any(res["dW3"][i])
    # dW2 = h^T do is not zero
    assert any(np.abs(g).max() > 0 for g in res["dW2"])


def test_linear_in_output_gradient():
    c = _case(7)
    r1 = _backward(c)
    c2 = dict(c, dy=(np.random.default_rng(8).standard_normal(c["dy"].shape)).astype(np.float32))
    r2 = _backward(c2)
    c3 = dict(c, dy=(c["dy"].astype(np.float64) + 2 * c2["dy"].astype(np.float64)).astype(np.float32))
    r3 = _backward(c3)
    exact_sum = np.array_equal(c3["dy"].astype(np.float64), c["dy"].astype(np.float64) + 2 * c2["dy"].astype(np.float64))
    tol = 1e-12 if exact_sum else 1e-6
    for name in ("dx", "dlogits", "do_perm"):
        ref = r1[name] + 2 * r2[name]
        assert np.abs(r3[name] - ref).max() <= tol * max(1.0, np.abs(ref).max())


def test_dropped_and_remote_pairs_get_nothing():
    c = _case(9, capacity=2, e_begin=1, e_end=3)
    res = _backward(c)
    pp = np.asarray(res["fwd"]["pair_pos"]).reshape(res["dgate"].shape)
    assert np.all(res["dgate"][pp < 0] == 0.0)
    # tokens with no local kept pair get no gradient through the experts
    none = np.all(pp < 0, axis=1)
    assert none.any() and not np.any(res["dx"][none])


def test_planted_mistakes_are_caught(monkeypatch):
    c = _case(10, gate=O.GATE_SIGMOID)
    assert _check_fd(c, _backward(c)) < 1e-7
    good_swiglu = B.swiglu_backward

    def no_product_rule(a, g, dh):     # silu'(a) taken as sigmoid(a)
        s = 1.0 / (1.0 + np.exp(-a))
        return dh * g * s, dh * a * s
    monkeypatch.setattr(B, "swiglu_backward", no_product_rule)
    assert _check_fd(c, _backward(c)) > 1e-3
    monkeypatch.setattr(B, "swiglu_backward", good_swiglu)

    good_gate = B.gate_backward

    def sign_flip(logits, idx, dg, gate):
        return -good_gate(logits, idx, dg, gate)
    monkeypatch.setattr(B, "gate_backward", sign_flip)
    assert _check_fd(c, _backward(c)) > 1e-3
    monkeypatch.setattr(B, "gate_backward", good_gate)

    good_comb = B.combine_backward

    def unweighted(dy, yp, pp, w, n):  # output gradient not scaled by the gate
        return good_comb(dy, yp, pp, np.ones_like(w), n)
    monkeypatch.setattr(B, "combine_backward", unweighted)
    assert _check_fd(c, _backward(c)) > 1e-3
