"""Pins of the oracle's expert FFN, combine and whole layer."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import custom, make


def weights64(wl, e):
    w1, w3, w2 = wl.expert_weights(e)
    return O.widen(w1, wl.dtype), O.widen(w3, wl.dtype), O.widen(w2, wl.dtype)


def local_weights(wl):
    return lambda i: weights64(wl, wl.e_begin + i)


def run_layer(wl, cap=None):
    C = O.capacity(wl.T, wl.k, wl.E, wl.capacity_factor) if cap is None else cap
    return O.moe_layer(wl.x, wl.dtype, wl.logits, wl.k, wl.gate, local_weights(wl), wl.E, C,
                       wl.e_begin, wl.e_end)


def torch_swiglu(x, w1, w3, w2):
    """Library form: torch's own silu on fp64 tensors."""
    xt, a, b, c = (torch.from_numpy(np.ascontiguousarray(v)) for v in (x, w1, w3, w2))
    return (torch.nn.functional.silu(xt @ a) * (xt @ b) @ c).numpy()


def test_single_expert_reduces_to_plain_swiglu():
    wl = custom(T=33, d=16, f=24, E=1, k=1, dtype="f32", seed=5)
    out = run_layer(wl)
    x64 = O.widen(wl.x, "f32")
    ref = torch_swiglu(x64, *weights64(wl, 0))
    assert np.array_equal(out["topk_idx"], np.zeros((33, 1)))
    assert np.all(out["topk_w"] == 1.0)
    assert O.rel_err(out["y"], ref) < 1e-13


@pytest.mark.parametrize("name_kw", [
    dict(T=64, d=32, f=48, E=8, k=2, dtype="f32"),
    dict(T=50, d=16, f=32, E=5, k=3, dtype="bf16", gate=O.GATE_SIGMOID),
    dict(T=80, d=16, f=16, E=6, k=2, dtype="bf16", capacity_factor=0.5),
    dict(T=80, d=16, f=16, E=12, k=3, dtype="bf16", capacity_factor=1.0, e_begin=3, e_end=9),
])
def test_layer_equals_dense_masked_brute_force(name_kw):
    wl = custom(seed=1, **name_kw)
    out = run_layer(wl)
    y_bf = O.dense_masked_moe(O.widen(wl.x, wl.dtype), out["topk_idx"], out["topk_w"],
                              out["pair_pos"], wl.e_begin, local_weights(wl), wl.E_loc)
    assert O.rel_err(out["y"], y_bf) < 1e-12


def test_tiny_workload_equals_brute_force():
    wl = make("tiny_fp32")
    out = run_layer(wl)
    y_bf = O.dense_masked_moe(O.widen(wl.x, "f32"), out["topk_idx"], out["topk_w"],
                              out["pair_pos"], 0, local_weights(wl), wl.E)
    assert O.rel_err(out["y"], y_bf) < 1e-12


def test_identical_experts_give_plain_ffn():
    """All experts share one weight set; gates sum to 1, so y = FFN(x) for any routing."""
    wl = custom(T=90, d=24, f=40, E=16, k=4, dtype="bf16", gate=O.GATE_SIGMOID, seed=2)
    shared = weights64(wl, 0)
    out = O.moe_layer(wl.x, "bf16", wl.logits, 4, wl.gate, lambda i: shared, 16)
    ref = torch_swiglu(O.widen(wl.x, "bf16"), *shared)
    assert O.rel_err(out["y"], ref) < 1e-12


def test_zero_down_projection_gives_zero():
    wl = custom(T=20, d=8, f=8, E=4, k=2, dtype="f32", seed=3)
    def w(i):
        a, b, _ = weights64(wl, i)
        return a, b, np.zeros((8, 8))
    out = O.moe_layer(wl.x, "f32", wl.logits, 2, wl.gate, w, 4)
    assert np.all(out["y"] == 0.0)


def test_combine_one_hot_rows_reproduce_gates():
    wl = custom(T=40, d=4, f=4, E=8, k=3, dtype="f32", seed=4)
    idx, w = O.route(wl.logits, 3, wl.gate)
    plan = O.dispatch(idx, 8)
    n = plan["n_kept"]
    y_perm = np.zeros((n, 3))
    for row in range(n):
        y_perm[row, plan["sorted_pair"][row] % 3] = 1.0   # slot j of that pair
    y = O.combine(y_perm, plan["pair_pos"], w)
    assert np.array_equal(y, w)


def test_combine_skips_dropped_and_remote():
    w = np.array([[0.6, 0.4], [0.5, 0.5]])
    y_perm = np.array([[1.0, 2.0], [10.0, 20.0]])
    pp = np.array([1, O.DROPPED, O.REMOTE, 0])
    y = O.combine(y_perm, pp, w)
    assert np.allclose(y, [[6.0, 12.0], [0.5, 1.0]], rtol=0, atol=1e-15)


def test_capacity_zero_gives_zero_output():
    wl = custom(T=30, d=8, f=8, E=4, k=2, dtype="bf16", seed=6)
    out = run_layer(wl, cap=0)
    assert out["n_kept"] == 0 and np.all(out["y"] == 0.0)


def test_scaling_down_projection_scales_output():
    wl = custom(T=30, d=8, f=16, E=4, k=2, dtype="f32", seed=8)
    base = run_layer(wl)
    def w(i):
        a, b, c = weights64(wl, i)
        return a, b, 3.0 * c
    out = O.moe_layer(wl.x, "f32", wl.logits, 2, wl.gate, w, 4)
    assert O.rel_err(out["y"], 3.0 * base["y"]) < 1e-14


def test_silu_against_library():
    a = np.linspace(-30, 30, 1001)
    ref = torch.nn.functional.silu(torch.from_numpy(a)).numpy()
    assert np.max(np.abs(O.silu(a) - ref)) < 1e-13


def test_token_outputs_match_layer():
    wl = custom(T=70, d=16, f=24, E=10, k=3, dtype="bf16", capacity_factor=1.0, e_begin=2,
                e_end=8, seed=9)
    out = run_layer(wl)
    toks = [0, 5, 17, 69]
    y = O.token_outputs(toks, O.widen(wl.x[toks], "bf16"), out["topk_idx"], out["topk_w"],
                        out["pair_pos"], wl.e_begin, lambda e: weights64(wl, e))
    assert O.rel_err(y, out["y"][toks]) < 1e-13


@pytest.mark.slow
def test_ep_rank_share_subset_layer_brute_force():
    """Capacity-limited EP share on a token subset: layer == brute force."""
    wl = make("ep_rank_share", T=512, d=64, f=32)
    out = run_layer(wl)
    y_bf = O.dense_masked_moe(O.widen(wl.x, "bf16"), out["topk_idx"], out["topk_w"],
                              out["pair_pos"], 0, local_weights(wl), wl.E_loc)
    assert O.rel_err(out["y"], y_bf) < 1e-12
    assert (out["pair_pos"] == O.DROPPED).sum() > 0
    assert (out["pair_pos"] == O.REMOTE).sum() > 0
