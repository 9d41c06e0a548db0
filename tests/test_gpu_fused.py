"""GPU parity of moe_forward_fused (the whole layer in one persistent launch)
against the CPU oracle and, bit for bit, against the separate calls, on small
seeded layers: several tiles, ragged tails, capacity drops, a local expert
range, skewed routing, and the degenerate cases (one token, everything
dropped)."""
import numpy as np
import pytest

import routing_dispatch_expert_moe_amd as M
from oracle import moe_oracle as O
from workloads import custom

from gpu_util import (as64, capacity_of, fused_matches_unfused, layer_for, log, packed_weights,
                      t_in, t_out, weights_fn)

pytestmark = pytest.mark.gpu

GATE_TOL = 1e-6
TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.mark.parametrize("kw", [
    dict(name="tiny", T=64, d=128, f=256, E=8, k=2, dtype="f32"),
    dict(name="f2", T=300, d=64, f=96, E=16, k=4, dtype="f32", capacity_factor=1.0),
    dict(name="b1", T=200, d=128, f=192, E=8, k=2, dtype="bf16"),
    dict(name="b2", T=150, d=256, f=128, E=32, k=8, dtype="bf16", gate=O.GATE_SIGMOID),
    dict(name="b3", T=333, d=128, f=128, E=16, k=2, dtype="bf16", capacity_factor=1.25,
         e_begin=4, e_end=12, logit_bias="normal"),
    dict(name="b4", T=257, d=192, f=256, E=64, k=4, dtype="bf16", logit_bias="zipf"),
    dict(name="b5", T=100, d=64, f=64, E=4, k=2, dtype="bf16", capacity_factor=0.25),
    dict(name="b6", T=1300, d=128, f=128, E=4, k=1, dtype="bf16"),
    dict(name="b7", T=600, d=64, f=128, E=300, k=3, dtype="bf16"),
    dict(name="b8", T=1, d=64, f=64, E=8, k=2, dtype="bf16"),
    # 1000 local experts: the workgroup scan's runs of two experts per thread
    # (512 threads) and the widest routing phase
    dict(name="b9", T=300, d=64, f=64, E=1000, k=2, dtype="bf16", logit_bias="zipf"),
    # a 4224-deep second GEMM with few tiles: 256-row tiles over the full blocks,
    # the short remainders in 128 x 128 tiles
    dict(name="b10", T=1200, d=256, f=4224, E=4, k=1, dtype="bf16"),
])
def test_fused_layer(kw):
    kw = dict(kw)
    log(f"fused layer {kw}")
    name = kw.pop("name")
    wl = custom(name, seed=5, **kw)
    w13, w2p, host = packed_weights(wl, keep_host=True)
    layer = layer_for(wl, w13, w2p)
    x = t_in(wl.x, wl.dtype)
    logits = t_in(wl.logits, "f32")
    layer.forward(x, logits=logits)
    assert M.moe_check_error(layer.ws) == 0
    fl = fused_matches_unfused(wl, w13, w2p, layer, x, logits)
    ref = O.moe_layer(wl.x, wl.dtype, wl.logits, wl.k, wl.gate, weights_fn(wl, host), wl.E,
                      capacity_of(wl), wl.e_begin, wl.e_end)
    out = fl.outputs()
    n = ref["n_kept"]
    assert np.array_equal(t_out(out["topk_idx"]), ref["topk_idx"])
    assert O.rel_err(t_out(out["topk_w"]), ref["topk_w"]) <= GATE_TOL
    assert np.array_equal(t_out(out["counts"]), ref["counts"])
    assert np.array_equal(t_out(out["offsets"]), ref["offsets"])
    assert np.array_equal(t_out(out["sorted_pair"])[:n], ref["sorted_pair"])
    assert np.array_equal(t_out(out["pair_pos"]), ref["pair_pos"])
    assert O.rel_err(as64(fl.y, wl.dtype), ref["y"]) <= TOL[wl.dtype]


@pytest.mark.parametrize("kw", [
    dict(name="l1", T=200, d=128, f=192, E=8, k=2, dtype="bf16"),
    dict(name="l2", T=333, d=128, f=128, E=16, k=2, dtype="bf16", capacity_factor=1.25,
         e_begin=4, e_end=12, logit_bias="normal"),
    # 256-row tiles over the full blocks and 128 x 128 remainder tiles (K = 4224)
    dict(name="l3", T=1200, d=256, f=4224, E=4, k=1, dtype="bf16"),
    dict(name="l4", T=64, d=128, f=256, E=8, k=2, dtype="f32"),
])
def test_fused_layer_list(kw):
    """moe_forward_fused_list (per-expert weight buffers through pointer
    tables, the TensorList form) gives the same bits as moe_forward_fused on
    the packed weights, in both orders of the GEMM phases."""
    kw = dict(kw)
    log(f"fused layer, weight tables {kw}")
    name = kw.pop("name")
    wl = custom(name, seed=8, **kw)
    w13, w2p, _ = packed_weights(wl)
    x = t_in(wl.x, wl.dtype)
    logits = t_in(wl.logits, "f32")
    ref = layer_for(wl, w13, w2p)
    ref.forward_fused(x, logits)
    assert M.moe_check_error(ref.ws) == 0
    # every expert in a buffer of its own
    b13 = [w13[i].clone() for i in range(wl.E_loc)]
    b2 = [w2p[i].clone() for i in range(wl.E_loc)]
    t13, t2 = M.weight_table(b13), M.weight_table(b2)
    fl = layer_for(wl, w13, w2p)
    a = ref.outputs()
    n = int(t_out(a["n_kept"])[0])
    try:
        for mode in ("auto", "never", "always"):
            M.moe_set_fused_overlap(mode)
            fl.y.zero_()
            M.moe_forward_fused_list(logits, x, wl.k, wl.gate, fl.capacity, wl.e_begin, wl.e_end,
                                     t13, t2, wl.f, fl.ws, fl.plan, fl.topk_idx, fl.topk_w, fl.h,
                                     fl.y_perm, fl.y)
            assert M.moe_check_error(fl.ws) == 0
            b = fl.outputs()
            for key in ("topk_idx", "topk_w", "counts", "offsets", "pair_pos", "y"):
                assert np.array_equal(t_out(a[key]), t_out(b[key])), (mode, key)
            for key in ("sorted_pair", "h", "y_perm"):
                assert np.array_equal(t_out(a[key])[:n], t_out(b[key])[:n]), (mode, key)
    finally:
        M.moe_set_fused_overlap("auto")


def test_fused_all_dropped():
    wl = custom(T=40, d=64, f=64, E=4, k=2, dtype="bf16", seed=2)
    w13, w2p, _ = packed_weights(wl)
    layer = layer_for(wl, w13, w2p, capacity=0)
    y = layer.forward_fused(t_in(wl.x, "bf16"), t_in(wl.logits, "f32"))
    assert M.moe_check_error(layer.ws) == 0
    assert int(t_out(layer.plan.n_kept)[0]) == 0
    assert np.all(t_out(layer.plan.pair_pos) == -1)
    assert np.all(t_out(y) == 0)


@pytest.mark.parametrize("kw", [
    dict(name="r1", T=300, d=128, f=128, E=8, k=2, dtype="bf16", capacity_factor=0.8,
         logit_bias="zipf"),
    dict(name="r2", T=2500, d=64, f=128, E=16, k=2, dtype="bf16", capacity_factor=1.0,
         e_begin=2, e_end=11, logit_bias="normal"),                     # several resolver chunks
    dict(name="r3", T=200, d=64, f=64, E=32, k=8, dtype="f32", capacity_factor=1.0,
         gate=O.GATE_SIGMOID, logit_bias="zipf"),
    dict(name="r4", T=90, d=64, f=64, E=4, k=4, dtype="bf16", capacity_factor=0.5),  # k = E
    dict(name="r5", T=700, d=64, f=64, E=320, k=2, dtype="bf16", capacity_factor=1.0,
         logit_bias="zipf"),                                           # more than 256 experts
])
def test_fused_layer_with_rerouting(kw):
    """moe_forward_fused_reroute against the separate calls (bit for bit) and the
    oracle's rerouting -> dispatch -> FFN -> combine."""
    kw = dict(kw)
    log(f"fused layer with rerouting {kw}")
    name = kw.pop("name")
    wl = custom(name, seed=6, **kw)
    w13, w2p, host = packed_weights(wl, keep_host=True)
    C = capacity_of(wl)
    layer = layer_for(wl, w13, w2p, reroute=True)
    x = t_in(wl.x, wl.dtype)
    logits = t_in(wl.logits, "f32")
    layer.forward(x, logits=logits)
    assert M.moe_check_error(layer.ws) == 0
    fl = fused_matches_unfused(wl, w13, w2p, layer, x, logits)
    idx, w = O.route_reroute(wl.logits, wl.k, wl.gate, C)
    plan = O.dispatch(idx, wl.E, C, wl.e_begin, wl.e_end)
    x64 = O.widen(wl.x, wl.dtype)
    y_perm = O.expert_ffn(O.permute(x64, plan["sorted_pair"], wl.k), plan["offsets"],
                          weights_fn(wl, host))
    y = O.combine(y_perm, plan["pair_pos"], w)
    out = fl.outputs()
    assert np.array_equal(t_out(out["topk_idx"]), idx)
    assert O.rel_err(t_out(out["topk_w"]), w) <= GATE_TOL
    assert np.array_equal(t_out(out["pair_pos"]), plan["pair_pos"])
    moved = int((idx[:, 0] != O.route(wl.logits, wl.k, wl.gate)[0][:, 0]).sum())
    log(f"{name}: {moved} of {wl.T} tokens rerouted")
    assert O.rel_err(as64(fl.y, wl.dtype), y) <= TOL[wl.dtype]
