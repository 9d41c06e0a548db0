"""GPU parity of each library call against the CPU oracle on small seeded inputs
(several tiles plus ragged tails), through the C ABI.

Bars: routing indices, counts, offsets, permutation, pair positions and the
permuted rows bit-exact; gates max|err|/max|ref| <= 1e-6; FFN and combine
outputs max|err|/max|ref| <= 1e-5 (fp32) and <= 1e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import routing_dispatch_expert_moe_amd as M
from oracle import moe_oracle as O
from workloads import custom, make

from gpu_util import DEV, as64, capacity_of, layer_for, log, packed_weights, t_in, t_out, weights_fn

pytestmark = pytest.mark.gpu

GATE_TOL = 1e-6
TOL = {"f32": 1e-5, "bf16": 1e-2}


def test_library_is_loaded_from_tree():
    assert torch.cuda.is_available()
    lib = M.lib()
    assert lib._name.endswith("libmoe_mi355x.so")


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("T,E,k,gate", [
    (1, 1, 1, O.GATE_SOFTMAX), (64, 8, 2, O.GATE_SOFTMAX), (300, 64, 8, O.GATE_SIGMOID),
    (257, 256, 8, O.GATE_SIGMOID), (130, 128, 2, O.GATE_SOFTMAX), (77, 1024, 8, O.GATE_SOFTMAX),
    (33, 65, 8, O.GATE_SIGMOID), (50, 8, 8, O.GATE_SOFTMAX)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_route(T, E, k, gate, kind):
    log(f"route T={T} E={E} k={k} {gate} {kind}")
    rng = np.random.default_rng(T * 7 + E)
    if kind == "normal":
        logits = rng.standard_normal((T, E)).astype(np.float32)
    else:  # coarse grid: many exact ties, plus signed zeros
        logits = (rng.integers(-3, 4, size=(T, E)) * 0.5).astype(np.float32)
        z = rng.random((T, E)) < 0.2
        logits[z] = np.where(rng.random(z.sum()) < 0.5, -0.0, 0.0).astype(np.float32)
    idx, w = M.moe_route(t_in(logits, "f32"), k, gate)
    ridx, rw = O.route(logits, k, gate)
    assert np.array_equal(t_out(idx), ridx)
    assert O.rel_err(t_out(w), rw) <= GATE_TOL


# routing with capacity-overflow rerouting: indices bit-exact, gates 1e-6,
# and the dispatch plan that follows it
@pytest.mark.parametrize("T,E,k,gate,cap", [
    (200, 8, 2, O.GATE_SOFTMAX, 30), (257, 16, 4, O.GATE_SIGMOID, 40), (130, 64, 8, O.GATE_SOFTMAX, 5),
    (100, 4, 4, O.GATE_SOFTMAX, 10),          # k == E: nothing to reroute to
    (64, 8, 1, O.GATE_SIGMOID, 0),            # capacity 0: every token reroutes
    (77, 1024, 8, O.GATE_SIGMOID, 1), (300, 32, 2, O.GATE_SOFTMAX, -1),
    # several LDS chunks of candidates (1024, 768 and 384 tokens for k = 1..2, 4, 8), ragged last
    (2500, 16, 2, O.GATE_SOFTMAX, 250), (3001, 8, 1, O.GATE_SIGMOID, 330),
    (1000, 32, 4, O.GATE_SIGMOID, 110), (1700, 64, 8, O.GATE_SOFTMAX, 190)])
@pytest.mark.parametrize("kind", ["skewed", "ties"])
def test_route_reroute(T, E, k, gate, cap, kind):
    log(f"reroute T={T} E={E} k={k} {gate} cap={cap} {kind}")
    rng = np.random.default_rng(T + E + k)
    if kind == "skewed":
        logits = (rng.standard_normal((T, E)) + rng.standard_normal(E) * 1.5).astype(np.float32)
    else:
        logits = (rng.integers(-2, 3, size=(T, E)) * 0.5).astype(np.float32)
    ws = M.alloc_workspace(T, E, k, E)
    idx, w = M.moe_route_reroute(t_in(logits, "f32"), k, gate, cap, ws)
    ridx, rw = O.route_reroute(logits, k, gate, cap)
    assert np.array_equal(t_out(idx), ridx)
    assert O.rel_err(t_out(w), rw) <= GATE_TOL
    plan = M.moe_dispatch(idx, E, cap, 0, E, None, ws, d=64)
    ref = O.dispatch(ridx, E, cap, 0, E)
    assert np.array_equal(t_out(plan.offsets), ref["offsets"])
    assert np.array_equal(t_out(plan.pair_pos)[:T * k], ref["pair_pos"])
    assert M.moe_check_error(ws) == 0


def test_route_reroute_ep_rank_shape():
    # the EP-rank routing shape (T 16384, E 128, k 2, capacity 320, biased logits)
    wl = make("ep_rank_share")
    C = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    ws = M.alloc_workspace(wl.T, wl.E, wl.k, wl.E_loc)
    idx, w = M.moe_route_reroute(t_in(wl.logits, "f32"), wl.k, wl.gate, C, ws)
    ridx, rw = O.route_reroute(wl.logits, wl.k, wl.gate, C)
    assert np.array_equal(t_out(idx), ridx)
    assert O.rel_err(t_out(w), rw) <= GATE_TOL
    base, _ = O.route(wl.logits, wl.k, wl.gate)
    moved = int((ridx[:, 0] != base[:, 0]).sum())
    log(f"reroute at the EP-rank shape: {moved} of {wl.T} tokens took their third expert")
    assert moved > 0


def test_route_all_equal_rows_exact():
    logits = np.full((10, 256), 1.5, dtype=np.float32)
    idx, w = M.moe_route(t_in(logits, "f32"), 8, O.GATE_SIGMOID)
    assert (t_out(idx) == np.arange(8)).all()
    assert (t_out(w) == np.float32(0.125)).all()


def test_router_logits():
    rng = np.random.default_rng(5)
    # E > 64: tiles of 16 tokens (few tiles) or 64 tokens by 64 experts,
    # ragged in tokens, experts and the last K chunk
    for T, d, E in [(37, 256, 8), (300, 4096, 8), (5, 64, 64), (70, 512, 17),
                    (130, 7168, 256), (65, 264, 100), (3, 72, 1024), (200, 1024, 65),
                    (8192, 256, 256), (4100, 136, 520)]:
        log(f"router T={T} d={d} E={E}")
        wl = custom(T=T, d=d, f=64, E=E, k=1, logits_from_gate=True, seed=T)
        got = M.moe_router_logits(t_in(wl.x, "bf16"), t_in(wl.w_gate, "f32"))
        ref = O.router_logits(O.widen(wl.x, "bf16"), wl.w_gate.astype(np.float64))
        assert O.rel_err(t_out(got), ref) <= 1e-5


# ---------------------------------------------------------------- dispatch
@pytest.mark.parametrize("T,E,k,cap,e0,e1", [
    (1, 1, 1, -1, 0, 1), (64, 8, 2, -1, 0, 8), (300, 16, 4, 40, 0, 16), (700, 64, 8, 60, 16, 48),
    (1000, 128, 2, 0, 0, 32), (513, 256, 8, -1, 0, 256), (257, 1024, 8, 3, 100, 900),
    (200, 8, 2, 1000, 2, 3), (600, 4, 4, 150, 0, 4),
    # the scan's split of each expert's blocks over several threads: 79 blocks
    # over 16 parts (ragged last part); more than 512 experts: one thread each
    (20000, 64, 2, 700, 0, 64), (3000, 600, 4, -1, 100, 500)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dispatch(T, E, k, cap, e0, e1, dtype):
    log(f"dispatch T={T} E={E} k={k} cap={cap} [{e0},{e1}) {dtype}")
    rng = np.random.default_rng(T + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    d = 64 if dtype == "bf16" else 32
    wl = custom(T=T, d=d, f=64, E=E, k=k, dtype=dtype, seed=1)
    ridx, _ = O.route(logits, k, O.GATE_SOFTMAX)
    ref = O.dispatch(ridx, E, cap, e0, e1)
    ws = M.alloc_workspace(T, E, k, e1 - e0)
    plan = M.moe_dispatch(torch.from_numpy(ridx).to(DEV), E, cap, e0, e1, t_in(wl.x, dtype), ws)
    assert M.moe_check_error(ws) == 0
    n = ref["n_kept"]
    assert int(t_out(plan.n_kept)[0]) == n
    assert np.array_equal(t_out(plan.counts), ref["counts"])
    assert np.array_equal(t_out(plan.offsets), ref["offsets"])
    assert np.array_equal(t_out(plan.sorted_pair)[:n], ref["sorted_pair"])
    assert np.array_equal(t_out(plan.pair_pos)[:T * k], ref["pair_pos"])
    assert np.array_equal(t_out(plan.x_perm)[:n], O.permute(wl.x, ref["sorted_pair"], k))


def test_dispatch_flags_invalid_index():
    idx = torch.tensor([[0, 1], [2, 9]], dtype=torch.int32, device=DEV)
    ws = M.alloc_workspace(2, 4, 2, 4)
    M.moe_dispatch(idx, 4, -1, 0, 4, None, ws, d=8)
    assert M.moe_check_error(ws) == M._lib.MOE_ERR_INVALID_TOPK
    assert M.moe_check_error(ws) == 0   # flag cleared
    dup = torch.tensor([[3, 3]], dtype=torch.int32, device=DEV)
    M.moe_dispatch(dup, 4, -1, 0, 4, None, ws, d=8)
    assert M.moe_check_error(ws) == M._lib.MOE_ERR_INVALID_TOPK


# ---------------------------------------------------------------- expert FFN
@pytest.mark.parametrize("dtype,d,f,rows", [
    ("bf16", 64, 64, [1]), ("bf16", 128, 192, [0, 5, 130, 0, 257]), ("bf16", 256, 512, [300, 31, 64]),
    ("bf16", 192, 128, [40] * 8), ("bf16", 128, 128, [3, 2, 7, 0, 1, 11, 4, 5, 6, 9]),
    # large/small tile split boundaries: 256-row blocks, remainders of 127/128, empty experts
    ("bf16", 128, 192, [1024, 1152, 1100, 128, 127, 255, 256, 0, 384, 513]),
    # many tiles per pass (256 experts x 4 weight tiles each way): experts with
    # a full 256-row block keep their short last block (44 or 88 rows) in the
    # large tiles, the 50-row experts go to the small tiles
    ("bf16", 1024, 512, [50] * 200 + [300] * 20 + [600] * 10 + [160] * 10 + [512] * 10 + [0] * 6),
    # few tiles and more than 512 rows per expert by the host's bound: the up pass
    # runs every row in 256-row tiles (K = d <= 4096), the down pass (K = f > 4096)
    # 256-row tiles over the full blocks and 128-row remainder tiles (88, 6, 8 rows)
    ("bf16", 128, 4160, [600, 600]), ("bf16", 192, 4352, [1030, 520]),
    ("f32", 128, 256, [17, 0, 111]), ("f32", 32, 48, [5, 70, 1]), ("f32", 12, 20, [3, 64, 65])])
def test_expert_ffn(dtype, d, f, rows):
    log(f"ffn {dtype} d={d} f={f} rows={rows}")
    E_loc = len(rows)
    wl = custom(T=max(sum(rows), 1), d=d, f=f, E=E_loc, k=1, dtype=dtype, seed=d + f)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    n = int(offsets[-1])
    x = wl.x[:n] if n else wl.x[:0]
    w13, w2p, host = packed_weights(wl, keep_host=True)
    max_rows = n + 3
    xt = torch.zeros((max(max_rows, 1), d), dtype=w13.dtype, device=DEV)
    if n:
        xt[:n] = t_in(x, dtype)
    off_t = torch.from_numpy(offsets).to(DEV)
    h, y = M.moe_expert_ffn(xt, off_t, E_loc, max_rows, w13, w2p)
    ref = O.expert_ffn(O.widen(x, dtype), offsets, weights_fn(wl, host))
    if n:
        assert O.rel_err(as64(y[:n], dtype), ref) <= TOL[dtype]
        # h against its own definition
        w = weights_fn(wl, host)
        for i in range(E_loc):
            r0, r1 = offsets[i], offsets[i + 1]
            if r1 > r0:
                w1, w3, _ = w(i)
                href = O.swiglu_hidden(O.widen(x[r0:r1], dtype), w1, w3)
                assert O.rel_err(as64(h[r0:r1], dtype), href) <= TOL[dtype]


# per-expert weight buffers through a pointer table (TensorList): the same
# kernels and bits as the packed tensor, and the oracle's values
@pytest.mark.parametrize("dtype,d,f,rows", [
    ("bf16", 128, 192, [1024, 1152, 1100, 128, 127, 255, 256, 0, 384, 513]),  # 256-row + remainder tiles
    ("bf16", 256, 512, [300, 31, 64]),
    ("bf16", 128, 128, [3, 2, 7, 0, 1, 11, 4, 5, 6, 9]),                        # few rows per expert
    ("f32", 128, 256, [17, 0, 111])])
def test_expert_ffn_list(dtype, d, f, rows):
    log(f"ffn list {dtype} d={d} f={f} rows={rows}")
    E_loc = len(rows)
    wl = custom(T=max(sum(rows), 1), d=d, f=f, E=E_loc, k=1, dtype=dtype, seed=7 * d + f)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    n = int(offsets[-1])
    w13, w2p, host = packed_weights(wl, keep_host=True)
    # one allocation per expert, made in reverse order
    l13, l2 = [None] * E_loc, [None] * E_loc
    for i in reversed(range(E_loc)):
        l13[i] = w13[i].clone()
        l2[i] = w2p[i].clone()
    t13, t2 = M.weight_table(l13), M.weight_table(l2)
    max_rows = n + 3
    xt = torch.zeros((max(max_rows, 1), d), dtype=w13.dtype, device=DEV)
    if n:
        xt[:n] = t_in(wl.x[:n], dtype)
    off_t = torch.from_numpy(offsets).to(DEV)
    h0, y0 = M.moe_expert_ffn(xt, off_t, E_loc, max_rows, w13, w2p)
    h1, y1 = M.moe_expert_ffn_list(xt, off_t, E_loc, max_rows, t13, t2, d, f)
    assert np.array_equal(t_out(h1)[:n], t_out(h0)[:n])
    assert np.array_equal(t_out(y1)[:n], t_out(y0)[:n])
    ref = O.expert_ffn(O.widen(wl.x[:n], dtype), offsets, weights_fn(wl, host))
    assert O.rel_err(as64(y1, dtype)[:n], ref) <= TOL[dtype]


def test_pack_weights_layout():
    wl = custom(T=4, d=64, f=128, E=3, k=1, dtype="bf16", seed=3)
    w13, w2p, host = packed_weights(wl, keep_host=True)
    a, b, c = t_out(w13), t_out(w2p), host
    for e in range(3):
        assert np.array_equal(a[e, :128], c[e][0].T)
        assert np.array_equal(a[e, 128:], c[e][1].T)
        assert np.array_equal(b[e], c[e][2].T)


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("dtype,T,k,d", [("bf16", 300, 2, 256), ("bf16", 65, 8, 64),
                                         ("f32", 100, 3, 12), ("f32", 1, 1, 4)])
def test_combine(dtype, T, k, d):
    log(f"combine {dtype} T={T} k={k} d={d}")
    rng = np.random.default_rng(T)
    E = 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = O.route(logits, k, O.GATE_SOFTMAX)
    plan = O.dispatch(idx, E, max(1, T * k // E), 0, 12)   # some drops, some remote
    n = plan["n_kept"]
    yp = rng.standard_normal((max(n, 1), d)).astype(np.float32)
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        yp = f32_to_bf16_bits(yp)
    w32 = w.astype(np.float32)
    y = M.moe_combine(t_in(yp, dtype), torch.from_numpy(plan["pair_pos"]).to(DEV), t_in(w32, "f32"))
    ref = O.combine(O.widen(yp, dtype)[:n], plan["pair_pos"], w32.astype(np.float64))
    assert O.rel_err(as64(y, dtype), ref) <= TOL[dtype]
    # tokens with no local kept pair are exact zeros
    none = (plan["pair_pos"].reshape(T, k) < 0).all(axis=1)
    assert np.all(as64(y, dtype)[none] == 0)


# ---------------------------------------------------------------- whole layer, small
@pytest.mark.parametrize("kw", [
    dict(name="tiny", T=64, d=128, f=256, E=8, k=2, dtype="f32"),
    dict(name="b1", T=200, d=128, f=192, E=8, k=2, dtype="bf16"),
    dict(name="b2", T=150, d=256, f=128, E=32, k=8, dtype="bf16", gate=O.GATE_SIGMOID),
    dict(name="b3", T=333, d=128, f=128, E=16, k=2, dtype="bf16", capacity_factor=1.25,
         e_begin=4, e_end=12, logit_bias="normal"),
    dict(name="b4", T=257, d=192, f=256, E=64, k=4, dtype="bf16", logit_bias="zipf"),
    dict(name="b5", T=100, d=64, f=64, E=4, k=2, dtype="bf16", capacity_factor=0.25),
])
def test_layer_small(kw):
    kw = dict(kw)
    log(f"layer {kw}")
    name = kw.pop("name")
    wl = custom(name, seed=11, **kw)
    w13, w2p, host = packed_weights(wl, keep_host=True)
    layer = layer_for(wl, w13, w2p)
    x = t_in(wl.x, wl.dtype)
    y = layer.forward(x, logits=t_in(wl.logits, "f32"))
    assert M.moe_check_error(layer.ws) == 0
    ref = O.moe_layer(wl.x, wl.dtype, wl.logits, wl.k, wl.gate, weights_fn(wl, host), wl.E,
                      capacity_of(wl), wl.e_begin, wl.e_end)
    out = layer.outputs()
    n = ref["n_kept"]
    assert np.array_equal(t_out(out["topk_idx"]), ref["topk_idx"])
    assert O.rel_err(t_out(out["topk_w"]), ref["topk_w"]) <= GATE_TOL
    assert np.array_equal(t_out(out["offsets"]), ref["offsets"])
    assert np.array_equal(t_out(out["sorted_pair"])[:n], ref["sorted_pair"])
    assert np.array_equal(t_out(out["pair_pos"]), ref["pair_pos"])
    assert O.rel_err(as64(y, wl.dtype), ref["y"]) <= TOL[wl.dtype]
    # determinism: a second pass is bitwise identical
    y1 = t_out(y).copy()
    layer.forward(x, logits=t_in(wl.logits, "f32"))
    assert np.array_equal(t_out(layer.y), y1)


def test_empty_batch_and_all_dropped():
    wl = custom(T=40, d=64, f=64, E=4, k=2, dtype="bf16", seed=2)
    w13, w2p, _ = packed_weights(wl)
    layer = layer_for(wl, w13, w2p, capacity=0)
    y = layer.forward(t_in(wl.x, "bf16"), logits=t_in(wl.logits, "f32"))
    assert int(t_out(layer.plan.n_kept)[0]) == 0
    assert np.all(t_out(y) == 0)
    # T = 0 is a no-op everywhere
    z = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    idx, w = M.moe_route(z, 2, O.GATE_SOFTMAX)
    assert idx.shape == (0, 2)
