"""GPU parity of the FP8-weight calls against the CPU oracle (oracle/fp8_oracle.py):
the E4M3 codes and block scales bit-exact, the expert FFN on dequantised
weights within the bf16 bar (max|err| / max|ref| <= 1e-2)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import routing_dispatch_expert_moe_amd as M
from oracle import fp8_oracle as F
from oracle import moe_oracle as O
from workloads import custom, make

from gpu_util import DEV, as64, barrier_order_matches, log, packed_weights, t_in, t_out

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _bf16_bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _quantize_both(bits):
    """GPU codes/scales and the oracle's for packed bf16 bits [E][R][K]."""
    w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    q, s = M.moe_quantize_fp8(w)
    rq, rs = F.quantize_blocks(bits)
    return t_out(q), t_out(s), rq, rs


def test_quantize_random_blocks():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((3, 256, 384)).astype(np.float32)
    w *= rng.uniform(1e-4, 30, (3, 1, 384)).astype(np.float32)    # magnitudes vary by column
    w[1, :128, 128:256] = 0.0                                         # an all-zero block
    w[2, 128:, :128] *= 1e-3
    w[2, 200, 50] = 7.0                                               # one large value: the rest go subnormal
    q, s, rq, rs = _quantize_both(_bf16_bits(w))
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)


def test_quantize_every_bf16_value_with_unit_scale():
    # every finite bf16 of magnitude below 448 (ties between E4M3 values included),
    # in blocks whose largest magnitude is exactly 448, so the scale is 1 and the
    # codes are the plain E4M3 rounding of each bf16 value
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (pats.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) < 448.0)
    pats = pats[keep]
    per = 128 * 128 - 1
    nblk = -(-len(pats) // per)
    blocks = np.zeros((nblk, 128 * 128), np.uint16)
    for b in range(nblk):
        chunk = pats[b * per:(b + 1) * per]
        blocks[b, :len(chunk)] = chunk
        blocks[b, -1] = _bf16_bits(np.float32(448.0))
    bits = blocks.reshape(nblk, 128, 128)
    q, s, rq, rs = _quantize_both(bits)
    assert np.all(s == 1.0) and np.array_equal(s, rs)
    assert np.array_equal(q, rq)
    log(f"quantised {len(pats)} bf16 values exactly")


def _host_packed(host, f):
    """Packed bf16 bit arrays (w13 [E][2f][d], w2 [E][d][f]) from per-expert (W1, W3, W2)."""
    w13 = np.stack([np.concatenate([w1.T, w3.T], axis=0) for w1, w3, _ in host])
    w2 = np.stack([w2.T for _, _, w2 in host])
    return np.ascontiguousarray(w13), np.ascontiguousarray(w2)


@pytest.mark.parametrize("d,f,rows", [
    (256, 384, [5, 0, 40, 1]),                    # few rows per expert: 32-row tiles
    (128, 256, [3, 1, 0, 7, 2, 9, 4, 11]),
    # many rows per expert and K >= 256: the pipelined kernel (codes in LDS,
    # 128-row tiles, partial sums per 128-deep K block), ragged tiles
    (512, 256, [300, 0, 513]), (384, 640, [129, 127, 256, 1]),
    (1024, 2048, [700, 300, 0, 1100]), (256, 256, [129, 400, 77]),
    # many rows and K = 128 (up) / 256 (down): register-staged 64-row tiles, then the pipe
    (128, 256, [200, 90, 131]),
    # the bf16 passes' row classes with FP8 weights: a 4224-deep second GEMM with few
    # tiles (256-row tiles over full blocks, 128-row remainder tiles of 88 and 44 rows);
    # 64 experts x 16 weight tiles (many tiles: short last blocks ride along in the
    # 256-row tiles, the 50-row experts go to 128-row tiles)
    (256, 4224, [600, 300]),
    (256, 2048, [50] * 40 + [300] * 12 + [600] * 6 + [0] * 6),
])
def test_expert_ffn_fp8(d, f, rows):
    log(f"ffn fp8 d={d} f={f} rows={rows}")
    E_loc = len(rows)
    wl = custom(T=max(sum(rows), 1), d=d, f=f, E=E_loc, k=1, dtype="bf16", seed=d + 3 * f)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    n = int(offsets[-1])
    w13, w2p, host = packed_weights(wl, keep_host=True)
    q13, s13 = M.moe_quantize_fp8(w13)
    q2, s2 = M.moe_quantize_fp8(w2p)
    # the oracle quantises the same bf16 weights itself; the codes must agree
    h13, h2 = _host_packed(host, f)
    rq13, rs13 = F.quantize_blocks(h13)
    rq2, rs2 = F.quantize_blocks(h2)
    assert np.array_equal(t_out(q13), rq13) and np.array_equal(t_out(s13), rs13)
    assert np.array_equal(t_out(q2), rq2) and np.array_equal(t_out(s2), rs2)
    max_rows = n + 5
    xt = torch.zeros((max_rows, d), dtype=torch.bfloat16, device=DEV)
    xt[:n] = t_in(wl.x[:n], "bf16")
    off_t = torch.from_numpy(offsets).to(DEV)
    h, y = M.moe_expert_ffn_fp8(xt, off_t, E_loc, max_rows, q13, s13, q2, s2)
    x64 = O.widen(wl.x[:n], "bf16")
    wf = F.expert_weights(rq13, rs13, rq2, rs2, f)
    ref = O.expert_ffn(x64, offsets, wf)
    # rows past n are never written: slice before widening
    assert O.rel_err(as64(y[:n], "bf16"), ref) <= TOL
    for i in range(E_loc):
        r0, r1 = offsets[i], offsets[i + 1]
        if r1 > r0:
            w1, w3, _ = wf(i)
            href = O.swiglu_hidden(x64[r0:r1], w1, w3)
            assert O.rel_err(as64(h[r0:r1], "bf16"), href) <= TOL
    # same bits on a second call
    y1 = t_out(y).copy()
    M.moe_expert_ffn_fp8(xt, off_t, E_loc, max_rows, q13, s13, q2, s2, h, y)
    assert np.array_equal(t_out(y), y1)
    # the TensorList form: every expert's codes and scales in buffers of their
    # own (allocated in reverse order), same bits as the packed tensors
    bufs = [None] * E_loc
    for i in reversed(range(E_loc)):
        bufs[i] = (q13[i].clone(), s13[i].clone(), q2[i].clone(), s2[i].clone())
    tabs = [M.weight_table([b[j] for b in bufs]) for j in range(4)]
    hl, yl = M.moe_expert_ffn_fp8_list(xt, off_t, E_loc, max_rows, *tabs, f)
    assert np.array_equal(t_out(hl)[:n], t_out(h)[:n])
    assert np.array_equal(t_out(yl)[:n], y1[:n])
    # and the halves on their own
    hl.zero_()
    M.moe_ffn_up_fp8_list(xt, off_t, E_loc, max_rows, tabs[0], tabs[1], f, hl)
    yl2 = M.moe_ffn_down_fp8_list(hl, off_t, E_loc, max_rows, tabs[2], tabs[3], d)
    assert np.array_equal(t_out(hl)[:n], t_out(h)[:n])
    assert np.array_equal(t_out(yl2)[:n], y1[:n])


@pytest.mark.timeout(600)
def test_decode_layer_fp8_sampled_tokens():
    """The DeepSeek-shaped decode layer (T=128, E=256, k=8, d=7168, f=2048) with
    FP8 weights end to end: 16 tokens against the oracle on their experts, the
    experts' codes and scales bit-exact against the oracle's quantiser."""
    wl = make("dsv3_decode")
    w13, w2p, _ = packed_weights(wl, chunk=32)
    q13, s13 = M.moe_quantize_fp8(w13)
    q2, s2 = M.moe_quantize_fp8(w2p)
    del w13, w2p
    torch.cuda.empty_cache()
    C = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    layer = M.MoELayer(q13, q2, E=wl.E, k=wl.k, gate=wl.gate, T=wl.T, capacity=C,
                       w13_scale=s13, w2_scale=s2)
    y = layer.forward(t_in(wl.x, "bf16"), logits=torch.from_numpy(wl.logits).to(DEV))
    assert M.moe_check_error(layer.ws) == 0
    got = as64(y, "bf16")
    idx, gw = O.route(wl.logits, wl.k, wl.gate)
    assert np.array_equal(t_out(layer.topk_idx), idx)
    # 16 tokens chosen greedily so that they share experts (fewer to quantise on the host)
    sets = [set(r) for r in idx.tolist()]
    tokens, union = [0], set(sets[0])
    while len(tokens) < 16:
        t = min((u for u in range(wl.T) if u not in tokens), key=lambda u: len(sets[u] - union))
        tokens.append(t)
        union |= sets[t]
    x64 = O.widen(wl.x, "bf16")
    log(f"decode fp8: {len(tokens)} tokens over {len(union)} experts")

    def contribution(e):
        w1, w3, w2 = wl.expert_weights(e)
        h13, h2 = _host_packed([(w1, w3, w2)], wl.f)
        a, sa = F.quantize_blocks(h13)
        b, sb = F.quantize_blocks(h2)
        same = (np.array_equal(t_out(q13[e:e + 1]), a) and np.array_equal(t_out(s13[e:e + 1]), sa)
                and np.array_equal(t_out(q2[e:e + 1]), b) and np.array_equal(t_out(s2[e:e + 1]), sb))
        W1, W3, W2 = F.expert_weights(a, sa, b, sb, wl.f)(0)
        rows = [(i, j) for i, t in enumerate(tokens) for j in range(wl.k) if idx[t, j] == e]
        o = O.swiglu_ffn(x64[[tokens[i] for i, _ in rows]], W1, W3, W2)
        return same, rows, o

    ref = np.zeros((len(tokens), wl.d))
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        for same, rows, o in ex.map(contribution, sorted(union)):
            assert same, "FP8 codes or scales differ from the oracle's quantiser"
            for r, (i, j) in enumerate(rows):
                ref[i] += gw[tokens[i], j] * o[r]
    err = O.rel_err(got[tokens], ref)
    log(f"decode fp8: {len(tokens)} tokens rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("kw", [
    # ~128 rows per expert: 256-row tiles over every row
    dict(name="f8a", T=512, d=256, f=384, E=8, k=2),
    # capacity drops and a local expert range, ~188 rows per expert
    dict(name="f8b", T=600, d=256, f=256, E=16, k=4, capacity_factor=1.25, e_begin=2, e_end=14,
         logit_bias="normal"),
    # ~12 rows per expert: the code-streaming 32-row tiles (the fused launch runs
    # them in two parts per workgroup)
    dict(name="f8c", T=200, d=512, f=256, E=32, k=2),
    # ~12 rows per expert with 3 and 5 column tiles per expert: an odd number of
    # 32-row tiles, so one part of a fused workgroup has no tile in the last
    # round (it recomputes the last tile and stores nothing)
    dict(name="f8e", T=96, d=640, f=384, E=23, k=3),
    # a 4224-deep second GEMM with few tiles: 256-row tiles plus 128-row remainder tiles
    dict(name="f8d", T=900, d=256, f=4224, E=4, k=1),
    # 64 experts x 16 weight tiles in the first GEMM (many tiles): the ride-along
    # split, 8 experts of 128 rows or more in 256-row tiles, 56 below in 128-row tiles
    dict(name="f8f", T=1024, d=256, f=2048, E=64, k=4, logit_bias="normal"),
])
def test_fused_layer_fp8(kw):
    """moe_forward_fused_fp8 against the separate FP8 calls (bit for bit: the
    same step bodies) and the oracle on the dequantised weights."""
    kw = dict(kw)
    log(f"fused layer fp8 {kw}")
    name = kw.pop("name")
    wl = custom(name, seed=7, dtype="bf16", **kw)
    w13, w2p, host = packed_weights(wl, keep_host=True)
    q13, s13 = M.moe_quantize_fp8(w13)
    q2, s2 = M.moe_quantize_fp8(w2p)
    del w13, w2p
    C = M.moe_capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    assert C == O.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)

    def layer():
        return M.MoELayer(q13, q2, E=wl.E, k=wl.k, gate=wl.gate, T=wl.T, capacity=C,
                          e_begin=wl.e_begin, e_end=wl.e_end, w13_scale=s13, w2_scale=s2)

    x = t_in(wl.x, "bf16")
    lg = t_in(wl.logits, "f32")
    sep = layer()
    sep.forward(x, logits=lg)
    assert M.moe_check_error(sep.ws) == 0
    fl = layer()
    fl.forward_fused(x, lg)
    assert M.moe_check_error(fl.ws) == 0
    a, b = sep.outputs(), fl.outputs()
    n = int(t_out(a["n_kept"])[0])
    assert int(t_out(b["n_kept"])[0]) == n
    for key in ("topk_idx", "topk_w", "counts", "offsets", "pair_pos"):
        assert np.array_equal(t_out(a[key]), t_out(b[key])), key
    assert np.array_equal(t_out(a["sorted_pair"])[:n], t_out(b["sorted_pair"])[:n])
    for key in ("h", "y_perm"):
        assert np.array_equal(t_out(a[key])[:n], t_out(b[key])[:n]), key
    assert np.array_equal(t_out(a["y"]), t_out(b["y"]))
    if name == "f8f":
        cu = torch.cuda.get_device_properties(DEV).multi_processor_count
        mr = M.moe_max_rows(wl.T, wl.k, wl.E_loc, C)
        assert M.moe_ffn_plan("up", mr, wl.E_loc, wl.d, wl.f, "bf16", cu) == "big_ride"
    if name == "f8e":
        # the case is meant to leave a part idle: an odd 32-row tile count
        rows = np.diff(t_out(b["offsets"]).astype(np.int64))
        mt = int(((rows + 31) // 32).sum())
        assert (mt * (wl.f // 128)) % 2 == 1 or (mt * (wl.d // 128)) % 2 == 1, mt
    h13, h2 = _host_packed(host, wl.f)
    rq13, rs13 = F.quantize_blocks(h13)
    rq2, rs2 = F.quantize_blocks(h2)
    wf = F.expert_weights(rq13, rs13, rq2, rs2, wl.f)
    ref = O.moe_layer(wl.x, "bf16", wl.logits, wl.k, wl.gate, wf, wl.E, C, wl.e_begin, wl.e_end)
    assert np.array_equal(t_out(b["topk_idx"]), ref["topk_idx"])
    assert O.rel_err(as64(fl.y, "bf16"), ref["y"]) <= TOL
    y1 = t_out(fl.y).copy()
    fl.forward_fused(x, lg)
    assert M.moe_check_error(fl.ws) == 0
    assert np.array_equal(t_out(fl.y), y1)
    # the GEMM phases separated by a barrier instead of the per-expert waits
    barrier_order_matches(fl, x, lg, y1)
    # the TensorList form: every expert's codes and scales in buffers of
    # their own, same bits in each order of the GEMM phases
    bufs = [None] * wl.E_loc
    for i in reversed(range(wl.E_loc)):
        bufs[i] = (q13[i].clone(), s13[i].clone(), q2[i].clone(), s2[i].clone())
    tabs = [M.weight_table([bb[j] for bb in bufs]) for j in range(4)]
    tl = layer()
    try:
        for mode in ("auto", "never", "always"):
            M.moe_set_fused_overlap(mode)
            tl.y.zero_()
            M.moe_forward_fused_fp8_list(lg, x, wl.k, wl.gate, tl.capacity, wl.e_begin, wl.e_end,
                                         *tabs, wl.f, tl.ws, tl.plan, tl.topk_idx, tl.topk_w,
                                         tl.h, tl.y_perm, tl.y)
            assert M.moe_check_error(tl.ws) == 0
            c = tl.outputs()
            assert np.array_equal(t_out(c["y"]), y1), mode
            for key in ("h", "y_perm"):
                assert np.array_equal(t_out(c[key])[:n], t_out(b[key])[:n]), (mode, key)
    finally:
        M.moe_set_fused_overlap("auto")
