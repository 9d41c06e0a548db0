"""GPU parity of the FP8-weight calls against the CPU oracle (oracle/fp8_oracle.py):
the E4M3 codes and block scales bit-exact, the expert FFN on dequantised
weights within the bf16 bar (max|err| / max|ref| <= 1e-2)."""
import numpy as np
import pytest
import torch

import routing_dispatch_expert_moe_amd as M
from oracle import fp8_oracle as F
from oracle import moe_oracle as O
from workloads import custom, make

from gpu_util import DEV, as64, log, packed_weights, t_in, t_out

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
    (512, 256, [300, 0, 513]),                    # many rows: 128-row tiles, ragged tails
    (384, 640, [129, 127, 256, 1]),
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
    assert O.rel_err(as64(y, "bf16")[:n], ref) <= TOL
    for i in range(E_loc):
        r0, r1 = offsets[i], offsets[i + 1]
        if r1 > r0:
            w1, w3, _ = wf(i)
            href = O.silu(x64[r0:r1] @ w1) * (x64[r0:r1] @ w3)
            assert O.rel_err(as64(h, "bf16")[r0:r1], href) <= TOL
    # same bits on a second call
    y1 = t_out(y).copy()
    M.moe_expert_ffn_fp8(xt, off_t, E_loc, max_rows, q13, s13, q2, s2, h, y)
    assert np.array_equal(t_out(y), y1)


def test_decode_layer_fp8_sampled_tokens():
    """The DeepSeek-shaped decode layer (T=128, E=256, k=8, d=7168, f=2048) with
    FP8 weights end to end; sampled tokens against the oracle on their experts."""
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
    x64 = O.widen(wl.x, "bf16")
    for t in (0, 77):
        yt = np.zeros(wl.d)
        for j in range(wl.k):
            e = int(idx[t, j])
            w1, w3, w2 = wl.expert_weights(e)
            h13, h2 = _host_packed([(w1, w3, w2)], wl.f)
            a, sa = F.quantize_blocks(h13)
            b, sb = F.quantize_blocks(h2)
            assert np.array_equal(t_out(q13[e:e + 1]), a) and np.array_equal(t_out(s13[e:e + 1]), sa)
            W1, W3, W2 = F.expert_weights(a, sa, b, sb, wl.f)(0)
            yt += gw[t, j] * O.swiglu_ffn(x64[t:t + 1], W1, W3, W2)[0]
        err = np.abs(got[t] - yt).max() / np.abs(yt).max()
        log(f"decode fp8 token {t}: rel err {err:.2e}")
        assert err <= TOL
