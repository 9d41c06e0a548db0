"""Pins of the FP8 (E4M3-FN) weight oracle: format values, rounding by brute
force over the code table, round trips, block scales and their error bound."""
import numpy as np

from oracle import fp8_oracle as F
from oracle import moe_oracle as O


def test_defining_values():
    # OCP E4M3-FN: bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x44: 3.0, 0x7E: 448.0,
             0xB0: -0.5, 0xFE: -448.0}
    for c, v in cases.items():
        assert F.e4m3_decode(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(F.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    neg0 = F.e4m3_decode(np.array([0x80], np.uint8))[0]
    assert neg0 == 0.0 and np.signbit(neg0)


def test_positive_codes_are_ascending_and_distinct():
    v = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert v[-1] == F.E4M3_MAX


def _brute_force(x):
    """Nearest finite E4M3 value by exhaustive search; ties to the even code."""
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    out = np.empty(len(x), np.uint8)
    for i, xi in enumerate(np.asarray(x, np.float32).astype(np.float64)):
        d = np.abs(vals - abs(xi))
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        out[i] = c | (0x80 if np.signbit(np.float32(xi)) else 0)
    return out


def test_encode_matches_brute_force_nearest():
    rng = np.random.default_rng(0)
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2                     # exact ties (fp32-representable)
    x = np.concatenate([
        rng.standard_normal(3000) * 50,
        rng.standard_normal(1000) * 1e-2,               # subnormal range
        np.exp(rng.uniform(np.log(1e-4), np.log(1e4), 2000)) * rng.choice([-1, 1], 2000),
        mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
        [0.0, -0.0, 448.0, 455.0, 464.0, 470.0, 1e6, -1e9, 2.0 ** -10, 2.0 ** -10 * 3],
    ]).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(x), _brute_force(x))


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes).astype(np.float32)), codes)


def _bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_block_scale_hand_example():
    # a block whose largest magnitude is exactly 448: the scale is 1 and the
    # codes are the plain E4M3 codes of the weights
    w = np.zeros((1, 128, 128), np.float32)
    w[0, 0, 0] = 448.0
    w[0, 1, 2] = 1.0
    w[0, 2, 3] = -0.5
    w[0, 3, 4] = 3.0
    w[0, 4, 5] = 1.0625          # tie between 1.0 (even) and 1.125 -> 1.0
    q, s = F.quantize_blocks(_bf16(w))
    assert s.shape == (1, 1, 1) and s[0, 0, 0] == 1.0
    assert (q[0, 0, 0], q[0, 1, 2], q[0, 2, 3], q[0, 3, 4], q[0, 4, 5]) == (0x7E, 0x38, 0xB0, 0x44, 0x38)
    assert np.count_nonzero(q) == 5


def test_power_of_two_scale_hand_example():
    # block 0: amax 450 (a bf16 value): 450 > 448 * 1, 450 <= 448 * 2, so the
    # scale is 2; 450 / 2 = 225 lies in the binade [128, 256) of quantum 16 and
    # rounds to 224 = 1.75 * 2^7, code (7 + 7) << 3 | 6 = 0x76.
    # block 1: amax 1.0: 1 <= 448 * 2^-8 = 1.75 but 1 > 448 * 2^-9 = 0.875, so
    # the scale is 2^-8; 1.0 -> 256 = 2^8, code 15 << 3 = 0x78; bf16(0.3) =
    # 0.30078125 -> 77, quantum 8 in [64, 128): 9.625 quanta -> 10 -> 80 =
    # 1.25 * 2^6, code 13 << 3 | 2 = 0x6A, dequantised 80 / 256 = 0.3125.
    w = np.zeros((1, 128, 256), np.float32)
    w[0, 5, 7] = 450.0
    w[0, 9, 130] = 1.0
    w[0, 10, 140] = 0.3
    q, s = F.quantize_blocks(_bf16(w))
    assert s.shape == (1, 1, 2) and s[0, 0, 0] == 2.0 and s[0, 0, 1] == 2.0 ** -8
    assert (q[0, 5, 7], q[0, 9, 130], q[0, 10, 140]) == (0x76, 0x78, 0x6A)
    deq = F.dequantize_blocks(q, s)
    assert (deq[0, 5, 7], deq[0, 9, 130], deq[0, 10, 140]) == (448.0, 1.0, 0.3125)


def test_zero_block_and_block_independence():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((2, 256, 384)).astype(np.float32) * 0.02
    w[1, 128:, 256:] = 0.0
    q, s = F.quantize_blocks(_bf16(w))
    assert s.shape == (2, 2, 3)
    assert s[1, 1, 2] == 1.0 and not q[1, 128:, 256:].any()
    # each block quantised on its own: scaling one block leaves the others' codes alone
    w2 = w.copy()
    w2[0, :128, :128] *= 1000.0
    q2, s2 = F.quantize_blocks(_bf16(w2))
    mask = np.ones(q.shape, bool)
    mask[0, :128, :128] = False
    assert np.array_equal(q[mask], q2[mask])
    assert np.array_equal(np.delete(s.ravel(), 0), np.delete(s2.ravel(), 0))


def test_block_scale_property_and_error_bound():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((3, 256, 256)) * rng.uniform(1e-3, 10, (3, 1, 1))).astype(np.float32)
    bits = _bf16(w)
    q, s = F.quantize_blocks(bits)
    wexact = O.widen(bits, "bf16")
    deq = F.dequantize_blocks(q, s)
    blocks = wexact.reshape(3, 2, 128, 2, 128)
    amax = np.abs(blocks).max(axis=(2, 4))
    # the scale is a power of two, the smallest with amax / scale <= 448
    s64 = s.astype(np.float64)
    mant, _ = np.frexp(s64)
    assert np.all(mant == 0.5)
    assert np.all(amax / s64 <= 448.0) and np.all(amax / (s64 / 2) > 448.0)
    # so the block's largest code lies in [224, 448] and none saturates
    qa = np.abs(F.e4m3_decode(q)).reshape(3, 2, 128, 2, 128).max(axis=(2, 4))
    assert np.all((qa >= 224.0) & (qa <= 448.0))
    # |dequant - w| <= half a quantum of |w / scale| (plus the fp32 division's rounding)
    r = np.abs(wexact) / np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)
    _, ex = np.frexp(np.where(r > 0, r, 1.0))
    half_q = np.ldexp(1.0, np.maximum(ex - 1, -6) - 4)
    bound = (half_q * (1 + 2.0 ** -20) + r * 2.0 ** -23) * np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)
    assert np.all(np.abs(deq - wexact) <= bound)
    # relative error of the whole tensor: a few per cent at 3 mantissa bits
    assert O.rel_err(deq, wexact) < 0.07


def test_representable_weights_reduce_to_the_bf16_ffn():
    # weights that are E4M3 values with a 448 in every block: scale 1, exact dequantisation,
    # so the FP8 expert FFN equals the plain FFN of the same weights
    rng = np.random.default_rng(3)
    pos = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    d, f, n = 128, 256, 20

    def draw(shape):
        v = rng.choice(pos[40:100], size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v[..., 0, 0] = 448.0
        return v.astype(np.float32)
    w13 = draw((1, 2 * f, d))
    w13[0, 128::128, 0] = 448.0
    w13[0, 0, ::128] = 448.0
    w2 = draw((1, d, f))
    w2[0, 0, ::128] = 448.0
    q13, s13 = F.quantize_blocks(_bf16(w13))
    q2, s2 = F.quantize_blocks(_bf16(w2))
    assert np.all(s13 == 1.0) and np.all(s2 == 1.0)
    wf = F.expert_weights(q13, s13, q2, s2, f)
    w1, w3, w2t = wf(0)
    assert np.array_equal(w1, w13[0, :f].T.astype(np.float64))
    assert np.array_equal(w3, w13[0, f:].T.astype(np.float64))
    assert np.array_equal(w2t, w2[0].T.astype(np.float64))
    x = (rng.standard_normal((n, d)) * 1e-3).astype(np.float32)
    offsets = np.array([0, n], np.int32)
    got = O.expert_ffn(x.astype(np.float64), offsets, wf)
    ref = O.expert_ffn(x.astype(np.float64), offsets,
                       lambda i: (w13[0, :f].T.astype(np.float64), w13[0, f:].T.astype(np.float64),
                                  w2[0].T.astype(np.float64)))
    assert np.array_equal(got, ref)
