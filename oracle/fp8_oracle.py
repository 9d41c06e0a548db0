"""CPU oracle of FP8 expert weights: E4M3 encoding, 128 x 128 block scales, dequantisation.

TEST INFRASTRUCTURE ONLY.  Like moe_oracle, this module is the plain reference
the GPU library is checked against; only the test suite, the package smoke
check and the CPU-baseline leg of the benchmark may import it, and it shares
no code, table or helper with the library.

Source: NCCL EP page ("NCCL EP架构解析"), §2.1, expert-compute stage: the
experts compute in FP8, which needs a scale tensor next to the quantised
weights.  The page gives neither the FP8 format nor the scale granularity;
the readings below fix them (each also listed in the design notes):

  R22 Format: E4M3 in the OCP "FN" flavour (1 sign, 4 exponent bits with bias
      7, 3 mantissa bits; no infinities; S.1111.111 is NaN), the FP8 type of
      gfx950.  Largest finite magnitude 448, smallest normal 2^-6, smallest
      subnormal 2^-9.
  R23 Scales: one fp32 scale per block of 128 rows x 128 K-columns of each
      expert's packed (K-contiguous) weight matrix: W1 || W3 rows for the
      first GEMM, W2^T rows for the second.  scale = the smallest power of
      two 2^e with amax <= 448 * 2^e (amax = the block's largest |w|), so the
      block's largest code lies in (224, 448] and nothing saturates; an
      all-zero block gets scale 1.  (A power of two, as the shared exponents
      of the OCP microscaling formats are, makes code * scale exactly
      representable in bf16.)
  R24 Codes: q = E4M3(w / scale) with the division in fp32 (exact for a power
      of two) and the rounding to nearest, ties to the even code, saturating
      at +-448 (no NaN is ever produced).  Weights are the exact bf16 inputs.
  R25 The method computes with the dequantised weights decode(q) * scale;
      activations (x, h) stay bf16 and the GEMMs accumulate in fp32, so the
      oracle's FFN is moe_oracle's FFN applied to the dequantised weights.

Pins: tests/test_oracle_fp8.py (the format's defining values, a brute-force
nearest-code search over the whole code table, round trips, the block
scale's defining property and the quantisation error bound).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3-FN code (uint8) as float64; NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m.astype(np.float64), -9)  # m * 2^-9 (e == 0)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


# the 127 non-negative finite values, ascending (code c has value _POS[c])
_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3-FN codes: nearest value, ties to the even
    code (even mantissa), magnitudes at or above 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    neg = np.signbit(x)
    # the quantum of the binade containing a (subnormals share 2^-9)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                        # floor(log2 a), at least -6
    quantum = np.ldexp(1.0, e - 3)
    q = np.rint(a / quantum)                          # a / quantum is exact; rint = ties to even
    v = np.minimum(q * quantum, E4M3_MAX)
    code = np.searchsorted(_POS, v).astype(np.int64)  # v is one of _POS exactly
    assert np.all(_POS[np.minimum(code, 0x7E)] == v)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """The smallest integer e with amax <= 448 * 2^e, for amax > 0 (exact:
    amax = m * 2^ex with m in [0.5, 1) and 448 = 0.875 * 2^9)."""
    m, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    return np.where(m <= 0.875, ex - 9, ex - 8)


def quantize_blocks(w_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise packed bf16 weights [E][R][K] (uint16 bit patterns; R, K
    multiples of 128) to (codes uint8 [E][R][K], scales float32
    [E][R/128][K/128])."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    E, R, K = w_bits.shape
    assert R % BLOCK == 0 and K % BLOCK == 0
    w = (w_bits.astype(np.uint32) << 16).view(np.float32)
    blocks = w.reshape(E, R // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=(2, 4)).astype(np.float64)       # [E][R/128][K/128]
    scale = np.where(amax > 0, np.ldexp(1.0, scale_exponent(amax)), 1.0).astype(np.float32)
    ratio = (blocks / scale[:, :, None, :, None]).astype(np.float32)  # fp32 division
    codes = e4m3_encode(ratio).reshape(E, R, K)
    return codes, scale


def dequantize_blocks(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """decode(q) * scale in float64 (exact), [E][R][K]."""
    E, R, K = codes.shape
    v = e4m3_decode(codes).reshape(E, R // BLOCK, BLOCK, K // BLOCK, BLOCK)
    v = v * scale.astype(np.float64)[:, :, None, :, None]
    return v.reshape(E, R, K)


def expert_weights(w13_codes, w13_scale, w2_codes, w2_scale, f: int):
    """Per-expert (W1 [d, f], W3 [d, f], W2 [f, d]) in float64 from the
    quantised packed operands (w13 rows 0..f-1 are W1^T, f..2f-1 are W3^T;
    w2 rows are W2^T), in the x.W orientation moe_oracle expects."""
    w13 = dequantize_blocks(w13_codes, w13_scale)
    w2 = dequantize_blocks(w2_codes, w2_scale)

    def weights(i: int):
        return (w13[i, :f].T.copy(), w13[i, f:].T.copy(), w2[i].T.copy())
    return weights
