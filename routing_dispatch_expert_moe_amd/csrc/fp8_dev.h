// E4M3-FN (OCP FP8: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, S.1111.111 = NaN) conversions for the FP8 expert weights.
//
// NCCL EP page, §2.1 (expert-compute stage): the experts compute in FP8 with
// a scale tensor beside the quantised weights.  Weights are stored as E4M3
// codes with one fp32 scale per 128 x 128 block of each expert's packed
// weight matrix.  (The GEMMs decode codes with the hardware conversion to
// bf16, which is exact for E4M3, and apply the scales to partial sums.)
#pragma once

#include "common.h"

namespace moe {

constexpr int kFp8Block = 128;        // rows and K-columns covered by one scale
constexpr float kE4M3Max = 448.0f;    // largest finite E4M3-FN magnitude

// value -> code: nearest E4M3 value, ties to the even code, magnitudes from
// 448 up saturate to 448.  Normal results keep the top 3 of fp32's 23
// mantissa bits with round-to-nearest-even on the 20 dropped bits (a carry
// moves into the exponent); below 2^-6 the values are multiples of 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (a >= 0x43E00000u) {          // |x| >= 448
    c = 0x7Eu;
  } else if (a < 0x3C800000u) {    // |x| < 2^-6
    c = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  } else {
    c = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | c;
}

}  // namespace moe
