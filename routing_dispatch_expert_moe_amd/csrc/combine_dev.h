// Weighted combine (NCCL EP page §2.1, LL combine): for each token, the sum
// over its k choices of gate weight times that pair's expert output row.
// One wave per token; 16-byte loads of every contributing row; fp32
// accumulation in ascending j; one rounding at the store.  No atomics: each
// output row is owned by exactly one wave, so the result is deterministic.
#pragma once

#include "common.h"

namespace moe {

// Output row of token t, computed by one whole wave.  topk_w == nullptr: every
// weight is 1 (the plain sum of the token's rows, as the backward pass needs
// for the input gradient).
template <bool BF16>
__device__ __forceinline__ void combine_token(const uint4* __restrict__ y_perm,
                                              const int32_t* __restrict__ pair_pos,
                                              const float* __restrict__ topk_w, int t, int k,
                                              int chunks, uint4* __restrict__ y) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int lane = lane_id();
  int rows[MOE_MAX_K];
  float w[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    rows[j] = j < k ? pair_pos[(size_t)t * k + j] : -1;
    w[j] = j < k ? (topk_w != nullptr ? topk_w[(size_t)t * k + j] : 1.f) : 0.f;
  }
  // U chunks per lane: all of their k row loads are in flight before the sums
  constexpr int U = 2;
  for (int c0 = lane; c0 < chunks; c0 += U * kWave) {
    uint4 v[U][MOE_MAX_K];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j)
        if (rows[j] >= 0 && c0 + u * kWave < chunks)
          v[u][j] = y_perm[(size_t)rows[j] * chunks + c0 + u * kWave];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= chunks) break;
      float acc[EPC];
#pragma unroll
      for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j) {
        if (rows[j] < 0) continue;
        float f[EPC];
        if constexpr (BF16) {
          unpack8(v[u][j], f);
        } else {
          f[0] = __uint_as_float(v[u][j].x); f[1] = __uint_as_float(v[u][j].y);
          f[2] = __uint_as_float(v[u][j].z); f[3] = __uint_as_float(v[u][j].w);
        }
#pragma unroll
        for (int i = 0; i < EPC; ++i) acc[i] = fmaf(w[j], f[i], acc[i]);
      }
      uint4 o;
      if constexpr (BF16) {
        o = pack8(acc);
      } else {
        o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                       __float_as_uint(acc[3]));
      }
      y[(size_t)t * chunks + c] = o;
    }
  }
}

}  // namespace moe
