// Weighted combine (NCCL EP page §2.1, LL combine): for each token, the sum
// over its k choices of gate weight times that pair's expert output row.
// One wave per token; 16-byte loads of every contributing row; fp32
// accumulation in ascending j; one rounding at the store.  No atomics: each
// output row is owned by exactly one wave, so the result is deterministic.
#pragma once

#include "common.h"

namespace moe {

// Pair rows and gate weights of token t (KS slots; slots j >= k get row -1).
// topk_w == nullptr: every weight is 1 (the plain sum of the token's rows, as
// the backward pass needs for the input gradient).
template <int KS>
__device__ __forceinline__ void combine_pairs(const int32_t* __restrict__ pair_pos,
                                              const float* __restrict__ topk_w, int t, int k,
                                              int (&rows)[KS], float (&w)[KS]) {
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    rows[j] = j < k ? pair_pos[(size_t)t * k + j] : -1;
    w[j] = j < k ? (topk_w != nullptr ? topk_w[(size_t)t * k + j] : 1.f) : 0.f;
  }
}

// Output rows of NT tokens t[0..NT) from their pair rows and weights,
// computed by one whole wave; a token t[n] >= T (no token) has rows of -1 and
// stores nothing.  U: chunks per lane whose NT x KS row loads are all in
// flight before the sums.  Every output is the same fmaf chain over
// j = 0 .. k - 1 for any NT, KS and U.
template <bool BF16, int NT, int KS, int U>
__device__ __forceinline__ void combine_rows(const uint4* __restrict__ y_perm,
                                             const int (&rows)[NT][KS],
                                             const float (&w)[NT][KS], const int (&t)[NT], int T,
                                             int chunks, uint4* __restrict__ y) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int lane = lane_id();
  for (int c0 = lane; c0 < chunks; c0 += U * kWave) {
    uint4 v[NT][U][KS];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < KS; ++j)
          if (rows[n][j] >= 0 && c0 + u * kWave < chunks)
            v[n][u][j] = y_perm[(size_t)rows[n][j] * chunks + c0 + u * kWave];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (t[n] >= T) continue;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave;
        if (c >= chunks) break;
        float acc[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          if (rows[n][j] < 0) continue;
          float f[EPC];
          if constexpr (BF16) {
            unpack8(v[n][u][j], f);
          } else {
            f[0] = __uint_as_float(v[n][u][j].x); f[1] = __uint_as_float(v[n][u][j].y);
            f[2] = __uint_as_float(v[n][u][j].z); f[3] = __uint_as_float(v[n][u][j].w);
          }
#pragma unroll
          for (int i = 0; i < EPC; ++i) acc[i] = fmaf(w[n][j], f[i], acc[i]);
        }
        uint4 o;
        if constexpr (BF16) {
          o = pack8(acc);
        } else {
          o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                         __float_as_uint(acc[2]), __float_as_uint(acc[3]));
        }
        y[(size_t)t[n] * chunks + c] = o;
      }
    }
  }
}

// Output row of token t, computed by one whole wave (any k <= MOE_MAX_K).
template <bool BF16>
__device__ __forceinline__ void combine_token(const uint4* __restrict__ y_perm,
                                              const int32_t* __restrict__ pair_pos,
                                              const float* __restrict__ topk_w, int t, int k,
                                              int chunks, uint4* __restrict__ y) {
  int rows[1][MOE_MAX_K];
  float w[1][MOE_MAX_K];
  const int tt[1] = {t};
  combine_pairs(pair_pos, topk_w, t, k, rows[0], w[0]);
  combine_rows<BF16, 1, MOE_MAX_K, 2>(y_perm, rows, w, tt, t + 1, chunks, y);
}

// One wave's tokens t0, t0 + stride, ... below T, with k = KS pairs each, two
// at a time: both tokens' row loads are in flight before either's sums and
// stores (with one workgroup per CU a wave's chain of tokens is
// latency-bound, and its stores hold up the next loads' waits).
template <bool BF16, int KS, int U>
__device__ __forceinline__ void combine_tokens(const uint4* __restrict__ y_perm,
                                               const int32_t* __restrict__ pair_pos,
                                               const float* __restrict__ topk_w, int t0,
                                               int stride, int T, int chunks,
                                               uint4* __restrict__ y) {
  for (int t = t0; t < T; t += 2 * stride) {
    int rows[2][KS];
    float w[2][KS];
    const int tt[2] = {t, t + stride};
    combine_pairs(pair_pos, topk_w, t, KS, rows[0], w[0]);
    if (tt[1] < T) {
      combine_pairs(pair_pos, topk_w, tt[1], KS, rows[1], w[1]);
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        rows[1][j] = -1;
        w[1][j] = 0.f;
      }
    }
    combine_rows<BF16, 2, KS, U>(y_perm, rows, w, tt, T, chunks, y);
  }
}

}  // namespace moe
