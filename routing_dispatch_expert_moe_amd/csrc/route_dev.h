// Per-token top-k routing (MoE sparse-activation page, §3.2 stage 2): the k
// largest fp32 logits, ties to the lower expert index, best first; gates
// softmax-renormalised over the k, or sigmoid normalised over the k.
#pragma once

#include "common.h"

namespace moe {

// ---------------------------------------------------------------------------
// A1: one wave per token.  Each lane holds EPL logits (expert e = lane + 64*i)
// as 64-bit keys: high word = order-preserving image of the fp32 value (with
// -0.0 mapped to +0.0), low word = ~e, so the largest key is the largest
// logit and, among equal logits, the lowest expert index.  k rounds of a
// wave-wide max pick the experts best first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 and +0.0 share one key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

// This lane's logits of token t: v[i] is expert lane + 64 i (0 past E).
template <int EPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ logits, int t, int E,
                                            float (&v)[EPL]) {
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : 0.f;
  }
}

// The kc best experts (best first) and their logits among the wave's values v
// (as load_logits leaves them), by one whole wave (E <= 64 * EPL, kc <= KMAX);
// entries past kc are 0.
template <int EPL, int KMAX>
__device__ __forceinline__ void select_top_vals(const float (&v)[EPL], int E, int kc,
                                                int (&sel_e)[KMAX], float (&sel_v)[KMAX]) {
  const int lane = lane_id();
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0;
    if (e < E) key[i] = (static_cast<uint64_t>(ordered_bits(v[i])) << 32) | static_cast<uint32_t>(~e);
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < kc) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (key[i] == best) key[i] = 0;
      sel_e[j] = static_cast<int>(~static_cast<uint32_t>(best));
      sel_v[j] = from_ordered(static_cast<uint32_t>(best >> 32));
    } else {
      sel_e[j] = 0;
      sel_v[j] = 0.f;
    }
  }
}

// The kc best experts of token t (best first) and their logits, by one whole
// wave (E <= 64 * EPL, kc <= KMAX); entries past kc are 0.
template <int EPL, int KMAX>
__device__ __forceinline__ void select_top(const float* __restrict__ logits, int t, int E, int kc,
                                           int (&sel_e)[KMAX], float (&sel_v)[KMAX]) {
  float v[EPL];
  load_logits<EPL>(logits, t, E, v);
  select_top_vals<EPL, KMAX>(v, E, kc, sel_e, sel_v);
}

// Top-k and gates of token t from the wave's values v of its logits (as
// load_logits leaves them), computed by one whole wave (E <= 64 * EPL).
template <int EPL>
__device__ __forceinline__ void route_token_vals(const float (&v)[EPL], int t, int E, int k,
                                                 int gate, int32_t* __restrict__ topk_idx,
                                                 float* __restrict__ topk_w) {
  const int lane = lane_id();
  int sel_e[MOE_MAX_K];
  float sel_v[MOE_MAX_K];
  select_top_vals<EPL, MOE_MAX_K>(v, E, k, sel_e, sel_v);
  float g[MOE_MAX_K];
  float sum = 0.f;
  if (gate == 0) {
    const float m = sel_v[0];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      g[j] = j < k ? expf(sel_v[j] - m) : 0.f;
      sum += g[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      g[j] = j < k ? 1.f / (1.f + expf(-sel_v[j])) : 0.f;
      sum += g[j];
    }
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    if (j < k && lane == j) {
      topk_idx[(size_t)t * k + j] = sel_e[j];
      topk_w[(size_t)t * k + j] = g[j] / sum;
    }
  }
}

// Top-k and gates of token t, computed by one whole wave (E <= 64 * EPL).
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int gate, int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w) {
  float v[EPL];
  load_logits<EPL>(logits, t, E, v);
  route_token_vals<EPL>(v, t, E, k, gate, topk_idx, topk_w);
}

}  // namespace moe
