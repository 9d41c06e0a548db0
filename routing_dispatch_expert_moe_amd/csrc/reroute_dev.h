// Per-token top-k routing with capacity-overflow rerouting (MoE
// sparse-activation page §3.2, stage 3: a token whose best expert has reached
// its capacity takes the next expert after its k instead).  In token order, an
// expert's load is the number of earlier tokens whose final choice holds it.
//
// Step 1 (all tokens in parallel, one wave per token): the k + 1 best experts
// and their logits, as candidates.  Step 2 (one workgroup) decides which
// tokens reroute, and nothing else: the candidate experts pass through LDS in
// chunks; while one wave resolves a chunk, the other waves stage the next, so
// the sequential chain never waits on HBM.  The resolving wave takes the
// tokens in groups of 64, one per lane, and reads each lane's best-expert
// load as of the group's start from LDS.  A token whose best expert is
// already full surely reroutes, and one that stays below the capacity even if
// every earlier lane of the group took its expert surely does not; only the
// others are resolved, in lane order, with ballots against a wave-uniform
// mask of the rerouted lanes (no memory round trip).  The group's final
// choices are added to the LDS loads and its mask stored.  Step 3 (all tokens
// in parallel): final experts and gates from the candidates and the masks.
// The dependence between tokens is inherent in the rule; step 2 keeps only it
// on the chain.  The stand-alone kernels (route.hip) and the fused layer
// (fused.hip) run the same bodies.
#pragma once

#include "route_dev.h"

namespace moe {

constexpr int kMaxCand = MOE_MAX_K + 1;

// Step 1 for token t, by one whole wave: its kc best experts and logits.
template <int EPL>
__device__ __forceinline__ void reroute_candidates_token(const float* __restrict__ logits, int t,
                                                         int E, int kc,
                                                         int32_t* __restrict__ cand_e,
                                                         float* __restrict__ cand_v) {
  int sel_e[kMaxCand];
  float sel_v[kMaxCand];
  select_top<EPL, kMaxCand>(logits, t, E, kc, sel_e, sel_v);
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < kMaxCand; ++j) {
    if (j < kc && lane == j) {
      cand_e[(size_t)t * kc + j] = sel_e[j];
      cand_v[(size_t)t * kc + j] = sel_v[j];
    }
  }
}

// tokens per LDS chunk of the resolver (two chunk buffers: 2 x 30 KB at most)
template <int K>
constexpr int reroute_chunk() {
  constexpr int ch = (7680 / (K + 1)) & ~63;
  return ch < 2048 ? ch : 2048;
}

// LDS bytes of reroute_resolve_body<K>: the loads, then the two chunk buffers
template <int K>
constexpr size_t reroute_resolve_lds_bytes() {
  return static_cast<size_t>(MOE_MAX_E) * 4 + 2 * static_cast<size_t>(reroute_chunk<K>()) * (K + 1) * 4;
}

// Step 2 by a whole workgroup of NT threads (wave 0 resolves, the others
// stage); requires capacity >= 0 and K < E (k + 1 candidates per token).
// rerouted[g] bit l: token 64 g + l reroutes.  load: LDS, MOE_MAX_E ints; ce:
// LDS, 2 * reroute_chunk<K>() * (K + 1) ints.
template <int K, int NT>
__device__ __forceinline__ void reroute_resolve_body(const int32_t* __restrict__ cand_e, int T,
                                                     int E, int capacity,
                                                     uint64_t* __restrict__ rerouted, int* load,
                                                     int32_t* ce) {
  constexpr int KC = K + 1;
  constexpr int CH = reroute_chunk<K>();  // tokens per chunk
  static_assert(CH >= kWave, "chunk smaller than a wave");
  static_assert(NT > kWave, "the resolver needs loader waves");
  constexpr int kLoaders = NT - kWave;
  constexpr int U = 8;  // loads in flight per loader thread
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const bool resolver = tid < kWave;
  for (int e = tid; e < E; e += NT) load[e] = 0;
  // loader threads: chunk c's candidates (contiguous in memory) into buffer b
  auto stage = [&](int c, int b) {
    const int t0 = c * CH;
    const int n = min(CH, T - t0) * KC;
    const int32_t* src = cand_e + (size_t)t0 * KC;
    int32_t* dst = ce + b * CH * KC;
    for (int i0 = tid - kWave; i0 < n; i0 += kLoaders * U) {
      int32_t re[U];
#pragma unroll
      for (int u = 0; u < U; ++u) re[u] = src[min(i0 + u * kLoaders, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * kLoaders < n) dst[i0 + u * kLoaders] = re[u];
    }
  };
  const int nch = (T + CH - 1) / CH;
  if (!resolver) stage(0, 0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (!resolver) {
      if (c + 1 < nch) stage(c + 1, (c + 1) & 1);
    } else {
      const int t0 = c * CH;
      const int ntok = min(CH, T - t0);
      const int32_t* be = ce + (c & 1) * CH * KC;
      // candidates are read one group ahead, unconditionally: g + lane stays
      // inside the chunk buffer, and lanes past the chunk's tokens are masked
      int rn[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) rn[j] = be[lane * KC + j];
      for (int g = 0; g < ntok; g += kWave) {
        const int tl = g + lane;
        const bool valid = tl < ntok;
        int r[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) r[j] = valid ? rn[j] : -1;
        if (g + kWave < CH) {
#pragma unroll
          for (int j = 0; j < KC; ++j) rn[j] = be[(tl + kWave) * KC + j];
        }
        // the best expert's load before this group; within the group at
        // most `lane` earlier tokens can add to it
        const int base = load[valid ? r[0] : 0];
        // rerouted lanes as a wave-uniform bit mask: those whose best expert
        // is already full surely are; those that stay below the capacity
        // even if every earlier lane of the group took their expert surely
        // are not
        uint64_t rep = __ballot(valid && base >= capacity);
        uint64_t open = __ballot(valid && base < capacity && base + lane >= capacity);
        // the undecided lanes, in order: lane i's load adds the earlier lanes
        // whose final choice holds its best expert x.  Lane j's final choice
        // holds x through its middle candidates whatever it decides, through
        // its best one if it stays and through its (k+1)-th if it reroutes,
        // so the count is a few ballots against the mask decided so far.
        while (open != 0) {
          const int i = __builtin_ctzll(open);
          open &= open - 1;
          const int x = __builtin_amdgcn_readlane(r[0], i);
          bool mid = false;
#pragma unroll
          for (int j = 1; j < K; ++j) mid = mid || r[j] == x;
          const uint64_t held =
              __ballot(mid) | (__ballot(r[0] == x) & ~rep) | (__ballot(r[K] == x) & rep);
          const uint64_t before = (uint64_t{1} << i) - 1;
          if (__builtin_amdgcn_readlane(base, i) + __popcll(held & before) >= capacity)
            rep |= uint64_t{1} << i;
        }
        if (valid) {
          const bool rr = (rep >> lane) & 1;
#pragma unroll
          for (int j = 0; j < K; ++j) atomicAdd(&load[rr ? r[j + 1] : r[j]], 1);
        }
        if (lane == 0) rerouted[(t0 + g) / kWave] = rep;
      }
    }
    __syncthreads();
  }
}

// Step 3 for token t (one thread): final experts (best first) and gates;
// rerouted == nullptr: no token reroutes.
template <int K>
__device__ __forceinline__ void reroute_finalize_token(const int32_t* __restrict__ cand_e,
                                                       const float* __restrict__ cand_v,
                                                       const uint64_t* __restrict__ rerouted,
                                                       int t, int kc, int gate,
                                                       int32_t* __restrict__ topk_idx,
                                                       float* __restrict__ topk_w) {
  const bool rr = rerouted != nullptr && ((rerouted[t / kWave] >> (t % kWave)) & 1);
  const int s = rr ? 1 : 0;  // the first candidate taken
  float w[K];
  float sum = 0.f;
  const float x0 = cand_v[(size_t)t * kc + s];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float x = cand_v[(size_t)t * kc + s + j];
    w[j] = gate == 0 ? expf(x - x0) : 1.f / (1.f + expf(-x));
    sum += w[j];
    topk_idx[(size_t)t * K + j] = cand_e[(size_t)t * kc + s + j];
  }
#pragma unroll
  for (int j = 0; j < K; ++j) topk_w[(size_t)t * K + j] = w[j] / sum;
}

}  // namespace moe
