// Fused persistent MoE layer: route -> dispatch -> GEMM1 + SwiGLU -> GEMM2 ->
// combine in ONE launch.
//
// MegaMoE comparison page, core differences §1 and the closing summary: the
// whole MoE layer as one persistent kernel instead of a chain of launches,
// which removes the launches, the host round trips and the idle gaps between
// them.  MoE sparse-activation page, §4.2 layer 1: router, top-k and expert
// compute fused into one kernel.
//
// One workgroup per CU (cooperative launch: every workgroup is resident, so
// the device-wide barriers below cannot deadlock): 8 waves for bf16 (two per
// SIMD, as the stand-alone GEMM kernels run), 4 for fp32.  Phases, each
// a loop over the phase's work units with stride = grid size:
//   1. route (one wave per token); with rerouting: candidates (one wave per
//      token), the sequential resolver on workgroup 0, then the gates (one
//      thread per token), each step followed by a barrier;
//   2. dispatch count pass of each 256-token block;
//   3. every workgroup rebuilds the local segment offsets from the per-block
//      counts (workgroup 0 also writes counts / offsets / n_kept), then places
//      the pairs of its slices of token blocks;
//   4. GEMM1 + SwiGLU over the tile list (the pipelined MFMA body of the
//      stand-alone kernels, for FP8 weights with few rows per expert their
//      code-streaming body, or the fp32 body), reading each row straight from
//      x through the dispatch permutation: no permuted copy is made (DWDP
//      page, key optimisations: the row gather fused into the grouped GEMM);
//   5. GEMM2;
//   6. weighted combine (one wave per token).
// Phases are separated by a device-wide barrier (arrival counters +
// generation word in the workspace header; agent-scope release / acquire, so
// rows written through one XCD's L2 are seen by the others), except GEMM1 and
// GEMM2 when both run the pipelined body and the workspace holds the
// per-expert readiness counters: then a GEMM2 tile waits only for its own
// expert's GEMM1 rows, so workgroups that run out of GEMM1 tiles start on the
// experts already done instead of idling at a barrier.  The bodies are the
// same device functions the stand-alone kernels run, so both paths compute
// identical bits.
#include "combine_dev.h"
#include "common.h"
#include "dispatch_dev.h"
#include "gemm_f32.h"
#include "gemm_fp8w.h"
#include "gemm_pipe.h"
#include "launch.h"
#include "reroute_dev.h"
#include "route_dev.h"

namespace moe {

namespace {

// bounded wait: 2^21 polls at >= 512 clocks each (0.5 s or more, a few
// seconds at most); a barrier not completed by then raises MOE_ERR_HIP in the
// error word and lets the workgroup go on instead of hanging the GPU
constexpr uint32_t kSpinLimit = 1u << 21;

// Device-wide barrier in two levels: workgroups arrive on one of 8 group
// counters (workgroup ids are dealt round-robin over the 8 XCDs, so group x is
// normally XCD x), the last arrival of each group on the top counter, and the
// last arrival there re-arms every counter and advances the generation word
// the others poll.  Arrivals release (this workgroup's writes become visible
// device-wide), polls are relaxed loads, and one acquire fence follows the
// wait, so waiting does not keep invalidating the L2.
__device__ __forceinline__ void grid_barrier(const FusedArgs& a, uint32_t G) {
  // every wave's stores reach the L2 before the workgroup arrives (the
  // arrival's release writes the L2 back; it does not wait for other waves)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    // the generation is read before arriving: it cannot advance until every
    // workgroup, this one included, has arrived (the release below keeps the
    // read ahead of the arrival)
    const uint32_t g = __hip_atomic_load(a.bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t x = blockIdx.x & 7;
    const uint32_t group_size = (G + 7 - x) / 8;  // workgroups x, x + 8, ... below G
    const uint32_t groups = G < 8 ? G : 8;
    uint32_t* gc = a.bar_group + x * kWsBarStride;
    bool last = false;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1u ==
        group_size) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = __hip_atomic_fetch_add(a.bar_count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) +
                 1u == groups;
    }
    if (last) {
      // every group counter was re-armed before its group arrived here
      __hip_atomic_store(a.bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(a.bar_gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t spins = 0;
      while (__hip_atomic_load(a.bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
        __builtin_amdgcn_s_sleep(4);
        if (++spins == kSpinLimit) {
          raise_error(a.err, MOE_ERR_HIP);
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Inclusive-to-exclusive scan over n <= 1024 ints held in LDS `v` into `out`
// (out[0..n]), by the whole workgroup (at most 8 waves; each thread owns a
// contiguous run of 4 (256 threads) or 2 (512)).  scratch: one int per wave.
__device__ __forceinline__ void block_exclusive_scan(const int* v, int n, int* out, int* scratch) {
  const int tid = threadIdx.x;
  const int per = (MOE_MAX_E + static_cast<int>(blockDim.x) - 1) / static_cast<int>(blockDim.x);
  const int lo = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) local += v[lo + i];
  // wave-level inclusive scan, then across the waves
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if ((tid & (kWave - 1)) >= off) incl += o;
  }
  if ((tid & (kWave - 1)) == kWave - 1) scratch[tid >> 6] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < (tid >> 6); ++w) wave_base += scratch[w];
  int run = wave_base + incl - local;
  for (int i = 0; i < per; ++i) {
    if (lo + i < n) {
      out[lo + i] = run;
      run += v[lo + i];
    }
  }
  if (tid == blockDim.x - 1) out[n] = run;
  __syncthreads();
}

}  // namespace

// sum over blocks [0, nb) of expert e's per-block pair counts, eight loads in
// flight (integer sums: the value does not depend on the order)
__device__ __forceinline__ int sum_block_counts(const int* __restrict__ block_counts, int E, int e,
                                                int nb) {
  constexpr int U = 8;
  int part[U] = {};
  int b = 0;
  for (; b + U <= nb; b += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) part[u] += block_counts[(size_t)(b + u) * E + e];
  }
  for (; b < nb; ++b) part[0] += block_counts[(size_t)b * E + e];
  int c = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) c += part[u];
  return c;
}

// tile shape of one pipelined GEMM phase: BM activation rows x BNW weight
// rows, STAGES pipeline stages, the rows of class CLASS
template <int BM_, int BNW_, int STAGES_, int CLASS_>
struct TileCfg {
  static constexpr int BM = BM_, BNW = BNW_, STAGES = STAGES_, CLASS = CLASS_;
};

template <bool BF16>
constexpr int fused_threads() { return BF16 ? 512 : 256; }

// FP8 (with BF16 only): the GEMM phases read E4M3 weight codes and their
// block scales (a.w13s, a.w2s) through the FP8 pipelined body
// OVERLAP: the GEMM phases meet through the per-expert readiness counters
// instead of a barrier (a separate instantiation, so the barrier form's GEMM
// loops carry none of the waiting code)
template <bool BF16, bool FP8 = false, bool OVERLAP = false>
__global__ __launch_bounds__(fused_threads<BF16>(), 1) void moe_fused_kernel(FusedArgs a) {
  static_assert(BF16 || !FP8, "FP8 weights take bf16 activations");
  static_assert(BF16 || !OVERLAP, "the fp32 GEMM body does not count its tiles");
  constexpr int NT = fused_threads<BF16>();
  constexpr int NWV = NT / kWave;  // waves per workgroup
  extern __shared__ uint4 lds[];
  __shared__ int prefix[MOE_MAX_E + 1];
  __shared__ int segs[MOE_MAX_E + 1];
  __shared__ int scan_scratch[NWV];
  const int bid = blockIdx.x, G = gridDim.x;
  const int T = a.T, E = a.E, k = a.k;
  const int E_loc = a.e_end - a.e_begin;
  const int nb = (T + kTB - 1) / kTB;
  unsigned long long* bits = reinterpret_cast<unsigned long long*>(lds);
  int* cnt_s = reinterpret_cast<int*>(bits + static_cast<size_t>(E) * kWords);  // [E]
  int* base_s = cnt_s + E;                                                     // [E]

  const int wave = threadIdx.x >> 6;
  const int chunks = static_cast<int>((static_cast<size_t>(a.d) * (BF16 ? 2 : 4)) / 16);

  // ---- 1: route, one wave per token
  if (a.reroute) {
    const int kc = k < E ? k + 1 : k;
    for (int t = bid * NWV + wave; t < T; t += G * NWV) {
      if (E <= 64) reroute_candidates_token<1>(a.logits, t, E, kc, a.cand_e, a.cand_v);
      else if (E <= 256) reroute_candidates_token<4>(a.logits, t, E, kc, a.cand_e, a.cand_v);
      else reroute_candidates_token<16>(a.logits, t, E, kc, a.cand_e, a.cand_v);
    }
    grid_barrier(a, G);
    const bool can = a.capacity >= 0 && k < E;
    if (can && bid == 0) {
      int* load = reinterpret_cast<int*>(lds);
      int32_t* ce = load + MOE_MAX_E;
      switch (k) {
#define MOE_FUSED_RESOLVE(KK)                                                                   \
  case KK:                                                                                     \
    reroute_resolve_body<KK, NT>(a.cand_e, T, E, a.capacity, a.rerouted, load, ce);            \
    break;
        MOE_FUSED_RESOLVE(1) MOE_FUSED_RESOLVE(2) MOE_FUSED_RESOLVE(3) MOE_FUSED_RESOLVE(4)
        MOE_FUSED_RESOLVE(5) MOE_FUSED_RESOLVE(6) MOE_FUSED_RESOLVE(7) MOE_FUSED_RESOLVE(8)
#undef MOE_FUSED_RESOLVE
        default: break;
      }
    }
    grid_barrier(a, G);
    for (int t = bid * NT + static_cast<int>(threadIdx.x); t < T; t += G * NT) {
      const uint64_t* rr = can ? a.rerouted : nullptr;
      switch (k) {
#define MOE_FUSED_GATES(KK)                                                                     \
  case KK:                                                                                     \
    reroute_finalize_token<KK>(a.cand_e, a.cand_v, rr, t, kc, a.gate, a.topk_idx, a.topk_w);   \
    break;
        MOE_FUSED_GATES(1) MOE_FUSED_GATES(2) MOE_FUSED_GATES(3) MOE_FUSED_GATES(4)
        MOE_FUSED_GATES(5) MOE_FUSED_GATES(6) MOE_FUSED_GATES(7) MOE_FUSED_GATES(8)
#undef MOE_FUSED_GATES
        default: break;
      }
    }
  } else {
    // a wave routes several tokens in turn: the next token's logits are loaded
    // while the current one is ranked
    auto route_all = [&](auto epl) {
      constexpr int EPL = decltype(epl)::value;
      int t = bid * NWV + wave;
      float cur[EPL];
      if (t < T) load_logits<EPL>(a.logits, t, E, cur);
      for (; t < T; t += G * NWV) {
        float nxt[EPL] = {};
        if (t + G * NWV < T) load_logits<EPL>(a.logits, t + G * NWV, E, nxt);
        route_token_vals<EPL>(cur, t, E, k, a.gate, a.topk_idx, a.topk_w);
#pragma unroll
        for (int i = 0; i < EPL; ++i) cur[i] = nxt[i];
      }
    };
    if (E <= 64) route_all(std::integral_constant<int, 1>{});
    else if (E <= 128) route_all(std::integral_constant<int, 2>{});
    else if (E <= 256) route_all(std::integral_constant<int, 4>{});
    else route_all(std::integral_constant<int, 16>{});
  }
  grid_barrier(a, G);

  // ---- 2: dispatch count pass, per 256-token block
  for (int vb = bid; vb < nb; vb += G)
    dispatch_count_block(vb, bits, a.topk_idx, T, E, k, a.block_counts, a.err);
  grid_barrier(a, G);

  // ---- 3: plan, then place.  Work unit = (token block, slice): every
  // workgroup rebuilds the block's bitmaps and places only its slice of the
  // block's pairs, so the work spreads over the grid.
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int c = sum_block_counts(a.block_counts, E, e, nb);
    cnt_s[e] = c;
    if (bid == 0) a.counts[e] = c;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E_loc; i += blockDim.x) {
    const int c = cnt_s[a.e_begin + i];
    base_s[i] = a.capacity < 0 ? c : min(c, a.capacity);  // kept rows per local expert
  }
  __syncthreads();
  block_exclusive_scan(base_s, E_loc, segs, scan_scratch);
  if (bid == 0) {
    for (int i = threadIdx.x; i <= E_loc; i += blockDim.x) a.offsets[i] = segs[i];
    if (threadIdx.x == 0) *a.n_kept = segs[E_loc];
    // the GEMM1 readiness counts start at zero (the barrier below publishes it
    // before any tile adds to them)
    if (OVERLAP)
      for (int i = threadIdx.x; i < E_loc; i += blockDim.x)
        __hip_atomic_store(a.up_ready + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int slices = nb > 0 ? max(1, min(kTB / 4, G / nb)) : 1;
  const int per_slice = (kTB + slices - 1) / slices;
  for (int u = bid; u < nb * slices; u += G) {
    const int vb = u / slices, sl = u - vb * slices;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      base_s[e] = sum_block_counts(a.block_counts, E, e, vb);
    __syncthreads();
    const int t0 = vb * kTB + sl * per_slice;
    dispatch_place_block(vb, bits, a.topk_idx, T, E, k, a.capacity, a.e_begin, a.e_end, base_s,
                         segs, a.sorted_pair, a.pair_pos, t0, t0 + per_slice);
  }
  grid_barrier(a, G);

  // ---- 3 / 4: the two grouped GEMMs.  With OVERLAP (every GEMM phase on
  // the pipelined body) no barrier separates them: GEMM1 tiles count their
  // stored rows per expert in a.up_ready and a GEMM2 tile of expert e starts
  // once e's count is complete (MegaMoE comparison page, core differences §1:
  // the stages of different experts overlap instead of waiting for each
  // other).  A workgroup runs all its GEMM1 tiles before any GEMM2 tile and
  // every workgroup is resident, so every wait ends.
  // (the launcher never picks OVERLAP with the FP8 code-streaming body,
  // which does not count its tiles)
  uint32_t* up = OVERLAP ? a.up_ready : nullptr;
  // (a.w13_list / a.w2_list: the weights or FP8 codes as per-expert tables;
  // a.w13s_list / a.w2s_list: the FP8 block scales as per-expert tables)
  auto pipe_up = [&](auto cfg, const uint16_t* w, const float* ws) {
    using C = decltype(cfg);
    gemm_pipe_body<true, C::BM, C::BNW, C::STAGES, C::CLASS, 8, false, FP8, 64>(
        static_cast<const uint16_t*>(a.x), a.offsets, E_loc, w, static_cast<uint16_t*>(a.h), a.f,
        a.d, bid, G, lds, prefix, segs, a.sorted_pair, k,
        reinterpret_cast<const uint16_t* const*>(a.w13_list), nullptr, ws, up, nullptr, a.err,
        a.w13s_list);
  };
  auto pipe_down = [&](auto cfg, const uint16_t* w, const float* ws) {
    using C = decltype(cfg);
    gemm_pipe_body<false, C::BM, C::BNW, C::STAGES, C::CLASS, 8, false, FP8, 64>(
        static_cast<const uint16_t*>(a.h), a.offsets, E_loc, w, static_cast<uint16_t*>(a.y_perm),
        a.d, a.f, bid, G, lds, prefix, segs, nullptr, 1,
        reinterpret_cast<const uint16_t* const*>(a.w2_list), nullptr, ws, nullptr, up, a.err,
        a.w2s_list);
  };
  if constexpr (FP8) {
    // the FP8 weights' row splits, as in the separate FP8 calls: few rows per
    // expert stream the codes through 32-row tiles (two 256-thread parts per
    // workgroup, each on a tile of its own), a wide first half takes 128-row
    // tiles, long-K passes with few tiles 256-row tiles plus 128-row
    // remainder tiles, passes with many tiles the ride-along split, the
    // others every row in 256-row tiles
    const uint16_t* w13 = static_cast<const uint16_t*>(a.w13);  // codes, read as bytes
    const uint16_t* w2 = static_cast<const uint16_t*>(a.w2);
    constexpr int kParts = NT / 256;
    if (a.ffn_all_rows) {
      gemm_fp8w_body<128, true, kParts>(static_cast<const uint16_t*>(a.x), a.offsets, E_loc,
                                        static_cast<const uint8_t*>(a.w13), a.w13s,
                                        static_cast<uint16_t*>(a.h), a.f, a.d, bid, G, lds, prefix,
                                        a.sorted_pair, k,
                                        reinterpret_cast<const uint8_t* const*>(a.w13_list),
                                        a.w13s_list);
    } else if (a.rows_up == kFusedWide) {
      pipe_up(TileCfg<128, 256, 4, ROWS_ALL>{}, w13, a.w13s);
    } else if (a.rows_up == kFusedBigTail) {
      pipe_up(TileCfg<256, 256, 3, ROWS_BIG>{}, w13, a.w13s);
      pipe_up(TileCfg<128, 256, 4, ROWS_TAIL>{}, w13, a.w13s);
    } else if (a.rows_up == kFusedRide) {
      pipe_up(TileCfg<256, 256, 3, ROWS_BIGR>{}, w13, a.w13s);
      pipe_up(TileCfg<128, 256, 4, ROWS_TAILR>{}, w13, a.w13s);
    } else {
      pipe_up(TileCfg<256, 256, 3, ROWS_ALL>{}, w13, a.w13s);
    }
    // (the code-streaming bodies do not count their tiles: always a barrier)
    if (!OVERLAP || a.ffn_all_rows) grid_barrier(a, G);
    if (a.ffn_all_rows) {
      gemm_fp8w_body<128, false, kParts>(static_cast<const uint16_t*>(a.h), a.offsets, E_loc,
                                         static_cast<const uint8_t*>(a.w2), a.w2s,
                                         static_cast<uint16_t*>(a.y_perm), a.d, a.f, bid, G, lds,
                                         prefix, nullptr, 1,
                                         reinterpret_cast<const uint8_t* const*>(a.w2_list),
                                         a.w2s_list);
    } else if (a.rows_down == kFusedBigTail) {
      pipe_down(TileCfg<256, 256, 3, ROWS_BIG>{}, w2, a.w2s);
      pipe_down(TileCfg<128, 256, 4, ROWS_TAIL>{}, w2, a.w2s);
    } else if (a.rows_down == kFusedRide) {
      pipe_down(TileCfg<256, 256, 3, ROWS_BIGR>{}, w2, a.w2s);
      pipe_down(TileCfg<128, 256, 4, ROWS_TAILR>{}, w2, a.w2s);
    } else {
      pipe_down(TileCfg<256, 256, 3, ROWS_ALL>{}, w2, a.w2s);
    }
  } else if constexpr (BF16) {
    const uint16_t* w13 = static_cast<const uint16_t*>(a.w13);
    const uint16_t* w2 = static_cast<const uint16_t*>(a.w2);
    if (a.ffn_all_rows || a.rows_up == kFusedWide) {
      pipe_up(TileCfg<128, 256, 3, ROWS_ALL>{}, w13, nullptr);
    } else if (a.rows_up == kFusedAllBig) {
      pipe_up(TileCfg<256, 256, 2, ROWS_ALL>{}, w13, nullptr);
    } else if (a.rows_up == kFusedRide) {
      pipe_up(TileCfg<256, 256, 2, ROWS_BIGR>{}, w13, nullptr);
      pipe_up(TileCfg<128, 256, 3, ROWS_TAILR>{}, w13, nullptr);
    } else {
      pipe_up(TileCfg<256, 256, 2, ROWS_BIG>{}, w13, nullptr);
      pipe_up(TileCfg<128, 256, 3, ROWS_TAIL>{}, w13, nullptr);
    }
    if (!OVERLAP) grid_barrier(a, G);
    if (a.ffn_all_rows) {
      pipe_down(TileCfg<128, 256, 3, ROWS_ALL>{}, w2, nullptr);
    } else if (a.rows_down == kFusedAllBig) {
      pipe_down(TileCfg<256, 256, 2, ROWS_ALL>{}, w2, nullptr);
    } else if (a.rows_down == kFusedRide) {
      pipe_down(TileCfg<256, 256, 2, ROWS_BIGR>{}, w2, nullptr);
      pipe_down(TileCfg<128, 256, 3, ROWS_TAILR>{}, w2, nullptr);
    } else {
      // few tiles (the split's condition): the remainders in 128 x 128 tiles,
      // twice as many as with 256 weight rows, as the separate call runs them
      pipe_down(TileCfg<256, 256, 2, ROWS_BIG>{}, w2, nullptr);
      pipe_down(TileCfg<128, 128, 4, ROWS_TAIL>{}, w2, nullptr);
    }
  } else {
    float* smem = reinterpret_cast<float*>(lds);
    gemm_f32_body<true>(static_cast<const float*>(a.x), a.offsets, E_loc,
                        static_cast<const float*>(a.w13), static_cast<float*>(a.h), a.f, a.d,
                        bid, G, smem, prefix, a.sorted_pair, k,
                        reinterpret_cast<const float* const*>(a.w13_list));
    grid_barrier(a, G);
    gemm_f32_body<false>(static_cast<const float*>(a.h), a.offsets, E_loc,
                         static_cast<const float*>(a.w2), static_cast<float*>(a.y_perm), a.d, a.f,
                         bid, G, smem, prefix, nullptr, 1,
                         reinterpret_cast<const float* const*>(a.w2_list));
  }
  grid_barrier(a, G);

  // ---- 5: combine.  With one workgroup per CU a wave holds few rows in
  // flight unless the token's row slots match k (for k <= 2, 8 chunks per
  // lane: 16 row loads, in the registers that k = 8 needs for 2), and each
  // token's row loads wait for its pair indices unless those are fetched a
  // token ahead
  const uint4* yp = static_cast<const uint4*>(a.y_perm);
  uint4* yo = static_cast<uint4*>(a.y);
  const int t0 = bid * NWV + wave, ts = G * NWV;
  const int32_t* pp = a.pair_pos;
  const float* tw = a.topk_w;
  switch (k) {
    case 1: combine_tokens<BF16, 1, 8>(yp, pp, tw, t0, ts, T, chunks, yo); break;
    case 2: combine_tokens<BF16, 2, 8>(yp, pp, tw, t0, ts, T, chunks, yo); break;
    case 4: combine_tokens<BF16, 4, 4>(yp, pp, tw, t0, ts, T, chunks, yo); break;
    case 8: combine_tokens<BF16, 8, 2>(yp, pp, tw, t0, ts, T, chunks, yo); break;
    default:
      for (int t = t0; t < T; t += ts) combine_token<BF16>(yp, pp, tw, t, k, chunks, yo);
  }
}

// the rerouting resolver's LDS for any k
constexpr size_t resolver_lds_bytes() {
  size_t m = reroute_resolve_lds_bytes<1>();
  const size_t b[] = {reroute_resolve_lds_bytes<2>(), reroute_resolve_lds_bytes<3>(),
                      reroute_resolve_lds_bytes<4>(), reroute_resolve_lds_bytes<5>(),
                      reroute_resolve_lds_bytes<6>(), reroute_resolve_lds_bytes<7>(),
                      reroute_resolve_lds_bytes<8>()};
  for (size_t v : b) m = v > m ? v : m;
  return m;
}

size_t fused_lds_bytes(int E, bool bf16, bool fp8) {
  size_t plan = static_cast<size_t>(E) * kWords * sizeof(unsigned long long) +
                2 * static_cast<size_t>(E) * sizeof(int);
  if (plan < resolver_lds_bytes()) plan = resolver_lds_bytes();
  size_t gemm = f32_lds_floats(true) * sizeof(float);
  if (bf16 && fp8) {
    gemm = pipe_lds_bytes(256, 256, 3, true, 64);
    if (gemm < pipe_lds_bytes(128, 256, 4, true, 64)) gemm = pipe_lds_bytes(128, 256, 4, true, 64);
    constexpr size_t stream = fp8w_lds_bytes<128, true>(fused_threads<true>() / 256);
    if (gemm < stream) gemm = stream;
  } else if (bf16) {
    // GEMM phases step K 64 deep (K = d or f, multiples of 64 for bf16)
    gemm = pipe_lds_bytes(256, 256, 2, false, 64);
    if (gemm < pipe_lds_bytes(128, 256, 3, false, 64)) gemm = pipe_lds_bytes(128, 256, 3, false, 64);
    if (gemm < pipe_lds_bytes(128, 128, 4, false, 64)) gemm = pipe_lds_bytes(128, 128, 4, false, 64);
  }
  return plan > gemm ? plan : gemm;
}

int launch_fused(const FusedArgs& a, bool bf16, int64_t max_rows, void* stream, bool fp8) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  fp8 = fp8 && bf16;
  const size_t lds = fused_lds_bytes(a.E, bf16, fp8);
  const bool ov = bf16 && a.overlap != 0;
  const void* kern =
      fp8    ? (ov ? reinterpret_cast<const void*>(moe_fused_kernel<true, true, true>)
                   : reinterpret_cast<const void*>(moe_fused_kernel<true, true>))
      : bf16 ? (ov ? reinterpret_cast<const void*>(moe_fused_kernel<true, false, true>)
                   : reinterpret_cast<const void*>(moe_fused_kernel<true>))
             : reinterpret_cast<const void*>(moe_fused_kernel<false>);
  // the largest dynamic LDS any E can ask for
  static LdsAttr attr[5];
  if (int rc = set_dynamic_lds_once(kern, fused_lds_bytes(MOE_MAX_E, bf16, fp8),
                                    attr[(fp8 ? 2 : bf16 ? 1 : 0) + (ov ? 2 : 0)]))
    return rc;
  int occ = 0;
  const int threads = bf16 ? fused_threads<true>() : fused_threads<false>();
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, lds);
  if (e != hipSuccess) return static_cast<int>(e);
  if (occ < 1) return static_cast<int>(hipErrorCooperativeLaunchTooLarge);
  // enough workgroups for the widest phase, never more than can be resident
  const int E_loc = a.e_end - a.e_begin;
  const int64_t nb = (a.T + kTB - 1) / kTB;
  const int64_t tok_groups = (a.T + 3) / 4;
  const int64_t mtiles = bf16 ? max_rows / 128 + E_loc : max_rows / 64 + E_loc;
  const int64_t up_tiles = mtiles * (bf16 ? (a.f + 63) / 64 : (a.f + 63) / 64);
  const int64_t down_tiles = mtiles * (bf16 ? (a.d + 127) / 128 : (a.d + 63) / 64);
  const int64_t gemm_tiles = up_tiles > down_tiles ? up_tiles : down_tiles;
  int64_t want = nb;
  if (tok_groups > want) want = tok_groups;
  if (gemm_tiles > want) want = gemm_tiles;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * occ;
  if (grid > want) grid = want;
  if (grid >= 8) grid &= ~static_cast<int64_t>(7);
  if (grid < 1) grid = 1;
  void* args[] = {const_cast<FusedArgs*>(&a)};
  e = hipLaunchCooperativeKernel(kern, dim3(static_cast<unsigned>(grid)), dim3(threads), args,
                                 static_cast<unsigned>(lds), s);
  if (e != hipSuccess) return static_cast<int>(e);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
