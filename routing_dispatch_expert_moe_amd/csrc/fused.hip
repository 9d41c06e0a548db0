// Fused persistent MoE layer: route -> dispatch -> GEMM1 + SwiGLU -> GEMM2 ->
// combine in ONE launch.
//
// MegaMoE comparison page, core differences §1 and the closing summary: the
// whole MoE layer as one persistent kernel instead of a chain of launches,
// which removes the launches, the host round trips and the idle gaps between
// them.  MoE sparse-activation page, §4.2 layer 1: router, top-k and expert
// compute fused into one kernel.
//
// One workgroup of 256 threads per CU (cooperative launch: every workgroup is
// resident, so the device-wide barriers below cannot deadlock).  Phases, each
// a loop over the phase's work units with stride = grid size:
//   1. route (one wave per token); with rerouting: candidates (one wave per
//      token), the sequential resolver on workgroup 0, then the gates (one
//      thread per token), each step followed by a barrier;
//   2. dispatch count pass of each 256-token block;
//   3. every workgroup rebuilds the local segment offsets from the per-block
//      counts (workgroup 0 also writes counts / offsets / n_kept), then places
//      the pairs of its slices of token blocks;
//   4. GEMM1 + SwiGLU over the tile list (the pipelined MFMA body of the
//      stand-alone kernels, or the fp32 body), reading each row straight from
//      x through the dispatch permutation: no permuted copy is made (DWDP
//      page, key optimisations: the row gather fused into the grouped GEMM);
//   5. GEMM2;
//   6. weighted combine (one wave per token).
// Phases are separated by a device-wide barrier (arrival counters +
// generation word in the workspace header; agent-scope release / acquire, so
// rows written through one XCD's L2 are seen by the others).  The bodies are the
// same device functions the stand-alone kernels run, so both paths compute
// identical bits.
#include "combine_dev.h"
#include "common.h"
#include "dispatch_dev.h"
#include "gemm_f32.h"
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
// (out[0..n]), by the whole workgroup (256 threads, each owns a run of 4).
__device__ __forceinline__ void block_exclusive_scan(const int* v, int n, int* out, int* scratch) {
  const int tid = threadIdx.x;
  const int lo = tid * 4;
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lo + i < n) local += v[lo + i];
  // wave-level inclusive scan, then across the 4 waves
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
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

template <bool BF16>
__global__ __launch_bounds__(256, 1) void moe_fused_kernel(FusedArgs a) {
  extern __shared__ uint4 lds[];
  __shared__ int prefix[MOE_MAX_E + 1];
  __shared__ int segs[MOE_MAX_E + 1];
  __shared__ int scan_scratch[4];
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
    for (int t = bid * 4 + wave; t < T; t += G * 4) {
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
    reroute_resolve_body<KK, 256>(a.cand_e, T, E, a.capacity, a.rerouted, load, ce);           \
    break;
        MOE_FUSED_RESOLVE(1) MOE_FUSED_RESOLVE(2) MOE_FUSED_RESOLVE(3) MOE_FUSED_RESOLVE(4)
        MOE_FUSED_RESOLVE(5) MOE_FUSED_RESOLVE(6) MOE_FUSED_RESOLVE(7) MOE_FUSED_RESOLVE(8)
#undef MOE_FUSED_RESOLVE
        default: break;
      }
    }
    grid_barrier(a, G);
    for (int t = bid * 256 + static_cast<int>(threadIdx.x); t < T; t += G * 256) {
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
      int t = bid * 4 + wave;
      float cur[EPL];
      if (t < T) load_logits<EPL>(a.logits, t, E, cur);
      for (; t < T; t += G * 4) {
        float nxt[EPL] = {};
        if (t + G * 4 < T) load_logits<EPL>(a.logits, t + G * 4, E, nxt);
        route_token_vals<EPL>(cur, t, E, k, a.gate, a.topk_idx, a.topk_w);
#pragma unroll
        for (int i = 0; i < EPL; ++i) cur[i] = nxt[i];
      }
    };
    if (E <= 64) route_all(std::integral_constant<int, 1>{});
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

  // ---- 3 / 4: the two grouped GEMMs
  if constexpr (BF16) {
    const uint16_t* xp = static_cast<const uint16_t*>(a.x);
    const uint16_t* w13 = static_cast<const uint16_t*>(a.w13);
    uint16_t* h = static_cast<uint16_t*>(a.h);
    if (a.ffn_all_rows) {
      gemm_pipe_body<true, 128, 128, 8, ROWS_ALL>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G, lds,
                                             prefix, segs, a.sorted_pair, k);
    } else if (a.rows_up == kFusedWide) {
      gemm_pipe_body<true, 128, 256, 6, ROWS_ALL>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G, lds,
                                             prefix, segs, a.sorted_pair, k);
    } else if (a.rows_up == kFusedAllBig) {
      gemm_pipe_body<true, 256, 256, 4, ROWS_ALL>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G, lds,
                                             prefix, segs, a.sorted_pair, k);
    } else if (a.rows_up == kFusedRide) {
      gemm_pipe_body<true, 256, 256, 4, ROWS_BIGR>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G,
                                              lds, prefix, segs, a.sorted_pair, k);
      gemm_pipe_body<true, 128, 128, 8, ROWS_TAILR>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G,
                                               lds, prefix, segs, a.sorted_pair, k);
    } else {
      gemm_pipe_body<true, 256, 256, 4, ROWS_BIG>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G, lds,
                                             prefix, segs, a.sorted_pair, k);
      gemm_pipe_body<true, 128, 128, 8, ROWS_TAIL>(xp, a.offsets, E_loc, w13, h, a.f, a.d, bid, G,
                                              lds, prefix, segs, a.sorted_pair, k);
    }
    grid_barrier(a, G);
    const uint16_t* w2 = static_cast<const uint16_t*>(a.w2);
    uint16_t* yp = static_cast<uint16_t*>(a.y_perm);
    if (a.ffn_all_rows) {
      gemm_pipe_body<false, 128, 128, 8, ROWS_ALL>(h, a.offsets, E_loc, w2, yp, a.d, a.f, bid, G, lds,
                                              prefix, segs);
    } else if (a.rows_down == kFusedAllBig) {
      gemm_pipe_body<false, 256, 256, 4, ROWS_ALL>(h, a.offsets, E_loc, w2, yp, a.d, a.f, bid, G, lds,
                                              prefix, segs);
    } else if (a.rows_down == kFusedRide) {
      gemm_pipe_body<false, 256, 256, 4, ROWS_BIGR>(h, a.offsets, E_loc, w2, yp, a.d, a.f, bid, G,
                                               lds, prefix, segs);
      gemm_pipe_body<false, 128, 128, 8, ROWS_TAILR>(h, a.offsets, E_loc, w2, yp, a.d, a.f, bid, G,
                                                lds, prefix, segs);
    } else {
      gemm_pipe_body<false, 256, 256, 4, ROWS_BIG>(h, a.offsets, E_loc, w2, yp, a.d, a.f, bid, G, lds,
                                              prefix, segs);
      gemm_pipe_body<false, 128, 128, 8, ROWS_TAIL>(h, a.offsets, E_loc, w2, yp, a.d, a.f, bid, G,
                                               lds, prefix, segs);
    }
  } else {
    float* smem = reinterpret_cast<float*>(lds);
    gemm_f32_body<true>(static_cast<const float*>(a.x), a.offsets, E_loc,
                        static_cast<const float*>(a.w13), static_cast<float*>(a.h), a.f, a.d,
                        bid, G, smem, prefix, a.sorted_pair, k);
    grid_barrier(a, G);
    gemm_f32_body<false>(static_cast<const float*>(a.h), a.offsets, E_loc,
                         static_cast<const float*>(a.w2), static_cast<float*>(a.y_perm), a.d, a.f,
                         bid, G, smem, prefix);
  }
  grid_barrier(a, G);

  // ---- 5: combine
  for (int t = bid * 4 + wave; t < T; t += G * 4)
    combine_token<BF16>(static_cast<const uint4*>(a.y_perm), a.pair_pos, a.topk_w, t, k, chunks,
                        static_cast<uint4*>(a.y));
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

size_t fused_lds_bytes(int E, bool bf16) {
  size_t plan = static_cast<size_t>(E) * kWords * sizeof(unsigned long long) +
                2 * static_cast<size_t>(E) * sizeof(int);
  if (plan < resolver_lds_bytes()) plan = resolver_lds_bytes();
  size_t gemm = f32_lds_floats(true) * sizeof(float);
  if (bf16) {
    gemm = pipe_lds_bytes(128, 128, 8);
    if (gemm < pipe_lds_bytes(256, 256, 4)) gemm = pipe_lds_bytes(256, 256, 4);
    if (gemm < pipe_lds_bytes(128, 256, 6)) gemm = pipe_lds_bytes(128, 256, 6);
  }
  return plan > gemm ? plan : gemm;
}

int launch_fused(const FusedArgs& a, bool bf16, int64_t max_rows, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t lds = fused_lds_bytes(a.E, bf16);
  const void* kern = bf16 ? reinterpret_cast<const void*>(moe_fused_kernel<true>)
                          : reinterpret_cast<const void*>(moe_fused_kernel<false>);
  // the largest dynamic LDS any E can ask for
  static LdsAttr attr[2];
  if (int rc = set_dynamic_lds_once(kern, fused_lds_bytes(MOE_MAX_E, bf16), attr[bf16 ? 1 : 0]))
    return rc;
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, lds);
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
  e = hipLaunchCooperativeKernel(kern, dim3(static_cast<unsigned>(grid)), dim3(256), args,
                                 static_cast<unsigned>(lds), s);
  if (e != hipSuccess) return static_cast<int>(e);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
