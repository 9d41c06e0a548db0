// Router logits and top-k routing on gfx950.
//
// Router (MoE sparse-activation page, §3.1 router row and §5.3 scenario 3):
// logits = x . W_g with fp32 products and accumulation.
// Top-k (same page §3.2 stage 2): the k largest fp32 logits per token, ties to
// the lower expert index, best first; gates softmax-renormalised over the k,
// or sigmoid normalised over the k.
#include "common.h"
#include "launch.h"
#include "route_dev.h"

namespace moe {

// ---------------------------------------------------------------------------
// A0: logits[t][e] = sum_i x[t][i] * wg[i][e]; x bf16 (exact in fp32), wg fp32,
// fp32 products and sums.
// A workgroup takes TPW = 64 / EB tokens (EB = E rounded up to 8, 16, 32 or
// 64), so each lane's partial sums are TPW x EB = 64 values.  The 4 waves
// split d into quarters; in a wave, lane c takes 8-element chunks c, c + 64,
// ... of its quarter: the x loads of one token are 1 KB contiguous per wave,
// and each wg row segment a lane loads serves all TPW tokens.  The 64 partial
// sums are then reduce-scattered across the 64 lanes (6 xor rounds, halving
// the values each round: lane l ends with the wave's total of value l) and
// the 4 waves' totals are added in wave order through LDS.  Every sum has a
// fixed order, so the result is deterministic.
// ---------------------------------------------------------------------------
template <int EB>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wg,
                                                            int T, int d, int E,
                                                            float* __restrict__ logits) {
  constexpr int TPW = 64 / EB;  // tokens per workgroup
  __shared__ float part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * TPW;
  const int nchunk = d >> 3;
  const int per = (nchunk + 3) / 4;
  const int c_lo = wave * per, c_hi = min(nchunk, c_lo + per);
  const bool vec = (E & 3) == 0;  // wg rows are 16-byte aligned runs of E floats
  float v[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = 0.f;
  for (int c = c_lo + lane; c < c_hi; c += kWave) {
    float xf[TPW][8];
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      if (t0 + a < T) {
        unpack8(*reinterpret_cast<const uint4*>(x + (size_t)(t0 + a) * d + c * 8), xf[a]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xf[a][i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* wrow = wg + (size_t)(c * 8 + i) * E;
#pragma unroll
      for (int e4 = 0; e4 < EB / 4; ++e4) {
        float w[4];
        if (vec) {
          float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
          if (e4 * 4 < E) q = reinterpret_cast<const float4*>(wrow)[e4];
          w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) w[u] = e4 * 4 + u < E ? wrow[e4 * 4 + u] : 0.f;
        }
#pragma unroll
        for (int a = 0; a < TPW; ++a)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            v[a * EB + e4 * 4 + u] = fmaf(xf[a][i], w[u], v[a * EB + e4 * 4 + u]);
      }
    }
  }
  // reduce-scatter over the wave: after the round with mask m a lane keeps
  // the upper half of its values if (lane & m), so lane l ends with value l
#pragma unroll
  for (int m = 32, n = 64; m >= 1; m >>= 1, n >>= 1) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < n / 2; ++j) {
      const float keep = up ? v[j + n / 2] : v[j];
      const float give = up ? v[j] : v[j + n / 2];
      v[j] = keep + __shfl_xor(give, m, kWave);
    }
  }
  part[wave][lane] = v[0];
  __syncthreads();
  if (wave == 0) {
    const float sum = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    const int a = lane / EB, e = lane % EB;
    if (t0 + a < T && e < E) logits[(size_t)(t0 + a) * E + e] = sum;
  }
}

int launch_router_logits(const void* x, const float* wg, int T, int d, int E, float* logits,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const dim3 block(256);
  if (E <= 8)
    hipLaunchKernelGGL(router_logits_kernel<8>, dim3((T + 7) / 8), block, 0, s, xb, wg, T, d, E, logits);
  else if (E <= 16)
    hipLaunchKernelGGL(router_logits_kernel<16>, dim3((T + 3) / 4), block, 0, s, xb, wg, T, d, E, logits);
  else if (E <= 32)
    hipLaunchKernelGGL(router_logits_kernel<32>, dim3((T + 1) / 2), block, 0, s, xb, wg, T, d, E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<64>, dim3(T), block, 0, s, xb, wg, T, d, E, logits);
  return static_cast<int>(hipGetLastError());
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int gate, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<EPL>(logits, t, E, k, gate, topk_idx, topk_w);
}

int launch_route(const float* logits, int T, int E, int k, int gate, int32_t* idx, float* w,
                 void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL((route_kernel<1>), grid, block, 0, s, logits, T, E, k, gate, idx, w);
  else if (E <= 128)
    hipLaunchKernelGGL((route_kernel<2>), grid, block, 0, s, logits, T, E, k, gate, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL((route_kernel<4>), grid, block, 0, s, logits, T, E, k, gate, idx, w);
  else if (E <= 512)
    hipLaunchKernelGGL((route_kernel<8>), grid, block, 0, s, logits, T, E, k, gate, idx, w);
  else
    hipLaunchKernelGGL((route_kernel<16>), grid, block, 0, s, logits, T, E, k, gate, idx, w);
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Routing with overflow rerouting (MoE sparse-activation page §3.2, stage 3:
// a token whose best expert has reached its capacity takes the next expert
// after its k instead).  In token order, an expert's load is the number of
// earlier tokens whose final choice holds it.
//
// Step 1 (all tokens in parallel, one wave per token): the k + 1 best experts
// and their logits, as candidates.  Step 2 (one workgroup) decides which
// tokens reroute, and nothing else: the candidate experts pass through LDS in
// chunks; while one wave resolves a chunk, the other seven stage the next, so
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
// on the chain.
// ---------------------------------------------------------------------------
constexpr int kMaxCand = MOE_MAX_K + 1;

template <int EPL>
__global__ __launch_bounds__(256) void route_candidates_kernel(const float* __restrict__ logits,
                                                               int T, int E, int kc,
                                                               int32_t* __restrict__ cand_e,
                                                               float* __restrict__ cand_v) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
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

constexpr int kRerouteThreads = 512;  // one resolving wave + seven loader waves

// Step 2; requires capacity >= 0 and K < E (k + 1 candidates per token).
// rerouted[g] bit l: token 64 g + l reroutes.
template <int K>
__global__ __launch_bounds__(kRerouteThreads) void reroute_resolve_kernel(
    const int32_t* __restrict__ cand_e, int T, int E, int capacity,
    uint64_t* __restrict__ rerouted) {
  constexpr int KC = K + 1;
  constexpr int CH0 = (7680 / KC) & ~63;
  constexpr int CH = CH0 < 2048 ? CH0 : 2048;  // tokens per chunk (LDS: 2 x 30 KB at most)
  static_assert(CH >= kWave, "chunk smaller than a wave");
  constexpr int kLoaders = kRerouteThreads - kWave;
  constexpr int U = 8;  // loads in flight per loader thread
  __shared__ int load[MOE_MAX_E];
  __shared__ int32_t ce[2][CH * KC];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const bool resolver = tid < kWave;
  for (int e = tid; e < E; e += kRerouteThreads) load[e] = 0;
  // loader threads: chunk c's candidates (contiguous in memory) into buffer b
  auto stage = [&](int c, int b) {
    const int t0 = c * CH;
    const int n = min(CH, T - t0) * KC;
    const int32_t* src = cand_e + (size_t)t0 * KC;
    for (int i0 = tid - kWave; i0 < n; i0 += kLoaders * U) {
      int32_t re[U];
#pragma unroll
      for (int u = 0; u < U; ++u) re[u] = src[min(i0 + u * kLoaders, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * kLoaders < n) ce[b][i0 + u * kLoaders] = re[u];
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
      const int32_t* be = ce[c & 1];
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

// Step 3: final experts (best first) and gates, one token per thread;
// rerouted == nullptr: no token reroutes.
template <int K>
__global__ __launch_bounds__(256) void reroute_finalize_kernel(
    const int32_t* __restrict__ cand_e, const float* __restrict__ cand_v,
    const uint64_t* __restrict__ rerouted, int T, int kc, int gate,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
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

int launch_route_reroute(const float* logits, int T, int E, int k, int gate, int capacity,
                         int32_t* idx, float* w, int32_t* cand_e, float* cand_v,
                         uint64_t* rerouted, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return 0;
  const int kc = k < E ? k + 1 : k;
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL((route_candidates_kernel<1>), grid, block, 0, s, logits, T, E, kc, cand_e, cand_v);
  else if (E <= 128)
    hipLaunchKernelGGL((route_candidates_kernel<2>), grid, block, 0, s, logits, T, E, kc, cand_e, cand_v);
  else if (E <= 256)
    hipLaunchKernelGGL((route_candidates_kernel<4>), grid, block, 0, s, logits, T, E, kc, cand_e, cand_v);
  else if (E <= 512)
    hipLaunchKernelGGL((route_candidates_kernel<8>), grid, block, 0, s, logits, T, E, kc, cand_e, cand_v);
  else
    hipLaunchKernelGGL((route_candidates_kernel<16>), grid, block, 0, s, logits, T, E, kc, cand_e, cand_v);
  const bool can = capacity >= 0 && k < E;
  const dim3 fgrid((T + 255) / 256);
  switch (k) {
#define MOE_REROUTE_K(KK)                                                                     \
  case KK:                                                                                   \
    if (can)                                                                                 \
      hipLaunchKernelGGL(reroute_resolve_kernel<KK>, dim3(1), dim3(kRerouteThreads), 0, s,  \
                         cand_e, T, E, capacity, rerouted);                                  \
    hipLaunchKernelGGL(reroute_finalize_kernel<KK>, fgrid, dim3(256), 0, s, cand_e, cand_v, \
                       can ? rerouted : nullptr, T, kc, gate, idx, w);                       \
    break;
    MOE_REROUTE_K(1) MOE_REROUTE_K(2) MOE_REROUTE_K(3) MOE_REROUTE_K(4)
    MOE_REROUTE_K(5) MOE_REROUTE_K(6) MOE_REROUTE_K(7) MOE_REROUTE_K(8)
#undef MOE_REROUTE_K
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
