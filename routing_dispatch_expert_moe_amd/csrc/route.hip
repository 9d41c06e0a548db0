// Router logits and top-k routing on gfx950.
//
// Router (MoE sparse-activation page, §3.1 router row and §5.3 scenario 3):
// logits = x . W_g with fp32 products and accumulation.
// Top-k (same page §3.2 stage 2): the k largest fp32 logits per token, ties to
// the lower expert index, best first; gates softmax-renormalised over the k,
// or sigmoid normalised over the k.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "reroute_dev.h"
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

// More than 64 experts: a workgroup computes a tile of TT tokens x 64
// experts (TT = 64, or 16 when there are few tokens, for more workgroups).
// K-chunks of KC = 32 of x (bf16 -> fp32, exact) and of wg go through LDS,
// the next chunk's loads in flight in registers while the current chunk is
// summed; thread (ty, tx) of 16 x 16 accumulates tokens ty * TT/16 ..
// (ty + 1) * TT/16 - 1 by experts 4tx .. 4tx+3, each sum one fp32 fma per i in
// increasing order, so the result is deterministic.  x is read once per
// 64-expert column of tiles and wg once per row of token tiles.
constexpr int kRlE = 64;

template <int TT, int KC>
__global__ __launch_bounds__(256) void router_logits_tiled_kernel(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ wg,
                                                                  int T, int d, int E,
                                                                  float* __restrict__ logits) {
  constexpr int R = TT / 16;                // token rows per thread
  constexpr int XCH = KC / 8;               // 8-value x chunks per token and K-chunk
  constexpr int WPT = KC * kRlE / 256;      // wg values staged per thread
  static_assert(TT * XCH <= 256 && WPT * 256 == KC * kRlE, "staging roles");
  __shared__ float xs[TT][KC + 1];          // [token][i], padded against bank conflicts
  __shared__ float ws[KC][kRlE];            // [i][expert]
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * kRlE;
  float acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  // staging roles: x, thread < TT * XCH -> (token tid / XCH, 8 values at
  // chunk tid % XCH); wg, element j * 256 + tid of the KC x 64 tile (row
  // 4j + tid / 64, expert tid % 64): coalesced loads, conflict-free LDS writes
  const int xt = tid / XCH, xc = (tid % XCH) * 8;
  const bool xrole = tid < TT * XCH;
  const int wi = tid / kRlE, we = tid % kRlE;
  constexpr int WROWS = 256 / kRlE;  // tile rows one pass of the threads covers
  uint4 xr = make_uint4(0u, 0u, 0u, 0u);
  float wr[WPT];
  auto fetch = [&](int d0) {
    xr = make_uint4(0u, 0u, 0u, 0u);
    if (xrole && t0 + xt < T && d0 + xc < d)  // d % 8 == 0: a chunk is wholly in or out
      xr = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + xt) * d + d0 + xc);
    const int e = e0 + we;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int i = d0 + j * WROWS + wi;
      wr[j] = (i < d && e < E) ? wg[(size_t)i * E + e] : 0.f;
    }
  };
  fetch(0);
  for (int d0 = 0; d0 < d; d0 += KC) {
    if (xrole) {
      float xf[8];
      unpack8(xr, xf);
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[xt][xc + i] = xf[i];
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j) ws[j * WROWS + wi][we] = wr[j];
    __syncthreads();
    if (d0 + KC < d) fetch(d0 + KC);
#pragma unroll 8
    for (int i = 0; i < KC; ++i) {
      float a[R], b[4];
#pragma unroll
      for (int r = 0; r < R; ++r) a[r] = xs[ty * R + r][i];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = ws[i][tx * 4 + c];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + ty * R + r;
    if (t >= T) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = e0 + tx * 4 + c;
      if (e < E) logits[(size_t)t * E + e] = acc[r][c];
    }
  }
}

int launch_router_logits(const void* x, const float* wg, int T, int d, int E, float* logits,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const dim3 block(256);
  if (E > 64) {
    // 64-token tiles once they give a few workgroups per CU, else 16
    const int ecol = (E + kRlE - 1) / kRlE;
    if (static_cast<int64_t>((T + 63) / 64) * ecol >= 2 * device_cu_count()) {
      const dim3 grid((T + 63) / 64, ecol);
      hipLaunchKernelGGL((router_logits_tiled_kernel<64, 32>), grid, block, 0, s, xb, wg, T, d, E, logits);
    } else {
      const dim3 grid((T + 15) / 16, ecol);
      hipLaunchKernelGGL((router_logits_tiled_kernel<16, 32>), grid, block, 0, s, xb, wg, T, d, E, logits);
    }
    return static_cast<int>(hipGetLastError());
  }
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

// Routing with overflow rerouting: the stand-alone launches of the three steps
// of reroute_dev.h (candidates, the one-workgroup resolver with seven loader
// waves, gates).
constexpr int kRerouteThreads = 512;

template <int EPL>
__global__ __launch_bounds__(256) void route_candidates_kernel(const float* __restrict__ logits,
                                                               int T, int E, int kc,
                                                               int32_t* __restrict__ cand_e,
                                                               float* __restrict__ cand_v) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  reroute_candidates_token<EPL>(logits, t, E, kc, cand_e, cand_v);
}

template <int K>
__global__ __launch_bounds__(kRerouteThreads) void reroute_resolve_kernel(
    const int32_t* __restrict__ cand_e, int T, int E, int capacity,
    uint64_t* __restrict__ rerouted) {
  __shared__ int load[MOE_MAX_E];
  __shared__ int32_t ce[2 * reroute_chunk<K>() * (K + 1)];
  reroute_resolve_body<K, kRerouteThreads>(cand_e, T, E, capacity, rerouted, load, ce);
}

template <int K>
__global__ __launch_bounds__(256) void reroute_finalize_kernel(
    const int32_t* __restrict__ cand_e, const float* __restrict__ cand_v,
    const uint64_t* __restrict__ rerouted, int T, int kc, int gate,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  reroute_finalize_token<K>(cand_e, cand_v, rerouted, t, kc, gate, topk_idx, topk_w);
}

// The fixed scratch of moe_route_reroute_noalloc: one array per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel (in host code it is a host-side stand-in, not a device address):
// each device's address is looked up once, with that device current, and
// kept here.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
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
