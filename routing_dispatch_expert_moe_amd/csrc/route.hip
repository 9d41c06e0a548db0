// Router logits and top-k routing on gfx950.
//
// Router (MoE sparse-activation page, §3.1 router row and §5.3 scenario 3):
// logits = x . W_g with fp32 products and accumulation.
// Top-k (same page §3.2 stage 2): the k largest fp32 logits per token, ties to
// the lower expert index, best first; gates softmax-renormalised over the k,
// or sigmoid normalised over the k.
#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// A0: logits[t][e] = sum_i x[t][i] * wg[i][e]; x bf16, wg fp32.
// One wave handles TPW tokens; lanes stride over 8-element chunks of d, so
// each x load is a coalesced 16-byte access and wg rows are shared by the
// TPW tokens.  Partial sums meet in a fixed butterfly (deterministic).
// ---------------------------------------------------------------------------
template <int EB, int TPW>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wg,
                                                            int T, int d, int E,
                                                            float* __restrict__ logits) {
  const int lane = lane_id();
  const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  if (t0 >= T) return;
  float acc[TPW][EB];
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int e = 0; e < EB; ++e) acc[a][e] = 0.f;
  const int nchunk = d >> 3;
  for (int c = lane; c < nchunk; c += kWave) {
    float xv[TPW][8];
#pragma unroll
    for (int a = 0; a < TPW; ++a) {
      if (t0 + a < T) {
        uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + a) * d + c * 8);
        unpack8(v, xv[a]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[a][i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* wrow = wg + (size_t)(c * 8 + i) * E;
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        float wv = e < E ? wrow[e] : 0.f;
#pragma unroll
        for (int a = 0; a < TPW; ++a) acc[a][e] = fmaf(xv[a][i], wv, acc[a][e]);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      float s = wave_sum_f32(acc[a][e]);
      if (lane == a * EB + e && e < E && t0 + a < T) logits[(size_t)(t0 + a) * E + e] = s;
    }
}

int launch_router_logits(const void* x, const float* wg, int T, int d, int E, float* logits,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  auto grid = [&](int tpw) { return dim3((T + 4 * tpw - 1) / (4 * tpw)); };
  if (E <= 8)
    hipLaunchKernelGGL((router_logits_kernel<8, 4>), grid(4), dim3(256), 0, s, xb, wg, T, d, E, logits);
  else if (E <= 16)
    hipLaunchKernelGGL((router_logits_kernel<16, 2>), grid(2), dim3(256), 0, s, xb, wg, T, d, E, logits);
  else if (E <= 32)
    hipLaunchKernelGGL((router_logits_kernel<32, 1>), grid(1), dim3(256), 0, s, xb, wg, T, d, E, logits);
  else
    hipLaunchKernelGGL((router_logits_kernel<64, 1>), grid(1), dim3(256), 0, s, xb, wg, T, d, E, logits);
  return static_cast<int>(hipGetLastError());
}

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

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int gate, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0;
    if (e < E) key[i] = (static_cast<uint64_t>(ordered_bits(row[e])) << 32) | static_cast<uint32_t>(~e);
  }
  int sel_e[MOE_MAX_K];
  float sel_v[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    if (j < k) {
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

}  // namespace moe
