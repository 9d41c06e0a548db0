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

}  // namespace moe
