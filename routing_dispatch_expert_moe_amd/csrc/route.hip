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
// A workgroup takes 16 tokens; each token's 16 threads are 16 consecutive
// lanes of one wave and split d into interleaved 8-element chunks (lane s
// takes chunks s, s + 16, ...), so the 16 lanes of a token read 256
// contiguous bytes of x per step and the 4 tokens of a wave share every wg
// row they read.  Each thread keeps EB partial sums; the 16 partials of a
// token meet in a fixed xor butterfly (deterministic).
// ---------------------------------------------------------------------------
template <int EB>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wg,
                                                            int T, int d, int E,
                                                            float* __restrict__ logits) {
  constexpr int S = 16;  // threads per token
  const int s = threadIdx.x % S;
  const int t = blockIdx.x * (256 / S) + threadIdx.x / S;
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  if (t < T) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * d);
    const int nchunk = d >> 3;
    constexpr int U = 4;  // chunks per thread in flight
    for (int c0 = s; c0 < nchunk; c0 += U * S) {
      uint4 xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u * S < nchunk) xv[u] = xr[c0 + u * S];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * S;
        if (c >= nchunk) break;
        float xf[8];
        unpack8(xv[u], xf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float* wrow = wg + (size_t)(c * 8 + i) * E;
#pragma unroll
          for (int e = 0; e < EB; ++e)
            if (e < E) acc[e] = fmaf(xf[i], wrow[e], acc[e]);
        }
      }
    }
  }
  // butterfly over the token's 16 lanes (all 64 lanes take part)
#pragma unroll
  for (int e = 0; e < EB; ++e) {
#pragma unroll
    for (int off = 1; off < S; off <<= 1) acc[e] += __shfl_xor(acc[e], off, kWave);
  }
  if (t < T) {
#pragma unroll
    for (int e = 0; e < EB; ++e)
      if (e % S == s && e < E) logits[(size_t)t * E + e] = acc[e];
  }
}

int launch_router_logits(const void* x, const float* wg, int T, int d, int E, float* logits,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const dim3 grid((T + 15) / 16), block(256);
  if (E <= 8)
    hipLaunchKernelGGL(router_logits_kernel<8>, grid, block, 0, s, xb, wg, T, d, E, logits);
  else if (E <= 16)
    hipLaunchKernelGGL(router_logits_kernel<16>, grid, block, 0, s, xb, wg, T, d, E, logits);
  else if (E <= 32)
    hipLaunchKernelGGL(router_logits_kernel<32>, grid, block, 0, s, xb, wg, T, d, E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<64>, grid, block, 0, s, xb, wg, T, d, E, logits);
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
