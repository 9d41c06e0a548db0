// Weighted combine (NCCL EP page §2.1, LL combine): for each token, the sum
// over its k choices of gate weight times that pair's expert output row.
// One wave per token; 16-byte loads of every contributing row; fp32
// accumulation in ascending j; one rounding at the store.  No atomics: each
// output row is owned by exactly one wave, so the result is deterministic.
#include "common.h"
#include "launch.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y_perm,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int chunks, uint4* __restrict__ y) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int rows[MOE_MAX_K];
  float w[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    rows[j] = j < k ? pair_pos[(size_t)t * k + j] : -1;
    w[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
  }
  for (int c = lane; c < chunks; c += kWave) {
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (rows[j] < 0) continue;
      const uint4 v = y_perm[(size_t)rows[j] * chunks + c];
      float f[EPC];
      if constexpr (BF16) {
        unpack8(v, f);
      } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
      }
#pragma unroll
      for (int i = 0; i < EPC; ++i) acc[i] = fmaf(w[j], f[i], acc[i]);
    }
    uint4 o;
    if constexpr (BF16) {
      o = pack8(acc);
    } else {
      o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3]));
    }
    y[(size_t)t * chunks + c] = o;
  }
}

int launch_combine(const void* y_perm, const int32_t* pair_pos, const float* w, int T, int k,
                   int d, int bf16, void* y, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int chunks = bf16 ? d / 8 : d / 4;
  dim3 grid((T + 3) / 4), block(256);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, s, static_cast<const uint4*>(y_perm),
                       pair_pos, w, T, k, chunks, static_cast<uint4*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, s, static_cast<const uint4*>(y_perm),
                       pair_pos, w, T, k, chunks, static_cast<uint4*>(y));
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
