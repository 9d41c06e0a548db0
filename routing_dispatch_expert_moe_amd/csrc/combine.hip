// Stand-alone launcher of the weighted combine (combine_dev.h): one wave per
// token.
#include "combine_dev.h"
#include "launch.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y_perm,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int chunks, uint4* __restrict__ y) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  combine_token<BF16>(y_perm, pair_pos, topk_w, t, k, chunks, y);
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
