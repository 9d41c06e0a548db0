// Stand-alone launchers of the fp32 grouped expert GEMMs (gemm_f32.h).
#include "gemm_f32.h"
#include "launch.h"

namespace moe {

template <bool SWIGLU, bool SAVE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ offsets,
                                                       int E_loc, const float* __restrict__ W,
                                                       float* __restrict__ C, int N, int K,
                                                       const float* const* __restrict__ wlist,
                                                       float* __restrict__ AB) {
  __shared__ float smem[f32_lds_floats(SWIGLU)];
  __shared__ int prefix[MOE_MAX_E + 1];
  gemm_f32_body<SWIGLU, SAVE>(A, offsets, E_loc, W, C, N, K, blockIdx.x, gridDim.x, smem, prefix,
                              nullptr, 1, wlist, AB);
}

template <bool SWIGLU, bool SAVE = false>
static int launch_f32(const float* A, const int32_t* offsets, int E_loc, int64_t max_rows,
                      const float* W, float* C, int N, int K, const void* const* wlist,
                      hipStream_t s, float* AB = nullptr) {
  const int64_t NT = (N + 63) / 64;
  int64_t grid = (max_rows / 64 + E_loc) * NT;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 4;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((gemm_f32_kernel<SWIGLU, SAVE>), dim3(static_cast<unsigned>(grid)), dim3(256),
                     0, s, A, offsets, E_loc, W, C, N, K,
                     reinterpret_cast<const float* const*>(wlist), AB);
  return static_cast<int>(hipGetLastError());
}

int launch_ffn_up_f32(const float* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, const float* w13, float* h, const void* const* wlist,
                      void* stream) {
  if (max_rows == 0) return 0;
  return launch_f32<true>(x_perm, offsets, E_loc, max_rows, w13, h, f, d, wlist,
                          static_cast<hipStream_t>(stream));
}

int launch_ffn_up_train_f32(const float* x_perm, const int32_t* offsets, int E_loc,
                            int64_t max_rows, int d, int f, const float* w13, float* h, float* ab,
                            void* stream) {
  if (max_rows == 0) return 0;
  return launch_f32<true, true>(x_perm, offsets, E_loc, max_rows, w13, h, f, d, nullptr,
                                static_cast<hipStream_t>(stream), ab);
}

int launch_ffn_down_f32(const float* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, const float* w2, float* y, const void* const* wlist,
                        void* stream) {
  if (max_rows == 0) return 0;
  return launch_f32<false>(h, offsets, E_loc, max_rows, w2, y, d, f, wlist,
                           static_cast<hipStream_t>(stream));
}

}  // namespace moe
