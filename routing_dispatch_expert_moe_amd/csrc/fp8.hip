// Block quantisation of packed bf16 expert weights to E4M3-FN codes with one
// fp32 scale per 128 x 128 block (NCCL EP page §2.1: FP8 expert compute with
// a scale tensor).  For each block: amax = max |w|, scale = the smallest
// power of two 2^e with amax <= 448 * 2^e (an all-zero block gets scale 1),
// and code = E4M3(w / scale), rounded to nearest even (the division by a
// power of two is exact, and no weight reaches the saturation at 448).  A
// power-of-two scale lets the GEMMs dequantise each operand exactly in the
// hardware's scaled conversion (code * 2^e is a bf16 value), so their K loops
// carry no per-block rescaling of the accumulators.
//
// One 256-thread workgroup per block: thread t owns row t / 2 of the block
// and 64 consecutive K-columns (128 bytes of bf16 in, 64 bytes of codes out).
#include "fp8_dev.h"
#include "gemm_fp8w.h"
#include "launch.h"
#include "tile_sched.h"

namespace moe {

__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ w,
                                                           int R, int K,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scales) {
  const int KB = K / kFp8Block, RB = R / kFp8Block;
  const int kb = blockIdx.x, rb = blockIdx.y, e = blockIdx.z;
  const int row = rb * kFp8Block + (threadIdx.x >> 1);
  const int k0 = kb * kFp8Block + (threadIdx.x & 1) * 64;
  const size_t base = (static_cast<size_t>(e) * R + row) * K + k0;
  const uint4* src = reinterpret_cast<const uint4*>(w + base);
  float v[64];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 c = src[i];
    unpack8(c, v + 8 * i);
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // amax = m * 2^ex with m in [0.5, 1), and 448 = 0.875 * 2^9: the smallest e
  // with amax <= 448 * 2^e is ex - 9 when m <= 0.875, else ex - 8 (bf16
  // weights keep e >= -141, a normal or subnormal fp32 power of two)
  int ex = 0;
  const float m = frexpf(amax, &ex);
  const float scale = amax > 0.f ? ldexpf(1.f, m <= 0.875f ? ex - 9 : ex - 8) : 1.f;
  if (threadIdx.x == 0) scales[(static_cast<size_t>(e) * RB + rb) * KB + kb] = scale;
  uint4* dst = reinterpret_cast<uint4*>(q + base);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        word |= f32_to_e4m3(__fdiv_rn(v[16 * i + 4 * j + b], scale)) << (8 * b);
      wd[j] = word;
    }
    dst[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
}

int launch_quantize_fp8(const void* w, int E_loc, int R, int K, uint8_t* q, float* scales,
                        void* stream) {
  dim3 grid(K / kFp8Block, R / kFp8Block, E_loc);
  hipLaunchKernelGGL(quantize_fp8_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(w), R, K, q, scales);
  return static_cast<int>(hipGetLastError());
}

// Grouped expert GEMM over FP8 weights for few rows per expert (decode): the
// code-streaming body of gemm_fp8w.h, one 256-thread part per workgroup and
// three workgroups per CU (three steps of codes in flight per CU).
template <int BN, bool SWIGLU>
__global__ __launch_bounds__(256, 2) void gemm_fp8w_kernel(const uint16_t* __restrict__ A,
                                                        const int32_t* __restrict__ offsets,
                                                        int E_loc, const uint8_t* __restrict__ Wq,
                                                        const float* __restrict__ Ws,
                                                        uint16_t* __restrict__ C, int N, int K,
                                                        const uint8_t* const* __restrict__ wlist,
                                                        const float* const* __restrict__ slist) {
  __shared__ uint4 lds[Fp8wTile<BN, SWIGLU>::kLdsU4];
  __shared__ int prefix[MOE_MAX_E + 1];
  gemm_fp8w_body<BN, SWIGLU, 1>(A, offsets, E_loc, Wq, Ws, C, N, K, blockIdx.x, gridDim.x, lds,
                                prefix, nullptr, 1, wlist, slist);
}

int launch_gemm_fp8w(bool swiglu, const void* A, const int32_t* offsets, int E_loc,
                     int64_t max_rows, const uint8_t* Wq, const float* Ws, void* C, int N, int K,
                     void* stream, const void* const* wlist, const float* const* slist) {
  constexpr int BN = 128;
  const void* kern = swiglu ? reinterpret_cast<const void*>(gemm_fp8w_kernel<BN, true>)
                            : reinterpret_cast<const void*>(gemm_fp8w_kernel<BN, false>);
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, 0);
  if (e != hipSuccess) return static_cast<int>(e);
  if (occ < 1) occ = 1;
  const int64_t NT = (N + BN - 1) / BN;
  const int64_t tiles_ub = (max_rows / 32 + E_loc) * NT;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * occ;
  if (grid > tiles_ub) grid = tiles_ub;
  if (grid >= 8) grid &= ~static_cast<int64_t>(7);
  if (grid < 1) grid = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* a = static_cast<const uint16_t*>(A);
  uint16_t* c = static_cast<uint16_t*>(C);
  const uint8_t* const* wl = reinterpret_cast<const uint8_t* const*>(wlist);
  if (swiglu)
    hipLaunchKernelGGL((gemm_fp8w_kernel<BN, true>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, a, offsets, E_loc, Wq, Ws, c, N, K, wl, slist);
  else
    hipLaunchKernelGGL((gemm_fp8w_kernel<BN, false>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, a, offsets, E_loc, Wq, Ws, c, N, K, wl, slist);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
