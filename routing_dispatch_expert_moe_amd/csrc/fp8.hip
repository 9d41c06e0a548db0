// Block quantisation of packed bf16 expert weights to E4M3-FN codes with one
// fp32 scale per 128 x 128 block (NCCL EP page §2.1: FP8 expert compute with
// a scale tensor).  For each block: amax = max |w|, scale = amax / 448
// (correctly rounded fp32 division; an all-zero block gets scale 1), and
// code = E4M3(w / scale), rounded to nearest even and saturated at 448.
//
// One 256-thread workgroup per block: thread t owns row t / 2 of the block
// and 64 consecutive K-columns (128 bytes of bf16 in, 64 bytes of codes out).
#include "fp8_dev.h"
#include "launch.h"

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
  const float scale = amax > 0.f ? __fdiv_rn(amax, kE4M3Max) : 1.f;
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

}  // namespace moe
