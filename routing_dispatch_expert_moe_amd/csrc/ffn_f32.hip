// fp32 grouped expert GEMMs (VALU FMA, no reduced precision anywhere), for
// layers stored in fp32.  Same math and tile scheduler as the bf16 path:
//   up   : h = silu(A W1) * (A W3)      down : y = h W2
// (DWDP page, key optimisations; MegaMoE comparison page, core differences §1.)
#include "common.h"
#include "launch.h"
#include "tile_sched.h"

namespace moe {

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const int32_t* __restrict__ offsets,
                                                       int E_loc, const float* __restrict__ W,
                                                       float* __restrict__ C, int N, int K) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int BNW = SWIGLU ? 2 * BN : BN;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BNW + 4];
  __shared__ int prefix[MOE_MAX_E + 1];
  mtile_prefix<BM>(offsets, E_loc, prefix);
  const int NT = (N + BN - 1) / BN;
  const int total = prefix[E_loc] * NT;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int e = find_expert(prefix, E_loc, tile / NT);
    const int mt_e = prefix[e + 1] - prefix[e];
    const int local = tile - prefix[e] * NT;
    const int nt = local / mt_e, mti = local % mt_e;
    const int seg1 = offsets[e + 1];
    const int m0 = offsets[e] + mti * BM;
    const int n0 = nt * BN;
    const float* We = W + e * wstride;
    float acc[4][4] = {}, accg[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
      {  // A: 64 rows x 16 k, one float4 per thread, stored k-major
        const int r = tid >> 2, kq = (tid & 3) * 4;
        const int row = m0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < seg1 && k0 + kq < K) v = *reinterpret_cast<const float4*>(A + (size_t)row * K + k0 + kq);
        As[kq + 0][r] = v.x; As[kq + 1][r] = v.y; As[kq + 2][r] = v.z; As[kq + 3][r] = v.w;
      }
      for (int c = tid; c < BNW * 4; c += 256) {  // B: BNW weight rows x 16 k
        const int r = c >> 2, kq = (c & 3) * 4;
        const int half = SWIGLU ? r / BN : 0;
        const int n = n0 + (r % BN);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (n < N && k0 + kq < K)
          v = *reinterpret_cast<const float4*>(We + ((size_t)half * N + n) * K + k0 + kq);
        Bs[kq + 0][r] = v.x; Bs[kq + 1][r] = v.y; Bs[kq + 2][r] = v.z; Bs[kq + 3][r] = v.w;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4], g[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = As[kk][ty * 4 + i];
          b[i] = Bs[kk][tx * 4 + i];
          if (SWIGLU) g[i] = Bs[kk][BN + tx * 4 + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            if (SWIGLU) accg[i][j] = fmaf(a[i], g[j], accg[i][j]);
          }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      if (row >= seg1) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col >= N) continue;
        float v = acc[i][j];
        if (SWIGLU) v = v / (1.f + expf(-v)) * accg[i][j];
        C[(size_t)row * N + col] = v;
      }
    }
  }
}

template <bool SWIGLU>
static int launch_f32(const float* A, const int32_t* offsets, int E_loc, int64_t max_rows,
                      const float* W, float* C, int N, int K, hipStream_t s) {
  const int64_t NT = (N + 63) / 64;
  int64_t grid = (max_rows / 64 + E_loc) * NT;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 4;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(gemm_f32_kernel<SWIGLU>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     A, offsets, E_loc, W, C, N, K);
  return static_cast<int>(hipGetLastError());
}

int launch_ffn_up_f32(const float* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, const float* w13, float* h, void* stream) {
  if (max_rows == 0) return 0;
  return launch_f32<true>(x_perm, offsets, E_loc, max_rows, w13, h, f, d,
                          static_cast<hipStream_t>(stream));
}

int launch_ffn_down_f32(const float* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, const float* w2, float* y, void* stream) {
  if (max_rows == 0) return 0;
  return launch_f32<false>(h, offsets, E_loc, max_rows, w2, y, d, f,
                           static_cast<hipStream_t>(stream));
}

}  // namespace moe
