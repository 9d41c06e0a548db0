// fp32 grouped expert GEMMs (VALU FMA, no reduced precision anywhere), for
// layers stored in fp32.  Same math and tile scheduler as the bf16 path:
//   up   : h = silu(A W1) * (A W3)      down : y = h W2
// (DWDP page, key optimisations; MegaMoE comparison page, core differences §1.)
#pragma once

#include "common.h"
#include "tile_sched.h"

namespace moe {

constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

// LDS floats needed by gemm_f32_body
constexpr size_t f32_lds_floats(bool swiglu) {
  return static_cast<size_t>(kF32BK) * (kF32BM + 4) +
         static_cast<size_t>(kF32BK) * ((swiglu ? 2 : 1) * kF32BN + 4);
}

// Workgroup `bid` of `G` walks its tiles.  smem: f32_lds_floats(SWIGLU) floats
// of LDS; prefix: E_loc + 1 ints of LDS.  Every thread must call it.
// gather: if not null, activation row r is row gather[r] / gk of A.
// wlist: if not null, expert e's packed weights start at wlist[e].
// SAVE (SwiGLU only): also store a = A W1 at AB[row][col] and g = A W3 at
// AB[row][N + col] (row pitch 2N) for the backward pass.
template <bool SWIGLU, bool SAVE = false>
__device__ __forceinline__ void gemm_f32_body(const float* __restrict__ A,
                                              const int32_t* __restrict__ offsets, int E_loc,
                                              const float* __restrict__ W, float* __restrict__ C,
                                              int N, int K, int bid, int G, float* smem,
                                              int* prefix, const int32_t* __restrict__ gather = nullptr,
                                              int gk = 1,
                                              const float* const* __restrict__ wlist = nullptr,
                                              float* __restrict__ AB = nullptr) {
  static_assert(SWIGLU || !SAVE, "pre-activations exist only with SwiGLU");
  constexpr int BM = kF32BM, BN = kF32BN, BK = kF32BK;
  constexpr int BNW = SWIGLU ? 2 * BN : BN;
  float (*As)[BM + 4] = reinterpret_cast<float (*)[BM + 4]>(smem);
  float (*Bs)[BNW + 4] = reinterpret_cast<float (*)[BNW + 4]>(smem + BK * (BM + 4));
  mtile_prefix<BM>(offsets, E_loc, prefix);
  const int NT = (N + BN - 1) / BN;
  const int total = prefix[E_loc] * NT;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;

  for (int tile = bid; tile < total; tile += G) {
    const int e = find_expert(prefix, E_loc, tile / NT);
    const int mt_e = prefix[e + 1] - prefix[e];
    const int local = tile - prefix[e] * NT;
    const int nt = local / mt_e, mti = local % mt_e;
    const int seg1 = offsets[e + 1];
    const int m0 = offsets[e] + mti * BM;
    const int n0 = nt * BN;
    const float* We = wlist != nullptr ? wlist[e] : W + e * wstride;
    float acc[4][4] = {}, accg[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
      {  // A: 64 rows x 16 k, one float4 per thread, stored k-major
        const int r = tid >> 2, kq = (tid & 3) * 4;
        const int row = m0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < seg1 && k0 + kq < K) {
          const int src = gather != nullptr ? gather[row] / gk : row;
          v = *reinterpret_cast<const float4*>(A + (size_t)src * K + k0 + kq);
        }
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
        if constexpr (SAVE) {
          AB[(size_t)row * 2 * N + col] = v;
          AB[(size_t)row * 2 * N + N + col] = accg[i][j];
        }
        if (SWIGLU) v = v / (1.f + expf(-v)) * accg[i][j];
        C[(size_t)row * N + col] = v;
      }
    }
  }
  __syncthreads();  // prefix and smem are reused by the caller
}

}  // namespace moe
