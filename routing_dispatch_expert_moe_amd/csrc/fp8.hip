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

// Grouped expert GEMM over FP8 weights for few rows per expert (decode):
// the weight stream is the cost, so the weight tile stays in LDS as codes (one
// byte per weight) and each MFMA operand is converted to bf16 right after its
// LDS read (the hardware conversion is exact for E4M3).  One 128-deep K step
// per stage covers one scale block: its partial sums are multiplied by the
// block's scale and added to the result.  A single LDS stage (the next step's
// codes wait in registers) keeps a workgroup at 44 KB of LDS, so three run on
// a CU and three steps of codes are in flight per CU.
//
// Tile: 32 activation rows x BN output columns (SwiGLU: BN W1 rows + the BN
// matching W3 rows); 4 waves, each owning 32 x BN/4.  Rows of each expert are
// the segment [offsets[e], offsets[e+1]); the persistent grid walks tiles in
// expert order, M-tiles fastest, with the XCD-aware workgroup remap.
template <int BN, bool SWIGLU>
__global__ __launch_bounds__(256, 2) void gemm_fp8w_kernel(const uint16_t* __restrict__ A,
                                                        const int32_t* __restrict__ offsets,
                                                        int E_loc, const uint8_t* __restrict__ Wq,
                                                        const float* __restrict__ Ws,
                                                        uint16_t* __restrict__ C, int N, int K) {
  constexpr int BM = 32, BK = kFp8Block, WN = 4, NTHR = 256;
  constexpr int BNW = SWIGLU ? 2 * BN : BN;  // weight rows per tile
  constexpr int TN = BN / WN, FN = TN / 32;  // wave tile columns, 32-column MFMA blocks
  constexpr int AKC = BK / 8;                // 16-byte bf16 chunks per activation row
  constexpr int BU = BK / 16;                // 16-byte code units per weight row
  constexpr int CA = BM * AKC / NTHR;
  constexpr int CB = BNW * BU / NTHR;
  static_assert(FN >= 1 && TN % 32 == 0 && CA * NTHR == BM * AKC && CB * NTHR == BNW * BU,
                "tile / thread mismatch");
  __shared__ uint4 As[BM * AKC];   // row r, chunk c at c ^ (r & 15)
  __shared__ uint4 Bq[BNW * BU];   // row r, unit u at u ^ ((r >> 1) & 7)
  __shared__ int prefix[MOE_MAX_E + 1];

  mtile_prefix<BM, ROWS_ALL>(offsets, E_loc, prefix);
  const int NT = (N + BN - 1) / BN;
  const int total = prefix[E_loc] * NT;
  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int tid = threadIdx.x, wn = tid >> 6, lane = tid & 63;
  const int KT = K / BK;
  const int RB = (SWIGLU ? 2 * N : N) / kFp8Block;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;

  for (int tile = vb; tile < total; tile += G) {
    const int e = find_expert(prefix, E_loc, tile / NT);
    const int mt_e = prefix[e + 1] - prefix[e];
    const int local = tile - prefix[e] * NT;
    const int nt = local / mt_e, mti = local % mt_e;
    const int seg0 = offsets[e], seg1 = offsets[e + 1];
    const int m0 = seg0 + mti * BM, n0 = nt * BN;

    // per-thread load descriptors; rows past the segment or the matrix read a
    // valid row and are zeroed when staged (the loads stay branch-free)
    const uint16_t* a_src[CA];
    bool a_ok[CA];
    int a_dst[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NTHR, r = c / AKC, kc = c % AKC;
      a_ok[i] = m0 + r < seg1;
      a_src[i] = A + static_cast<size_t>(a_ok[i] ? m0 + r : seg0) * K + kc * 8;
      a_dst[i] = r * AKC + (kc ^ (r & 15));
    }
    const uint8_t* b_src[CB];
    bool b_ok[CB];
    int b_dst[CB];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NTHR, r = c / BU, u = c % BU;
      const int half = SWIGLU ? r / BN : 0, n = n0 + r % BN;
      b_ok[i] = n < N;
      b_src[i] = Wq + e * wstride + (static_cast<size_t>(half) * N + (b_ok[i] ? n : 0)) * K + u * 16;
      b_dst[i] = r * BU + (u ^ ((r >> 1) & 7));
    }
    uint4 ra[CA], rq[CB];
    auto gload = [&](int kt) {
      const int koff = kt * BK;
#pragma unroll
      for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + koff);
#pragma unroll
      for (int i = 0; i < CB; ++i) rq[i] = *reinterpret_cast<const uint4*>(b_src[i] + koff);
    };
    auto sel4 = [](bool ok, uint4 v) {
      return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
    };
    auto sstore = [&]() {
#pragma unroll
      for (int i = 0; i < CA; ++i) As[a_dst[i]] = sel4(a_ok[i], ra[i]);
#pragma unroll
      for (int i = 0; i < CB; ++i) Bq[b_dst[i]] = sel4(b_ok[i], rq[i]);
    };
    // 8 codes of weight row r at K offset ks * 16 + h * 8 of the stage, as bf16
    auto bfrag = [&](int r, int ks, int h) {
      const uint2 q = *reinterpret_cast<const uint2*>(
          reinterpret_cast<const char*>(Bq) + (r * BU + (ks ^ ((r >> 1) & 7))) * 16 + h * 8);
      const int x = static_cast<int>(q.x), y = static_cast<int>(q.y);
      const uint4 v = make_uint4(
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, true)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.f, true)));
      return __builtin_bit_cast(bf16x8_t, v);
    };

    f32x16_t acc[FN], accg[SWIGLU ? FN : 1], part[FN], partg[SWIGLU ? FN : 1];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[j] = part[j] = f32x16_t{};
      if constexpr (SWIGLU) accg[j] = partg[j] = f32x16_t{};
    }
    // block scales of step kt (the wave's columns lie in one 128-row block)
    float sc[FN], scg[SWIGLU ? FN : 1];
    auto sload = [&](int kt) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int rowb = (n0 + wn * TN + j * 32) / kFp8Block;
        sc[j] = Ws[(static_cast<size_t>(e) * RB + rowb) * KT + kt];
        if constexpr (SWIGLU)
          scg[j] = Ws[(static_cast<size_t>(e) * RB + N / kFp8Block + rowb) * KT + kt];
      }
    };
    sload(0);
    gload(0);
    sstore();
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      float scc[FN], scgc[SWIGLU ? FN : 1];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        scc[j] = sc[j];
        if constexpr (SWIGLU) scgc[j] = scg[j];
      }
      // the next step's scales and codes load under this step's MFMAs (the
      // last step re-fetches: valid, unused); the scheduling barrier keeps
      // them ahead of the MFMAs (left to itself the scheduler sinks them next
      // to the LDS stores that consume them, exposing the memory latency)
      sload(min(kt + 1, KT - 1));
      gload(min(kt + 1, KT - 1));
      __builtin_amdgcn_sched_barrier(0);
      const int h = lane >> 5;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ra_row = lane & 31, ch = ks * 2 + h;
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, As[ra_row * AKC + (ch ^ (ra_row & 15))]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * TN + j * 32 + (lane & 31);
          part[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfrag(r, ks, h), part[j], 0, 0, 0);
          if constexpr (SWIGLU)
            partg[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfrag(BN + r, ks, h), partg[j],
                                                               0, 0, 0);
        }
      }
      // the step is one scale block: scale its partial sums into the result
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[j] += scc[j] * part[j];
        part[j] = f32x16_t{};
        if constexpr (SWIGLU) {
          accg[j] += scgc[j] * partg[j];
          partg[j] = f32x16_t{};
        }
      }
      __syncthreads();  // every wave is done with this stage
      sstore();
      __syncthreads();
    }

    // epilogue: D[m][n] of a 32x32 tile sits in lane n + 32 * ((m / 4) % 2),
    // register 4 * (m / 8) + m % 4
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * TN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float v = acc[j][r];
        if constexpr (SWIGLU) v = v * __builtin_amdgcn_rcpf(1.f + __expf(-v)) * accg[j][r];
        if (row < seg1 && col < N) C[static_cast<size_t>(row) * N + col] = f32_to_bf16(v);
      }
    }
  }
}

int launch_gemm_fp8w(bool swiglu, const void* A, const int32_t* offsets, int E_loc,
                     int64_t max_rows, const uint8_t* Wq, const float* Ws, void* C, int N, int K,
                     void* stream) {
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
  if (swiglu)
    hipLaunchKernelGGL((gemm_fp8w_kernel<BN, true>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, a, offsets, E_loc, Wq, Ws, c, N, K);
  else
    hipLaunchKernelGGL((gemm_fp8w_kernel<BN, false>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, s, a, offsets, E_loc, Wq, Ws, c, N, K);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
