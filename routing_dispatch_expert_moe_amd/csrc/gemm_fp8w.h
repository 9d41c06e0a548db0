// Grouped expert GEMM over FP8 weights for few rows per expert (decode),
// shared by the stand-alone kernel (fp8.hip) and the fused layer (fused.hip).
//
// The weight stream is the cost, so the weight tile stays in LDS as codes (one
// byte per weight) and each MFMA operand is converted to bf16 right after its
// LDS read (the hardware conversion is exact for E4M3).  One 128-deep K step
// per stage covers one scale block: its partial sums are multiplied by the
// block's scale and added to the result.  A single LDS stage (the next step's
// codes wait in registers) keeps a 256-thread part at 44 KB of LDS.
//
// Tile: 32 activation rows x BN output columns (SwiGLU: BN W1 rows + the BN
// matching W3 rows); 4 waves, each owning 32 x BN/4.  Rows of each expert are
// the segment [offsets[e], offsets[e+1]); the persistent grid walks tiles in
// expert order, M-tiles fastest, with the XCD-aware workgroup remap.
#pragma once

#include "common.h"
#include "fp8_dev.h"
#include "tile_sched.h"

namespace moe {

template <int BN, bool SWIGLU>
struct Fp8wTile {
  static constexpr int BM = 32, BK = kFp8Block, WN = 4, NTHR = 256;
  static constexpr int BNW = SWIGLU ? 2 * BN : BN;  // weight rows per tile
  static constexpr int AKC = BK / 8;                // 16-byte bf16 chunks per activation row
  static constexpr int BU = BK / 16;                // 16-byte code units per weight row
  static constexpr int kLdsU4 = BM * AKC + BNW * BU;  // LDS of one part, in uint4
};

// LDS of a workgroup running `parts` 256-thread parts
template <int BN, bool SWIGLU>
constexpr size_t fp8w_lds_bytes(int parts) {
  return static_cast<size_t>(parts) * Fp8wTile<BN, SWIGLU>::kLdsU4 * sizeof(uint4);
}

// PARTS 256-thread parts of the workgroup each run a tile of their own (part
// p takes virtual workgroup PARTS * vb + p), with the workgroup's barriers in
// step: every part runs the same number of K steps per round, and a part with
// no tile left in the last round recomputes the last tile without storing it.
// lds: fp8w_lds_bytes(PARTS) bytes; prefix: MOE_MAX_E + 1 ints of LDS.
// gather: if not null, activation row r is row gather[r] / gk of A (the fused
// layer reads the token rows in place).  N and K are multiples of 128.
// wlist / slist: if not null, expert e's codes start at wlist[e] and its
// block scales at slist[e] (tables of per-expert buffers) instead of
// Wq + e * rows * K and Ws + e * (rows / 128) * (K / 128).
template <int BN, bool SWIGLU, int PARTS>
__device__ __forceinline__ void gemm_fp8w_body(const uint16_t* __restrict__ A,
                                               const int32_t* __restrict__ offsets, int E_loc,
                                               const uint8_t* __restrict__ Wq,
                                               const float* __restrict__ Ws,
                                               uint16_t* __restrict__ C, int N, int K, int bid,
                                               int G, uint4* lds, int* prefix,
                                               const int32_t* __restrict__ gather = nullptr,
                                               int gk = 1,
                                               const uint8_t* const* __restrict__ wlist = nullptr,
                                               const float* const* __restrict__ slist = nullptr) {
  using P = Fp8wTile<BN, SWIGLU>;
  constexpr int BM = P::BM, BK = P::BK, WN = P::WN, NTHR = P::NTHR;
  constexpr int BNW = P::BNW, AKC = P::AKC, BU = P::BU;
  constexpr int TN = BN / WN, FN = TN / 32;  // wave tile columns, 32-column MFMA blocks
  constexpr int CA = BM * AKC / NTHR;
  constexpr int CB = BNW * BU / NTHR;
  static_assert(FN >= 1 && TN % 32 == 0 && CA * NTHR == BM * AKC && CB * NTHR == BNW * BU,
                "tile / thread mismatch");
  static_assert(PARTS >= 1 && PARTS * NTHR <= 1024, "parts of one workgroup");

  mtile_prefix<BM, ROWS_ALL>(offsets, E_loc, prefix);
  const int NTn = (N + BN - 1) / BN;
  const int total = prefix[E_loc] * NTn;
  int vb = bid;
  if ((G & 7) == 0) vb = (bid & 7) * (G >> 3) + (bid >> 3);
  const int part = PARTS == 1 ? 0 : static_cast<int>(threadIdx.x) / NTHR;
  const int tid = static_cast<int>(threadIdx.x) % NTHR, wn = tid >> 6, lane = tid & 63;
  uint4* As = lds + part * P::kLdsU4;  // row r, chunk c at c ^ (r & 15)
  uint4* Bq = As + BM * AKC;           // row r, unit u at u ^ ((r >> 1) & 7)
  const int KT = K / BK;
  const int RB = (SWIGLU ? 2 * N : N) / kFp8Block;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;

  // `first` is the same for every part of the workgroup, so the loop and its
  // barriers are uniform
  for (int first = vb * PARTS; first < total; first += G * PARTS) {
    const bool live = PARTS == 1 || first + part < total;
    const int tile = live ? first + part : total - 1;
    const int e = find_expert(prefix, E_loc, tile / NTn);
    const int mt_e = prefix[e + 1] - prefix[e];
    const int local = tile - prefix[e] * NTn;
    const int nt = local / mt_e, mti = local % mt_e;
    const int seg0 = offsets[e], seg1 = offsets[e + 1];
    const int m0 = seg0 + mti * BM, n0 = nt * BN;

    // per-thread load descriptors; rows past the segment read a valid row and
    // are zeroed when staged (the loads stay branch-free)
    const uint16_t* a_src[CA];
    bool a_ok[CA];
    int a_dst[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NTHR, r = c / AKC, kc = c % AKC;
      a_ok[i] = m0 + r < seg1;
      int arow = a_ok[i] ? m0 + r : seg0;
      if (gather != nullptr) arow = gather[arow] / gk;
      a_src[i] = A + static_cast<size_t>(arow) * K + kc * 8;
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
      b_src[i] = (wlist != nullptr ? wlist[e] : Wq + e * wstride) +
                 (static_cast<size_t>(half) * N + (b_ok[i] ? n : 0)) * K + u * 16;
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

    f32x16_t acc[FN], accg[SWIGLU ? FN : 1], partial[FN], partialg[SWIGLU ? FN : 1];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      acc[j] = partial[j] = f32x16_t{};
      if constexpr (SWIGLU) accg[j] = partialg[j] = f32x16_t{};
    }
    // block scales of step kt (the wave's columns lie in one 128-row block)
    float sc[FN], scg[SWIGLU ? FN : 1];
    const float* se = slist != nullptr ? slist[e] : Ws + static_cast<size_t>(e) * RB * KT;
    auto sload = [&](int kt) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int rowb = (n0 + wn * TN + j * 32) / kFp8Block;
        sc[j] = se[static_cast<size_t>(rowb) * KT + kt];
        if constexpr (SWIGLU) scg[j] = se[static_cast<size_t>(N / kFp8Block + rowb) * KT + kt];
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
          partial[j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfrag(r, ks, h), partial[j], 0, 0, 0);
          if constexpr (SWIGLU)
            partialg[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfrag(BN + r, ks, h),
                                                                  partialg[j], 0, 0, 0);
        }
      }
      // the step is one scale block: scale its partial sums into the result
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[j] += scc[j] * partial[j];
        partial[j] = f32x16_t{};
        if constexpr (SWIGLU) {
          accg[j] += scgc[j] * partialg[j];
          partialg[j] = f32x16_t{};
        }
      }
      __syncthreads();  // every wave is done with this stage
      sstore();
      __syncthreads();
    }

    // epilogue: D[m][n] of a 32x32 tile sits in lane n + 32 * ((m / 4) % 2),
    // register 4 * (m / 8) + m % 4
    if (live) {
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
}

}  // namespace moe
