// Grouped expert GEMMs in bf16 on gfx950 MFMA (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation.
//
// DWDP page, key optimisations: the first grouped GEMM runs every local
// expert's rows against that expert's fused [W1 | W3] operand with SwiGLU in
// the epilogue; the second grouped GEMM applies W2.  MegaMoE comparison page,
// core differences §1: two linear layers with SwiGLU between them.
//
//   up   : h[r, n] = silu(sum_k A[r,k] W1t[n,k]) * (sum_k A[r,k] W3t[n,k])
//   down : y[r, n] = sum_k h[r,k] W2t[n,k]
//
// Weights are packed K-contiguous ("NT" GEMM), so both MFMA operands are
// 16-byte runs along K in LDS.  Rows of each expert are the segment
// [offsets[e], offsets[e+1]) of the expert-major activations; segment sizes
// live only on the device.
//
// Scheduling (persistent per-expert tile scheduler): a fixed grid of
// workgroups walks a linear tile space.  Each workgroup first scans the
// expert segment sizes into an LDS prefix of M-tiles, then maps a tile id to
// (expert, n-tile, m-tile) with m fastest, so consecutive tiles reuse one
// weight tile.  Workgroup ids are remapped so that each XCD (ids are dealt
// round-robin over the 8 XCDs) owns contiguous tile ranges and the tiles that
// share a weight tile meet in the same L2.
#include "common.h"
#include "fp8_dev.h"
#include "launch.h"
#include "tile_sched.h"

namespace moe {

__device__ __forceinline__ float silu_f(float a) { return a * __builtin_amdgcn_rcpf(1.f + __expf(-a)); }

// 16 / 8 bytes through a global-address-space pointer (a global load)
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_g __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload16(const __attribute__((address_space(1))) void* p) {
  const u32x4_g v = *static_cast<const __attribute__((address_space(1))) u32x4_g*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 gload8(const __attribute__((address_space(1))) void* p) {
  const u32x2_g v = *static_cast<const __attribute__((address_space(1))) u32x2_g*>(p);
  return make_uint2(v.x, v.y);
}

// FP8W: the weights are E4M3 codes (one byte each) with one fp32 scale per
// 128 x 128 block of the packed matrix (Ws: [E][rows / 128][K / 128]) (NCCL
// EP page §2.1: FP8 expert compute with a scale tensor).  Codes become bf16
// exactly (every E4M3 value is a bf16 value) as the weight tile is staged
// into LDS; the MFMAs accumulate each 128-deep K block into a partial sum,
// which is multiplied by its block's scale and added to the result, so the
// scale costs one fp32 FMA per output element and K block.  A 32 x 32 MFMA
// tile's columns lie in one 128-row block, so its scale is uniform.
template <int BM, int BN, int BK, int WM, int WN, bool SWIGLU, int CLASS, bool FP8W = false>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E_loc,
    const void* __restrict__ Wv, const float* __restrict__ Ws, uint16_t* __restrict__ C, int N,
    int K, const void* const* __restrict__ wlist, const float* const* __restrict__ slist) {
  constexpr int NTHR = WM * WN * 64;
  constexpr int BNW = SWIGLU ? 2 * BN : BN;  // weight rows per tile
  constexpr int KC = BK / 8;                 // 16-byte chunks per tile row
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
  constexpr int CA = BM * KC / NTHR;         // A chunks per thread per stage
  constexpr int CB = BNW * KC / NTHR;        // B chunks per thread per stage
  static_assert(BM * KC % NTHR == 0 && BNW * KC % NTHR == 0, "tile / thread mismatch");
  static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 16 == 0, "MFMA tiling");
  static_assert(!FP8W || kFp8Block % BK == 0, "a K-step stays inside one scale block");

  extern __shared__ uint4 lds[];
  uint4* As = lds;                      // [2][BM * KC]
  uint4* Bs = lds + 2 * BM * KC;        // [2][BNW * KC]
  __shared__ int prefix[MOE_MAX_E + 1];

  mtile_prefix<BM, CLASS>(offsets, E_loc, prefix);
  const int NT = (N + BN - 1) / BN;
  const int total = prefix[E_loc] * NT;
  const int G = gridDim.x;
  // XCD-aware remap of the workgroup id (ids are dealt round-robin over 8 XCDs)
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int KT = K / BK;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;
  const uint16_t* W = static_cast<const uint16_t*>(Wv);
  const uint8_t* Wq = static_cast<const uint8_t*>(Wv);
  const int KB = K / kFp8Block;                               // scale blocks along K
  const int RB = (SWIGLU ? 2 * N : N) / kFp8Block;            // scale blocks along the rows

  for (int tile = vb; tile < total; tile += G) {
    const int mt = tile / NT;  // global M-tile index ... expert from prefix
    const int e = find_expert(prefix, E_loc, mt);
    const int mt_e = prefix[e + 1] - prefix[e];
    const int local = tile - prefix[e] * NT;
    const int nt = local / mt_e;
    const int mti = local % mt_e;
    int first, count;
    class_rows<CLASS>(offsets[e + 1] - offsets[e], first, count);
    const int seg0 = offsets[e] + first, seg1 = seg0 + count;
    const int m0 = seg0 + mti * BM;
    const int n0 = nt * BN;
    // expert e's packed weights: W + e * stride, or wlist[e] (a table of
    // per-expert buffers).  A pointer read from the table is generic; marked
    // global, the weight loads stay global loads (a flat load also counts on
    // the LDS counter, so every LDS wait before an MFMA would wait for HBM)
    using gu16 = const __attribute__((address_space(1))) uint16_t;
    using gu8 = const __attribute__((address_space(1))) uint8_t;
    gu16* We = (gu16*)(wlist != nullptr ? static_cast<const uint16_t*>(wlist[e]) : W + e * wstride);
    gu8* Wqe = (gu8*)(wlist != nullptr ? static_cast<const uint8_t*>(wlist[e]) : Wq + e * wstride);

    // per-thread load descriptors
    const uint16_t* a_src[CA];
    bool a_ok[CA];
    int a_dst[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NTHR;
      const int r = c / KC, kc = c % KC;
      const int row = m0 + r;
      a_ok[i] = row < seg1;
      a_src[i] = A + static_cast<size_t>(a_ok[i] ? row : seg0) * K + kc * 8;
      a_dst[i] = r * KC + (kc ^ ((r >> 1) & (KC - 1)));
    }
    gu16* b_src[CB];
    gu8* bq_src[CB];
    bool b_ok[CB];
    int b_dst[CB];
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NTHR;
      const int r = c / KC, kc = c % KC;
      const int half = SWIGLU ? (r / BN) : 0;
      const int n = n0 + (r % BN);
      b_ok[i] = n < N;
      const size_t wrow = static_cast<size_t>(half) * N + (b_ok[i] ? n : 0);
      b_src[i] = We + wrow * K + kc * 8;
      bq_src[i] = Wqe + wrow * K + kc * 8;
      b_dst[i] = r * KC + (kc ^ ((r >> 1) & (KC - 1)));
    }

    f32x16_t acc[FM][FN];
    f32x16_t accg[SWIGLU ? FM : 1][SWIGLU ? FN : 1];
    // FP8W: partial sums of the current 128-deep K block (before its scale)
    f32x16_t part[FP8W ? FM : 1][FP8W ? FN : 1];
    f32x16_t partg[FP8W && SWIGLU ? FM : 1][FP8W && SWIGLU ? FN : 1];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = f32x16_t{};
        if constexpr (SWIGLU) accg[i][j] = f32x16_t{};
        if constexpr (FP8W) part[i][j] = f32x16_t{};
        if constexpr (FP8W && SWIGLU) partg[i][j] = f32x16_t{};
      }

    const bool wave_active = m0 + wm * TM < seg1;
    uint4 ra[CA], rb[CB];
    uint2 rq0[FP8W ? CB : 1];  // FP8W: the codes of the next K-step
    // Loads are unconditional (rows past the segment or the matrix read a
    // valid row instead) and the unused values are zeroed afterwards: no
    // branch separates the loads, so the waits for one K-step's data leave
    // the next step's loads in flight.
    auto sel4 = [](bool ok, uint4 v) {
      return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
    };
    auto gload_a = [&](int kt) {
      const int koff = kt * BK;
#pragma unroll
      for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + koff);
    };
    auto gload_b = [&](int kt) {
      const int koff = kt * BK;
#pragma unroll
      for (int i = 0; i < CB; ++i) rb[i] = gload16(b_src[i] + koff);
    };
    auto gload_q = [&](int kt, uint2 (&rq)[FP8W ? CB : 1]) {
      const int koff = kt * BK;
#pragma unroll
      for (int i = 0; i < CB; ++i)  // 8 codes (8 bytes) per chunk
        rq[i] = gload8(bq_src[i] + koff);
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < CA; ++i) As[buf * BM * KC + a_dst[i]] = sel4(a_ok[i], ra[i]);
#pragma unroll
      for (int i = 0; i < CB; ++i) Bs[buf * BNW * KC + b_dst[i]] = sel4(b_ok[i], rb[i]);
    };
    // E4M3 -> bf16 into the staging registers, two codes per conversion
    // (exact; unit scale)
    auto convert = [&](const uint2 (&rq)[FP8W ? CB : 1]) {
#pragma unroll
      for (int i = 0; i < (FP8W ? CB : 0); ++i) {
        const int x = static_cast<int>(rq[i].x), y = static_cast<int>(rq[i].y);
        rb[i] = make_uint4(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, true)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.f, true)));
      }
    };

    // the MFMAs of K-step kt from LDS buffer kt & 1 (FP8W: into the block's
    // partial sums, scaled into the result at the end of each 128-deep block)
    auto compute = [&](int kt) {
      const int buf = kt & 1;
      const uint4* Ab = As + buf * BM * KC;
      const uint4* Bb = Bs + buf * BNW * KC;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        // a wave whose rows all lie past the segment has nothing to compute
        if (!wave_active) break;
        const int ch = ks * 2 + (lane >> 5);
        bf16x8_t af[FM], bf[FN], gf[SWIGLU ? FN : 1];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * TM + i * 32 + (lane & 31);
          af[i] = __builtin_bit_cast(bf16x8_t, Ab[r * KC + (ch ^ ((r >> 1) & (KC - 1)))]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * TN + j * 32 + (lane & 31);
          bf[j] = __builtin_bit_cast(bf16x8_t, Bb[r * KC + (ch ^ ((r >> 1) & (KC - 1)))]);
          if constexpr (SWIGLU) {
            const int r2 = BN + r;
            gf[j] = __builtin_bit_cast(bf16x8_t, Bb[r2 * KC + (ch ^ ((r2 >> 1) & (KC - 1)))]);
          }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if constexpr (FP8W) {
              part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], part[i][j], 0, 0, 0);
              if constexpr (SWIGLU)
                partg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], gf[j], partg[i][j], 0, 0, 0);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
              if constexpr (SWIGLU)
                accg[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], gf[j], accg[i][j], 0, 0, 0);
            }
          }
      }
      if constexpr (FP8W) {
        if (wave_active && ((kt + 1) * BK) % kFp8Block == 0) {
          const int kb = (kt * BK) / kFp8Block;
          const float* se = slist != nullptr ? slist[e] : Ws + static_cast<size_t>(e) * RB * KB;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int rowb = (n0 + wn * TN + j * 32) / kFp8Block;  // W1 (or W2) block row
            const float sc = se[static_cast<size_t>(rowb) * KB + kb];
            float scg = 0.f;
            if constexpr (SWIGLU) scg = se[static_cast<size_t>(N / kFp8Block + rowb) * KB + kb];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
              acc[i][j] += sc * part[i][j];
              part[i][j] = f32x16_t{};
              if constexpr (SWIGLU) {
                accg[i][j] += scg * partg[i][j];
                partg[i][j] = f32x16_t{};
              }
            }
          }
        }
      }
    };

    if constexpr (FP8W) {
      gload_a(0);
      gload_q(0, rq0);
      convert(rq0);
      sstore(0);
      __syncthreads();
      // branch-free steps: the last one re-fetches step KT - 1 (valid, unused)
      // and stages it into the buffer no later step reads
      for (int kt = 0; kt < KT; ++kt) {
        gload_a(min(kt + 1, KT - 1));
        gload_q(min(kt + 1, KT - 1), rq0);
        compute(kt);
        convert(rq0);
        sstore((kt + 1) & 1);
        __syncthreads();
      }
    } else {
      gload_a(0);
      gload_b(0);
      sstore(0);
      __syncthreads();
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) {
          gload_a(kt + 1);
          gload_b(kt + 1);
        }
        compute(kt);
        if (kt + 1 < KT) sstore((kt + 1) & 1);
        __syncthreads();
      }
    }

    // epilogue: D[m][n] of a 32x32 tile sits in lane (n + 32 * ((m / 4) % 2)),
    // register 4 * (m / 8) + m % 4
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int row = m0 + wm * TM + i * 32 + m;
          float v = acc[i][j][r];
          if constexpr (SWIGLU) v = silu_f(v) * accg[i][j][r];
          if (row < seg1 && col < N) C[static_cast<size_t>(row) * N + col] = f32_to_bf16(v);
        }
      }
  }
}

template <int BM, int BN, int BK, int WM, int WN, bool SWIGLU, int CLASS, bool FP8W = false>
static int launch_gemm(const void* A, const int32_t* offsets, int E_loc, int64_t max_rows,
                       const void* W, void* C, int N, int K, hipStream_t s,
                       const float* Ws = nullptr, const void* const* wlist = nullptr,
                       const float* const* slist = nullptr) {
  constexpr int BNW = SWIGLU ? 2 * BN : BN;
  const size_t lds = static_cast<size_t>(2) * (BM + BNW) * BK * sizeof(uint16_t);
  auto kern = gemm_bf16_kernel<BM, BN, BK, WM, WN, SWIGLU, CLASS, FP8W>;
  static LdsAttr attr;
  if (int rc = set_dynamic_lds_once(reinterpret_cast<const void*>(kern), lds, attr)) return rc;
  const int64_t NT = (N + BN - 1) / BN;
  int64_t tiles_ub = (max_rows / BM + E_loc) * NT;
  if (is_tail_class(CLASS)) tiles_ub = static_cast<int64_t>(E_loc) * ((kTailMax + BM - 1) / BM) * NT;
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern),
                                                             WM * WN * 64, lds);
  if (e != hipSuccess) return static_cast<int>(e);
  if (occ < 1) occ = 1;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * occ;
  if (grid > tiles_ub) grid = tiles_ub;
  if (grid >= 8) grid &= ~static_cast<int64_t>(7);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(WM * WN * 64), lds, s,
                     static_cast<const uint16_t*>(A), offsets, E_loc, W, Ws,
                     static_cast<uint16_t*>(C), N, K, wlist, slist);
  return static_cast<int>(hipGetLastError());
}


// The kernels of each pass come from ffn_plan_bf16 (ffn_plan.cpp), which
// decides from the sizes on the host: with few rows per expert (or an
// operand of 4 GiB or more) one register-staged 32-row-tile kernel streams
// the weights over every row; a first-half pass with few tiles and few rows
// per expert runs 128-row tiles of 256 weight rows over every row (five
// stages of weight bytes in flight per CU where the 256-row tiles keep
// three); a pass with few, short tiles runs every row in 256-row tiles (an
// expert's last block shares its weight tiles with the expert's other tiles
// through L2); long-K passes with few tiles run 256-row tiles over the full
// blocks and 128-row tiles over the short remainders; passes with many tiles
// keep an expert's short last block in the 256-row tiles whenever the expert
// has a full block, and give the experts below 128 rows to the 128-row tiles,
// so no expert's weights are streamed by both kernels.  Row counts stay on
// the device.
int launch_ffn_up_bf16(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                       int d, int f, const void* w13, void* h, const void* const* wlist,
                       void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_rows == 0) return 0;
  auto pipe = [&](PipeRows r) {
    return launch_gemm_pipe_bf16(r, true, x_perm, offsets, E_loc, max_rows, w13, h, f, d, wlist, stream);
  };
  switch (ffn_plan_bf16(true, max_rows, E_loc, d, f, device_cu_count())) {
    case MOE_FFN_PLAN_STREAM:
    case MOE_FFN_PLAN_STREAM_WIDE_OPERANDS:
      return launch_gemm<32, 128, 64, 1, 4, true, ROWS_ALL>(x_perm, offsets, E_loc, max_rows, w13, h, f, d, s, nullptr, wlist);
    case MOE_FFN_PLAN_WIDE:
      return pipe(PipeRows::kAllRowsWide);
    case MOE_FFN_PLAN_BIG_ALL:
      return pipe(PipeRows::kBigAll);
    case MOE_FFN_PLAN_BIG_RIDE: {
      int e = pipe(PipeRows::kBigRide);
      return e != 0 ? e : pipe(PipeRows::kTailRide);
    }
    default: {
      int e = pipe(PipeRows::kBigTiles);
      return e != 0 ? e : pipe(PipeRows::kTailTiles);
    }
  }
}

// Always the pipelined kernels (the only ones with the pre-activation store);
// the caller checks that every operand is below 4 GiB.
int launch_ffn_up_train_bf16(const void* x_perm, const int32_t* offsets, int E_loc,
                             int64_t max_rows, int d, int f, const void* w13, void* h, void* ab,
                             void* stream) {
  if (max_rows == 0) return 0;
  auto pipe = [&](PipeRows r) {
    return launch_gemm_pipe_bf16(r, true, x_perm, offsets, E_loc, max_rows, w13, h, f, d, nullptr, stream, ab);
  };
  switch (ffn_plan_bf16(true, max_rows, E_loc, d, f, device_cu_count())) {
    case MOE_FFN_PLAN_STREAM:
    case MOE_FFN_PLAN_STREAM_WIDE_OPERANDS:
      return pipe(PipeRows::kAllRows);
    case MOE_FFN_PLAN_WIDE:
      return pipe(PipeRows::kAllRowsWide);
    case MOE_FFN_PLAN_BIG_ALL:
      return pipe(PipeRows::kBigAll);
    case MOE_FFN_PLAN_BIG_RIDE: {
      int e = pipe(PipeRows::kBigRide);
      return e != 0 ? e : pipe(PipeRows::kTailRide);
    }
    default: {
      int e = pipe(PipeRows::kBigTiles);
      return e != 0 ? e : pipe(PipeRows::kTailTiles);
    }
  }
}

int launch_ffn_down_bf16(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                         int d, int f, const void* w2, void* y, const void* const* wlist,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_rows == 0) return 0;
  auto pipe = [&](PipeRows r) {
    return launch_gemm_pipe_bf16(r, false, h, offsets, E_loc, max_rows, w2, y, d, f, wlist, stream);
  };
  switch (ffn_plan_bf16(false, max_rows, E_loc, d, f, device_cu_count())) {
    case MOE_FFN_PLAN_STREAM:
    case MOE_FFN_PLAN_STREAM_WIDE_OPERANDS:
      return launch_gemm<32, 128, 64, 1, 4, false, ROWS_ALL>(h, offsets, E_loc, max_rows, w2, y, d, f, s, nullptr, wlist);
    case MOE_FFN_PLAN_BIG_ALL:
      return pipe(PipeRows::kBigAll);
    case MOE_FFN_PLAN_BIG_RIDE: {
      int e = pipe(PipeRows::kBigRide);
      return e != 0 ? e : pipe(PipeRows::kTailRide);
    }
    default: {
      int e = pipe(PipeRows::kBigTiles);
      return e != 0 ? e : pipe(PipeRows::kTailTiles);
    }
  }
}

}  // namespace moe

namespace moe {

// FP8 weights: few rows per expert (decode) run the code-streaming kernel
// (fp8.hip: codes in LDS, 32-row tiles, three workgroups per CU); more rows
// run the pipelined kernels with the bf16 pass's tiles and row classes (codes
// in LDS; see fp8_pipe_pass), or, for K below their pipeline depth, register-staged 64-row
// tiles that convert codes to bf16 as they stage them.  Row counts stay on
// the device.
static int fp8_pipe_pass(bool up, const void* A, const int32_t* offsets, int E_loc,
                         int64_t max_rows, int d, int f, const uint8_t* wq, const float* ws,
                         void* C, const void* const* wlist, const float* const* slist,
                         void* stream) {
  const int N = up ? f : d, K = up ? d : f;
  auto run = [&](PipeRows r) {
    return launch_gemm_pipe_fp8(r, up, A, offsets, E_loc, max_rows, wq, ws, C, N, K, wlist, slist,
                                stream);
  };
  // the bf16 pass's row classes: 256-row tiles then 128-row remainder tiles
  // (long-K passes with few tiles), the ride-along split (many tiles: the
  // experts below 128 rows stream their codes through 128-row tiles), else
  // every row in 256-row tiles (the few-tile first half too)
  switch (ffn_plan_bf16(up, max_rows, E_loc, d, f, device_cu_count())) {
    case MOE_FFN_PLAN_BIG_TAIL: {
      const int e = run(PipeRows::kBigTiles);
      return e != 0 ? e : run(PipeRows::kTailTiles);
    }
    case MOE_FFN_PLAN_BIG_RIDE: {
      const int e = run(PipeRows::kBigRide);
      return e != 0 ? e : run(PipeRows::kTailRide);
    }
    default:
      return run(PipeRows::kBigAll);
  }
}
int launch_ffn_up_fp8(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, const uint8_t* w13q, const float* w13s, void* h,
                      void* stream, const void* const* wlist, const float* const* slist) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_rows == 0) return 0;
  if (max_rows / E_loc <= kStreamRows)
    return launch_gemm_fp8w(true, x_perm, offsets, E_loc, max_rows, w13q, w13s, h, f, d, stream,
                            wlist, slist);
  if (d >= fp8_pipe_min_k() && ffn_operands_fit32(true, max_rows, d, f))
    return fp8_pipe_pass(true, x_perm, offsets, E_loc, max_rows, d, f, w13q, w13s, h, wlist,
                         slist, stream);
  return launch_gemm<64, 128, 64, 2, 2, true, ROWS_ALL, true>(x_perm, offsets, E_loc, max_rows,
                                                              w13q, h, f, d, s, w13s, wlist, slist);
}

int launch_ffn_down_fp8(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, const uint8_t* w2q, const float* w2s, void* y,
                        void* stream, const void* const* wlist, const float* const* slist) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_rows == 0) return 0;
  if (max_rows / E_loc <= kStreamRows)
    return launch_gemm_fp8w(false, h, offsets, E_loc, max_rows, w2q, w2s, y, d, f, stream, wlist,
                            slist);
  if (f >= fp8_pipe_min_k() && ffn_operands_fit32(false, max_rows, d, f))
    return fp8_pipe_pass(false, h, offsets, E_loc, max_rows, d, f, w2q, w2s, y, wlist, slist,
                         stream);
  return launch_gemm<64, 128, 64, 2, 2, false, ROWS_ALL, true>(h, offsets, E_loc, max_rows, w2q,
                                                               y, d, f, s, w2s, wlist, slist);
}

}  // namespace moe
