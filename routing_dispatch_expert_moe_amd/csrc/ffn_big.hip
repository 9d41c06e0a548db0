// Launchers of the pipelined grouped GEMM (gemm_pipe.h) as stand-alone
// persistent kernels, one per row class.
#include "gemm_pipe.h"
#include "launch.h"

namespace moe {

// 256-row tiles run 8 waves (two per SIMD), the smaller tiles 4
template <int BM>
constexpr int pipe_waves() { return BM == 256 ? 8 : 4; }

template <bool SWIGLU, int BM, int BNW, int STAGES, int CLASS, bool SAVE, int BK>
__global__ __launch_bounds__(pipe_waves<BM>() * 64, 1) void gemm_bf16_pipe(const uint16_t* __restrict__ A,
                                                         const int32_t* __restrict__ offsets,
                                                         int E_loc,
                                                         const uint16_t* __restrict__ W,
                                                         uint16_t* __restrict__ C, int N, int K,
                                                         const uint16_t* const* __restrict__ wlist,
                                                         uint16_t* __restrict__ AB) {
  extern __shared__ uint4 lds[];
  __shared__ int prefix[MOE_MAX_E + 1];
  __shared__ int segs[MOE_MAX_E + 1];
  gemm_pipe_body<SWIGLU, BM, BNW, STAGES, CLASS, pipe_waves<BM>(), SAVE, false, BK>(
      A, offsets, E_loc, W, C, N, K, blockIdx.x, gridDim.x, lds, prefix, segs, nullptr, 1, wlist,
      AB);
}

// FP8 weights with many rows per expert: the bf16 kernels' tiles with the
// weight tiles held in LDS as codes, 64-deep steps (a stage is 48 KB for
// 256-row tiles, three stages; 32 KB for the 128-row remainder tiles, four).
// Every tile runs 8 waves: each MFMA operand is converted from codes first,
// and the second wave on a SIMD keeps its MFMA pipe busy meanwhile.
constexpr int kFp8BK = 64, kFp8Waves = 8;
template <int BM>
constexpr int fp8_stages() { return BM == 256 ? 3 : 4; }

// LIST: codes and scales through per-expert tables (wlist, slist); the packed
// kernels (LIST false) take null tables at compile time, so their code has no
// table lookups at all.
template <bool SWIGLU, int BM, int CLASS, bool LIST>
__global__ __launch_bounds__(kFp8Waves * 64, 1) void gemm_fp8_pipe(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E_loc,
    const uint8_t* __restrict__ Wq, const float* __restrict__ Ws, uint16_t* __restrict__ C,
    int N, int K, const uint16_t* const* __restrict__ wlist,
    const float* const* __restrict__ slist) {
  extern __shared__ uint4 lds[];
  __shared__ int prefix[MOE_MAX_E + 1];
  __shared__ int segs[MOE_MAX_E + 1];
  gemm_pipe_body<SWIGLU, BM, 256, fp8_stages<BM>(), CLASS, kFp8Waves, false, true, kFp8BK>(
      A, offsets, E_loc, reinterpret_cast<const uint16_t*>(Wq), C, N, K, blockIdx.x, gridDim.x,
      lds, prefix, segs, nullptr, 1, LIST ? wlist : nullptr, nullptr, Ws, nullptr, nullptr,
      nullptr, LIST ? slist : nullptr);
}

int fp8_pipe_min_k() {
  constexpr int a = fp8_stages<128>(), b = fp8_stages<256>();
  return (a > b ? a : b) * kFp8BK;
}

namespace {

template <bool SWIGLU, int BM, int CLASS, bool LIST>
int launch_fp8(const void* A, const int32_t* offsets, int E_loc, int64_t max_rows,
               const uint8_t* Wq, const float* Ws, void* C, int N, int K, const void* const* wlist,
               const float* const* slist, hipStream_t s) {
  constexpr size_t lds = pipe_lds_bytes(BM, 256, fp8_stages<BM>(), true, kFp8BK);
  static_assert(lds + 2 * (MOE_MAX_E + 1) * 4 <= 160 * 1024, "LDS budget");
  auto kern = gemm_fp8_pipe<SWIGLU, BM, CLASS, LIST>;
  static LdsAttr attr;
  if (int rc = set_dynamic_lds_once(reinterpret_cast<const void*>(kern), lds, attr)) return rc;
  const int BN = SWIGLU ? 128 : 256;
  const int64_t NT = (N + BN - 1) / BN;
  int64_t tiles_ub = (max_rows / BM + E_loc) * NT;
  if (is_tail_class(CLASS)) tiles_ub = static_cast<int64_t>(E_loc) * ((kTailMax + BM - 1) / BM) * NT;
  int64_t grid = device_cu_count();
  if (grid > tiles_ub) grid = tiles_ub;
  if (grid >= 8) grid &= ~static_cast<int64_t>(7);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kFp8Waves * 64), lds, s,
                     static_cast<const uint16_t*>(A), offsets, E_loc, Wq, Ws,
                     static_cast<uint16_t*>(C), N, K,
                     reinterpret_cast<const uint16_t* const*>(wlist), slist);
  return static_cast<int>(hipGetLastError());
}

template <bool SWIGLU, bool LIST>
int launch_fp8_kind(PipeRows rows, const void* A, const int32_t* offsets, int E_loc,
                    int64_t max_rows, const uint8_t* Wq, const float* Ws, void* C, int N, int K,
                    const void* const* wlist, const float* const* slist, hipStream_t s) {
  switch (rows) {
    case PipeRows::kBigTiles:
      return launch_fp8<SWIGLU, 256, ROWS_BIG, LIST>(A, offsets, E_loc, max_rows, Wq, Ws, C, N, K, wlist, slist, s);
    case PipeRows::kTailTiles:
      return launch_fp8<SWIGLU, 128, ROWS_TAIL, LIST>(A, offsets, E_loc, max_rows, Wq, Ws, C, N, K, wlist, slist, s);
    case PipeRows::kBigRide:
      return launch_fp8<SWIGLU, 256, ROWS_BIGR, LIST>(A, offsets, E_loc, max_rows, Wq, Ws, C, N, K, wlist, slist, s);
    case PipeRows::kTailRide:
      return launch_fp8<SWIGLU, 128, ROWS_TAILR, LIST>(A, offsets, E_loc, max_rows, Wq, Ws, C, N, K, wlist, slist, s);
    default:
      return launch_fp8<SWIGLU, 256, ROWS_ALL, LIST>(A, offsets, E_loc, max_rows, Wq, Ws, C, N, K, wlist, slist, s);
  }
}

}  // namespace

int launch_gemm_pipe_fp8(PipeRows rows, bool swiglu, const void* A, const int32_t* offsets,
                         int E_loc, int64_t max_rows, const uint8_t* Wq, const float* Ws, void* C,
                         int N, int K, const void* const* wlist, const float* const* slist,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool list = wlist != nullptr || slist != nullptr;
  if (swiglu)
    return list ? launch_fp8_kind<true, true>(rows, A, offsets, E_loc, max_rows, Wq, Ws, C, N, K,
                                              wlist, slist, s)
                : launch_fp8_kind<true, false>(rows, A, offsets, E_loc, max_rows, Wq, Ws, C, N, K,
                                               wlist, slist, s);
  return list ? launch_fp8_kind<false, true>(rows, A, offsets, E_loc, max_rows, Wq, Ws, C, N, K,
                                             wlist, slist, s)
              : launch_fp8_kind<false, false>(rows, A, offsets, E_loc, max_rows, Wq, Ws, C, N, K,
                                              wlist, slist, s);
}

namespace {

// bf16 tiles step K 64 deep (whole 128-byte lines per row and load; K is a
// multiple of 64 for bf16): 256 x 256 tiles in two 64 KB stages, 128 x 256
// in three of 48 KB, 128 x 128 in four of 32 KB
constexpr int kPipeBK = 64;

template <bool SWIGLU, int BM, int BNW, int STAGES, int CLASS, bool SAVE>
int launch_pipe(const void* A, const int32_t* offsets, int E_loc, int64_t max_rows, const void* W,
                void* C, int N, int K, const void* const* wlist, void* AB, hipStream_t s) {
  constexpr int BK = kPipeBK;
  const size_t lds = pipe_lds_bytes(BM, BNW, STAGES, false, BK);
  static_assert(pipe_lds_bytes(BM, BNW, STAGES, false, BK) + 2 * (MOE_MAX_E + 1) * 4 <= 160 * 1024,
                "LDS budget");
  if (K % BK != 0) return static_cast<int>(hipErrorInvalidValue);
  auto kern = gemm_bf16_pipe<SWIGLU, BM, BNW, STAGES, CLASS, SAVE, BK>;
  static LdsAttr attr;
  if (int rc = set_dynamic_lds_once(reinterpret_cast<const void*>(kern), lds, attr)) return rc;
  const int BN = SWIGLU ? BNW / 2 : BNW;
  const int64_t NT = (N + BN - 1) / BN;
  int64_t tiles_ub = (max_rows / BM + E_loc) * NT;
  if (is_tail_class(CLASS)) tiles_ub = static_cast<int64_t>(E_loc) * ((kTailMax + BM - 1) / BM) * NT;
  int64_t grid = device_cu_count();
  if (grid > tiles_ub) grid = tiles_ub;
  if (grid >= 8) grid &= ~static_cast<int64_t>(7);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(pipe_waves<BM>() * 64), lds, s,
                     static_cast<const uint16_t*>(A), offsets, E_loc,
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(C), N, K,
                     reinterpret_cast<const uint16_t* const*>(wlist), static_cast<uint16_t*>(AB));
  return static_cast<int>(hipGetLastError());
}

// The few-row tiles are 128 activation rows by 128 weight rows with 4 stages
// when the remainders would give few tiles (twice as many tiles as with 256
// weight rows keeps every CU busy when only a few experts have remainders),
// else 128 x 256 with 3 stages (half the re-reads of the activation rows).
constexpr int kSmallBM = 128, kSmallBNW = 128, kSmallStages = 4;
constexpr int kBigStages = 2, kWideStages = 3;

template <bool SWIGLU, bool SAVE>
int launch_kind(PipeRows rows, const void* A, const int32_t* offsets, int E_loc, int64_t max_rows,
                const void* W, void* C, int N, int K, const void* const* wlist, void* AB,
                hipStream_t s) {
  switch (rows) {
    case PipeRows::kBigTiles:
      return launch_pipe<SWIGLU, 256, 256, kBigStages, ROWS_BIG, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kBigRide:
      return launch_pipe<SWIGLU, 256, 256, kBigStages, ROWS_BIGR, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kTailRide:
      return launch_pipe<SWIGLU, 128, 256, kWideStages, ROWS_TAILR, SAVE>(A, offsets, E_loc, max_rows, W, C, N,
                                                                 K, wlist, AB, s);
    case PipeRows::kAllRowsWide:
      return launch_pipe<SWIGLU, 128, 256, kWideStages, ROWS_ALL, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kBigAll:
      return launch_pipe<SWIGLU, 256, 256, kBigStages, ROWS_ALL, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kTailTiles: {
      if (!few_gemm_tiles(E_loc, N, SWIGLU, device_cu_count()))
        return launch_pipe<SWIGLU, 128, 256, kWideStages, ROWS_TAIL, SAVE>(A, offsets, E_loc, max_rows, W, C,
                                                                  N, K, wlist, AB, s);
      return launch_pipe<SWIGLU, kSmallBM, kSmallBNW, kSmallStages, ROWS_TAIL, SAVE>(
          A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    }
    default:
      return launch_pipe<SWIGLU, kSmallBM, kSmallBNW, kSmallStages, ROWS_ALL, SAVE>(
          A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
  }
}

}  // namespace

int launch_gemm_pipe_bf16(PipeRows rows, bool swiglu, const void* A, const int32_t* offsets,
                          int E_loc, int64_t max_rows, const void* W, void* C, int N, int K,
                          const void* const* wlist, void* stream, void* ab) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (swiglu && ab != nullptr)
    return launch_kind<true, true>(rows, A, offsets, E_loc, max_rows, W, C, N, K, wlist, ab, s);
  if (swiglu)
    return launch_kind<true, false>(rows, A, offsets, E_loc, max_rows, W, C, N, K, wlist, nullptr, s);
  return launch_kind<false, false>(rows, A, offsets, E_loc, max_rows, W, C, N, K, wlist, nullptr, s);
}

}  // namespace moe
