// Launchers of the pipelined grouped GEMM (gemm_pipe.h) as stand-alone
// persistent kernels, one per row class.
#include "gemm_pipe.h"
#include "launch.h"

namespace moe {

// 256-row tiles run 8 waves (two per SIMD), the smaller tiles 4
template <int BM>
constexpr int pipe_waves() { return BM == 256 ? 8 : 4; }

template <bool SWIGLU, int BM, int BNW, int STAGES, int CLASS, bool SAVE>
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
  gemm_pipe_body<SWIGLU, BM, BNW, STAGES, CLASS, pipe_waves<BM>(), SAVE>(
      A, offsets, E_loc, W, C, N, K, blockIdx.x, gridDim.x, lds, prefix, segs, nullptr, 1, wlist,
      AB);
}

namespace {

template <bool SWIGLU, int BM, int BNW, int STAGES, int CLASS, bool SAVE>
int launch_pipe(const void* A, const int32_t* offsets, int E_loc, int64_t max_rows, const void* W,
                void* C, int N, int K, const void* const* wlist, void* AB, hipStream_t s) {
  const size_t lds = pipe_lds_bytes(BM, BNW, STAGES);
  static_assert(pipe_lds_bytes(BM, BNW, STAGES) + 2 * (MOE_MAX_E + 1) * 4 <= 160 * 1024,
                "LDS budget");
  auto kern = gemm_bf16_pipe<SWIGLU, BM, BNW, STAGES, CLASS, SAVE>;
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

// The few-row tiles are 128 activation rows by 128 weight rows with 8 stages
// when the remainders would give few tiles (twice as many tiles as with 256
// weight rows keeps every CU busy when only a few experts have remainders),
// else 128 x 256 with 6 stages (half the re-reads of the activation rows).
constexpr int kSmallBM = 128, kSmallBNW = 128, kSmallStages = 8;

template <bool SWIGLU, bool SAVE>
int launch_kind(PipeRows rows, const void* A, const int32_t* offsets, int E_loc, int64_t max_rows,
                const void* W, void* C, int N, int K, const void* const* wlist, void* AB,
                hipStream_t s) {
  switch (rows) {
    case PipeRows::kBigTiles:
      return launch_pipe<SWIGLU, 256, 256, 4, ROWS_BIG, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kBigRide:
      return launch_pipe<SWIGLU, 256, 256, 4, ROWS_BIGR, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kTailRide:
      return launch_pipe<SWIGLU, 128, 256, 6, ROWS_TAILR, SAVE>(A, offsets, E_loc, max_rows, W, C, N,
                                                                 K, wlist, AB, s);
    case PipeRows::kAllRowsWide:
      return launch_pipe<SWIGLU, 128, 256, 6, ROWS_ALL, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kBigAll:
      return launch_pipe<SWIGLU, 256, 256, 4, ROWS_ALL, SAVE>(A, offsets, E_loc, max_rows, W, C, N, K, wlist, AB, s);
    case PipeRows::kTailTiles: {
      if (!few_gemm_tiles(E_loc, N, SWIGLU))
        return launch_pipe<SWIGLU, 128, 256, 6, ROWS_TAIL, SAVE>(A, offsets, E_loc, max_rows, W, C,
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

bool few_gemm_tiles(int E_loc, int N, bool swiglu) {
  const int64_t tiles256 = static_cast<int64_t>(E_loc) * ((N + (swiglu ? 127 : 255)) /
                                                          (swiglu ? 128 : 256));
  return tiles256 < 4 * static_cast<int64_t>(device_cu_count());
}

bool remainders_with_big_tiles(int E_loc, int N, int K, bool swiglu) {
  // with few tiles the remainder tiles would re-stream whole weight matrices,
  // so they ride along with the expert's 256-row tiles; but a pass with long
  // tiles (large K) pays a whole extra round for a few of them
  return few_gemm_tiles(E_loc, N, swiglu) && K <= 4096;
}

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
