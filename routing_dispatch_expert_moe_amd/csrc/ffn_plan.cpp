// Which grouped-GEMM kernels one bf16 FFN half runs, decided on the host from
// the sizes alone (row counts stay on the device).  Shared by the launchers
// and by moe_ffn_plan, which reports the choice without a GPU.
//
// DWDP page, key optimisations (one grouped GEMM over all local experts) and
// its per-expert load imbalance: few rows per expert stream weights, many
// rows are MFMA work, and a skewed pass has both.
#include "launch.h"
#include "moe.h"

namespace moe {

bool few_gemm_tiles(int E_loc, int N, bool swiglu, int cu) {
  const int64_t tiles256 = static_cast<int64_t>(E_loc) * ((N + (swiglu ? 127 : 255)) /
                                                          (swiglu ? 128 : 256));
  return tiles256 < 4 * static_cast<int64_t>(cu);
}

bool remainders_with_big_tiles(int E_loc, int N, int K, bool swiglu, int cu) {
  // with few tiles the remainder tiles would re-stream whole weight matrices,
  // so they ride along with the expert's 256-row tiles; but a pass with long
  // tiles (large K) pays a whole extra round for a few of them
  return few_gemm_tiles(E_loc, N, swiglu, cu) && K <= 4096;
}

bool ffn_operands_fit32(bool up, int64_t max_rows, int d, int f) {
  // the pipelined kernels address the activations (max_rows x K), one
  // expert's weights and the output (max_rows x N) with 32-bit byte offsets
  const double rows = static_cast<double>(max_rows) * (d > f ? d : f) * 2;
  const double wts = static_cast<double>(up ? 2 : 1) * f * d * 2;
  return rows < 4294967296.0 && wts < 4294967296.0;
}

int ffn_plan_bf16(bool up, int64_t max_rows, int E_loc, int d, int f, int cu) {
  const int64_t avg = max_rows / E_loc;
  if (!ffn_operands_fit32(up, max_rows, d, f)) return MOE_FFN_PLAN_STREAM_WIDE_OPERANDS;
  if (avg <= kStreamRows) return MOE_FFN_PLAN_STREAM;
  const int N = up ? f : d, K = up ? d : f;
  if (up && few_gemm_tiles(E_loc, N, true, cu) && avg <= kWideRows) return MOE_FFN_PLAN_WIDE;
  if (remainders_with_big_tiles(E_loc, N, K, up, cu)) return MOE_FFN_PLAN_BIG_ALL;
  if (!few_gemm_tiles(E_loc, N, up, cu)) return MOE_FFN_PLAN_BIG_RIDE;
  return MOE_FFN_PLAN_BIG_TAIL;
}

}  // namespace moe

extern "C" int moe_ffn_plan(int half, int64_t max_rows, int E_loc, int d, int f, int dtype,
                            int cu_count) {
  if ((half != 0 && half != 1) || max_rows < 0 || E_loc < 1 || E_loc > MOE_MAX_E || d < 1 ||
      f < 1 || cu_count < 1 || (dtype != MOE_F32 && dtype != MOE_BF16))
    return -1;
  if (max_rows == 0) return MOE_FFN_PLAN_NONE;
  if (dtype == MOE_F32) return MOE_FFN_PLAN_F32;
  return moe::ffn_plan_bf16(half == 0, max_rows, E_loc, d, f, cu_count);
}
