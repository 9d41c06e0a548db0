// Internal launchers (C++ linkage, not exported).  Each returns a hipError_t
// as int (0 = success).  Arguments are already validated by the C ABI layer.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

// device error word lives at the start of the workspace
constexpr size_t kWsHeader = 2048;
constexpr int kDispatchTokensPerBlock = 256;

struct DispatchWs {
  int* err;           // [1]
  int* block_counts;  // [nb * E]
  int* block_base;    // [nb * E]
};

size_t dispatch_ws_bytes(int T, int E);
DispatchWs dispatch_ws(void* ws, int T, int E);

int launch_router_logits(const void* x, const float* wg, int T, int d, int E, float* logits,
                         void* stream);
int launch_route(const float* logits, int T, int E, int k, int gate, int32_t* idx, float* w,
                 void* stream);
// routing with overflow rerouting; cand_e / cand_v: [T][k+1] scratch,
// rerouted: ceil(T / 64) scratch masks
int launch_route_reroute(const float* logits, int T, int E, int k, int gate, int capacity,
                         int32_t* idx, float* w, int32_t* cand_e, float* cand_v,
                         uint64_t* rerouted, void* stream);
// workspace bytes of the rerouting candidates, placed after the dispatch scratch
size_t reroute_ws_bytes(int T, int k);
// this device's address of the library's fixed scratch array
// (MOE_NOALLOC_SCRATCH_BYTES, route.hip), looked up once per device
int noalloc_scratch(void** ptr);
int launch_dispatch(const int32_t* idx, int T, int E, int k, int capacity, int e_begin,
                    int e_end, const void* x, int d, int elem_bytes, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, int32_t* n_kept,
                    void* x_perm, const DispatchWs& ws, void* stream);
// wlist (all FFN launchers): null for one packed weight tensor (expert e at
// W + e * rows * K), else a device table of E_loc per-expert packed buffers
int launch_ffn_up_bf16(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                       int d, int f, const void* w13, void* h, const void* const* wlist,
                       void* stream);
int launch_ffn_down_bf16(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                         int d, int f, const void* w2, void* y, const void* const* wlist,
                         void* stream);
// Pipelined direct-to-LDS grouped GEMM over one row class: 256-row tiles over
// each expert's full blocks (kBigTiles), 256-row tiles over every row with
// the last block of an expert as a possibly half-empty tile (kBigAll),
// smaller tiles over the short remainders (kTailTiles), or smaller tiles over
// every row (kAllRows); kBigRide / kTailRide: 256-row tiles over every row of
// the experts with at least one full block, smaller tiles over the experts
// with fewer than 128 rows (passes with many tiles); kAllRowsWide: 128-row
// tiles of 256 weight rows (six stages) over every row.
// How the fused layer's bf16 GEMM phases split each expert's rows, chosen by
// the same rules as the separate FFN calls: 256-row tiles then 128-row tiles
// for the remainders; the ride-along split (ROWS_BIGR / ROWS_TAILR); every
// row in 256-row tiles; every row in 128-row tiles of 256 weight rows.
enum FusedRows { kFusedBigTail = 0, kFusedRide = 1, kFusedAllBig = 2, kFusedWide = 3 };
// first-half passes with few tiles and at most this many rows per expert (the
// host's bound) run 128-row tiles of 256 weight rows over every row
constexpr int64_t kWideRows = 512;
enum class PipeRows { kBigTiles, kBigAll, kTailTiles, kAllRows, kBigRide, kTailRide, kAllRowsWide };
// true when one GEMM pass over E_loc experts with N output columns gives few
// tiles (fewer than 4 per CU with 256-row weight tiles on a device of cu
// compute units): then remainders ride along with the 256-row tiles instead
// of a second kernel re-streaming weights
bool few_gemm_tiles(int E_loc, int N, bool swiglu, int cu);
// whether a pass runs every row in 256-row tiles (kBigAll) rather than
// 256-row tiles plus a remainder kernel
bool remainders_with_big_tiles(int E_loc, int N, int K, bool swiglu, int cu);
// whether every operand of a bf16 FFN half (activations, one expert's
// weights, output) fits 32-bit byte offsets (the pipelined kernels' rule)
bool ffn_operands_fit32(bool up, int64_t max_rows, int d, int f);
// rows per expert on average (host bound) at or below which a pass streams
// weights with 32-row tiles
constexpr int64_t kStreamRows = 48;
// the kernels of one bf16 FFN half (up = GEMM1 + SwiGLU, else GEMM2): a
// moe_ffn_plan_t value (include/moe.h)
int ffn_plan_bf16(bool up, int64_t max_rows, int E_loc, int d, int f, int cu);
// FP8 (E4M3-FN) weights with 128 x 128 block scales, many rows per expert:
// the pipelined kernels of one row class with codes in LDS (K must be at
// least fp8_pipe_min_k() and a multiple of 128; operands below 4 GiB)
int fp8_pipe_min_k();
int launch_gemm_pipe_fp8(PipeRows rows, bool swiglu, const void* A, const int32_t* offsets,
                         int E_loc, int64_t max_rows, const uint8_t* Wq, const float* Ws, void* C,
                         int N, int K, const void* const* wlist, const float* const* slist,
                         void* stream);
// ab (SwiGLU only): if not null, the pre-activations are stored there too
// ([rows][2N]: a then g)
int launch_gemm_pipe_bf16(PipeRows rows, bool swiglu, const void* A, const int32_t* offsets,
                          int E_loc, int64_t max_rows, const void* W, void* C, int N, int K,
                          const void* const* wlist, void* stream, void* ab = nullptr);
// training forward of the first FFN half: h as launch_ffn_up_* and the
// pre-activations ab [rows][2f] (a = x W1, then g = x W3) for the backward
int launch_ffn_up_train_bf16(const void* x_perm, const int32_t* offsets, int E_loc,
                             int64_t max_rows, int d, int f, const void* w13, void* h, void* ab,
                             void* stream);
int launch_ffn_up_train_f32(const float* x_perm, const int32_t* offsets, int E_loc,
                            int64_t max_rows, int d, int f, const float* w13, float* h, float* ab,
                            void* stream);
// FP8 (E4M3-FN) weights with 128 x 128 block scales

int launch_quantize_fp8(const void* w, int E_loc, int R, int K, uint8_t* q, float* scales,
                        void* stream);
// few rows per expert: codes kept in LDS, converted per MFMA operand
// (FP8 launchers: wlist / slist, if not null, are device tables of E_loc
// per-expert code and scale buffers used in place of Wq / Ws)
int launch_gemm_fp8w(bool swiglu, const void* A, const int32_t* offsets, int E_loc,
                     int64_t max_rows, const uint8_t* Wq, const float* Ws, void* C, int N, int K,
                     void* stream, const void* const* wlist = nullptr,
                     const float* const* slist = nullptr);
int launch_ffn_up_fp8(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, const uint8_t* w13q, const float* w13s, void* h,
                      void* stream, const void* const* wlist = nullptr,
                      const float* const* slist = nullptr);
int launch_ffn_down_fp8(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, const uint8_t* w2q, const float* w2s, void* y,
                        void* stream, const void* const* wlist = nullptr,
                        const float* const* slist = nullptr);
int launch_ffn_up_f32(const float* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, const float* w13, float* h, const void* const* wlist,
                      void* stream);
int launch_ffn_down_f32(const float* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, const float* w2, float* y, const void* const* wlist,
                        void* stream);
// w == nullptr: unit weights
int launch_combine(const void* y_perm, const int32_t* pair_pos, const float* w, int T, int k,
                   int d, int bf16, void* y, void* stream);
// backward pass (backward.hip, wgrad.hip, pack.hip)
int launch_pack_backward(const void* w1, const void* w3, int E_loc, int d, int f, int elem_bytes,
                         void* w13_t, void* stream);
int launch_combine_backward(const void* dy, const void* y_perm, const int32_t* pair_pos,
                            const float* topk_w, int T, int k, int d, int bf16, void* do_perm,
                            float* dgate, void* stream);
int launch_gate_backward(const float* logits, const int32_t* topk_idx, const float* dgate, int T,
                         int E, int k, int gate, float* dlogits, void* stream);
int launch_swiglu_backward(const void* dh, const void* ab, const int32_t* offsets, int E_loc,
                           int64_t max_rows, int f, int bf16, void* dab, void* stream);
size_t router_backward_ws_bytes(int T, int d, int E);
int launch_router_backward(const void* x, const float* wg, const float* dlogits, int T, int d,
                           int E, int bf16, void* dx, float* dwg, float* part, void* stream);
// padded row pitch of the transposed weight-gradient operands, and the
// workspace they need (bf16; fp32 needs only the segment table)
size_t wgrad_ldk(int64_t max_rows, int E_loc);
size_t wgrad_ws_bytes(int64_t max_rows, int E_loc, int d, int f, int bf16);
int launch_ffn_wgrad(const void* x_perm, const void* h, const void* do_perm, const void* dab,
                     const int32_t* offsets, int E_loc, int64_t max_rows, int d, int f, int bf16,
                     float* dw13, float* dw2, void* ws, void* stream);
int launch_pack(const void* w1, const void* w3, const void* w2, int E_loc, int d, int f,
                int elem_bytes, void* w13, void* w2p, void* stream);
int check_error(void* ws, void* stream, int* device_flags);

// Arguments of the fused persistent layer (every pointer already validated).
struct FusedArgs {
  const float* logits;
  const void* x;
  const void* w13;
  const void* w2;
  const void* const* w13_list;  // per-expert weight tables (TensorList form), else null
  const void* const* w2_list;
  const float* w13s;  // FP8 weights: the codes' 128 x 128 block scales (else null)
  const float* w2s;
  const float* const* w13s_list;  // FP8 per-expert scale tables (TensorList form), else null
  const float* const* w2s_list;
  int T, E, k, gate, capacity, e_begin, e_end, d, f;
  int ffn_all_rows;  // bf16: 1 = every row in 128-row tiles (few rows per expert)
  int rows_up, rows_down;  // bf16 GEMM phases (unless ffn_all_rows): a FusedRows value
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* n_kept;
  void* h;
  void* y_perm;
  void* y;
  int reroute;          // route with capacity-overflow rerouting (candidates below)
  int32_t* cand_e;      // rerouting scratch in the workspace: [T][k+1] candidates,
  float* cand_v;        //   their logits,
  uint64_t* rerouted;   //   one rerouted mask per 64 tokens
  int* err;             // workspace error word
  int* block_counts;    // workspace per-block expert counts
  uint32_t* bar_gen;    // workspace barrier words: generation,
  uint32_t* bar_count;  // top-level arrivals,
  uint32_t* bar_group;  // 8 group arrival counters, kWsBarStride words apart
  int overlap;          // 1: GEMM2 tiles wait per expert on up_ready instead of a barrier
  uint32_t* up_ready;   // workspace: [E_loc] GEMM1 stored rows x (columns / 32) per expert
};
// bytes of the per-expert readiness counters that follow the dispatch and
// rerouting scratch in a moe_workspace_bytes workspace
size_t ready_ws_bytes(int E_loc);
// byte offsets of the barrier words inside the workspace header (each on its
// own 128-byte line)
constexpr size_t kWsBarGen = 128;
constexpr size_t kWsBarCount = 256;
constexpr size_t kWsBarGroup = 512;
constexpr size_t kWsBarStride = 32;  // uint32 words = 128 bytes
size_t fused_lds_bytes(int E, bool bf16, bool fp8 = false);
// fp8 (bf16 activations only): w13 / w2 hold E4M3 codes with block scales
// w13s / w2s; their K (d and f) must be multiples of 128 and at least
// fp8_pipe_min_k()
int launch_fused(const FusedArgs& a, bool bf16, int64_t max_rows, void* stream, bool fp8 = false);

int device_cu_count();

// Per-kernel record of the devices on which the kernel's dynamic-LDS limit has
// been raised (hipFuncAttributeMaxDynamicSharedMemorySize); zero-initialised
// as a static object.
struct LdsAttr {
  static constexpr int kMaxDevices = 64;
  volatile int done[kMaxDevices];
};
// raises kern's dynamic-LDS limit to `bytes` on the current device the first
// time it is asked for there (racing first calls both set it: harmless)
int set_dynamic_lds_once(const void* kern, size_t bytes, LdsAttr& rec);

}  // namespace moe
