// C ABI of the MoE expert path: argument validation and launch.
//
// Validation is pure host code that makes no HIP call, so every invalid
// argument is rejected (and can be tested) without touching a GPU.  Only
// after validation do the entry points call the launchers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "launch.h"
#include "moe.h"

namespace {

thread_local int g_last_hip_error = 0;

// how the fused launch orders its two GEMM phases (moe_set_fused_overlap)
std::atomic<int> g_fused_overlap{MOE_OVERLAP_AUTO};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline moe_status hip_status(int e) {
  if (e != 0) {
    g_last_hip_error = e;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

inline bool elem_ok(int dtype) { return dtype == MOE_F32 || dtype == MOE_BF16; }
inline int elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

moe_status check_topk(int E, int k) {
  if (E < 1 || E > MOE_MAX_E) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > E || k > MOE_MAX_K) return MOE_ERR_INVALID_TOPK;
  return MOE_OK;
}

// FFN shape rules shared by moe_expert_ffn and its halves
moe_status check_ffn(const void* a, const int32_t* offsets, int E_loc, int64_t max_rows, int d,
                     int f, int dtype, const void* w, const void* out) {
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (E_loc < 1 || E_loc > MOE_MAX_E || max_rows < 0 || d < 1 || f < 1)
    return MOE_ERR_INVALID_ARG;
  if (max_rows > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (!offsets || !w) return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && (!a || !out)) return MOE_ERR_INVALID_ARG;
  if (dtype == MOE_BF16 && (d % 64 != 0 || f % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_F32 && (d % 4 != 0 || f % 4 != 0)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(offsets) || !aligned16(w) || !aligned16(out))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// FP8-weight FFN rules: bf16 activations, d and f multiples of the 128 x 128 scale blocks
moe_status check_ffn_fp8(const void* a, const int32_t* offsets, int E_loc, int64_t max_rows,
                         int d, int f, const void* wq, const float* ws, const void* out) {
  moe_status st = check_ffn(a, offsets, E_loc, max_rows, d, f, MOE_BF16, wq, out);
  if (st != MOE_OK) return st;
  if (d % 128 != 0 || f % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// the two FFN halves on packed weights (wlist null) or a per-expert weight table
moe_status launch_up(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows, int d,
                     int f, int dtype, const void* w13, const void* const* wlist, void* h,
                     void* stream) {
  if (dtype == MOE_BF16)
    return hip_status(moe::launch_ffn_up_bf16(x_perm, offsets, E_loc, max_rows, d, f, w13, h,
                                              wlist, stream));
  return hip_status(moe::launch_ffn_up_f32(static_cast<const float*>(x_perm), offsets, E_loc,
                                           max_rows, d, f, static_cast<const float*>(w13),
                                           static_cast<float*>(h), wlist, stream));
}

moe_status launch_down(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows, int d,
                       int f, int dtype, const void* w2, const void* const* wlist, void* y,
                       void* stream) {
  if (dtype == MOE_BF16)
    return hip_status(moe::launch_ffn_down_bf16(h, offsets, E_loc, max_rows, d, f, w2, y, wlist,
                                                stream));
  return hip_status(moe::launch_ffn_down_f32(static_cast<const float*>(h), offsets, E_loc,
                                             max_rows, d, f, static_cast<const float*>(w2),
                                             static_cast<float*>(y), wlist, stream));
}

// the rerouting launches with their scratch (candidates [T][k+1] as expert
// ids, then as logits, then one mask per 64 tokens; moe::reroute_ws_bytes)
// starting at c
moe_status launch_reroute_in(const float* logits, int T, int E, int k, int gate, int capacity,
                             int32_t* topk_idx, float* topk_w, char* c, void* stream) {
  const size_t n = static_cast<size_t>(T) * (k + 1);
  const size_t cand_bytes = (n * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
  int32_t* cand_e = reinterpret_cast<int32_t*>(c);
  float* cand_v = reinterpret_cast<float*>(c + cand_bytes);
  uint64_t* rerouted = reinterpret_cast<uint64_t*>(c + 2 * cand_bytes);
  return hip_status(moe::launch_route_reroute(logits, T, E, k, gate, capacity, topk_idx, topk_w,
                                              cand_e, cand_v, rerouted, stream));
}

}  // namespace

namespace moe {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int set_dynamic_lds_once(const void* kern, size_t bytes, LdsAttr& rec) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= LdsAttr::kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  if (rec.done[dev]) return 0;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e != hipSuccess) return static_cast<int>(e);
  rec.done[dev] = 1;
  return 0;
}

int check_error(void* ws, void* stream, int* device_flags) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return static_cast<int>(e);
  int flags = 0;
  e = hipMemcpy(&flags, ws, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return static_cast<int>(e);
  if (flags != 0) {
    // clear the error word; after a barrier time-out also re-arm the fused
    // layer's barrier words (the whole header)
    e = hipMemset(ws, 0, (flags & (1 << MOE_ERR_HIP)) ? kWsHeader : sizeof(int));
    if (e != hipSuccess) return static_cast<int>(e);
  }
  *device_flags = flags;
  return 0;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid size, range or pointer";
    case MOE_ERR_INVALID_TOPK: return "MOE_ERR_INVALID_TOPK: top-k out of range or invalid expert index";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: dtype or shape not supported";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    default: return "unknown moe_status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

size_t moe_workspace_bytes(int T, int E, int k, int E_loc) {
  if (T < 0 || E < 1 || E > MOE_MAX_E || k < 1 || k > MOE_MAX_K || k > E || E_loc < 1 || E_loc > E)
    return 0;
  return moe::dispatch_ws_bytes(T, E) + moe::reroute_ws_bytes(T, k) + moe::ready_ws_bytes(E_loc);
}

int64_t moe_capacity(int T, int k, int E, int64_t cf_num, int64_t cf_den) {
  if (cf_num < 0) return -1;
  if (T < 0 || k < 1 || E < 1 || cf_den < 1) return -2;
  const int64_t num = cf_num * static_cast<int64_t>(T) * k;  // callers keep cf_num small
  const int64_t den = cf_den * static_cast<int64_t>(E);
  return (num + den - 1) / den;
}

int64_t moe_max_rows(int T, int k, int E_loc, int capacity) {
  const int64_t all = static_cast<int64_t>(T) * k;
  if (capacity < 0) return all;
  const int64_t cap = static_cast<int64_t>(E_loc) * capacity;
  return cap < all ? cap : all;
}

moe_status moe_pack_weights(const void* w1, const void* w3, const void* w2, int E_loc, int d,
                            int f, moe_dtype dtype, void* w13_packed, void* w2_packed,
                            void* stream) {
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (E_loc < 1 || E_loc > MOE_MAX_E || d < 1 || f < 1) return MOE_ERR_INVALID_ARG;
  if (!w1 || !w3 || !w2 || !w13_packed || !w2_packed) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w1) || !aligned16(w3) || !aligned16(w2) || !aligned16(w13_packed) ||
      !aligned16(w2_packed))
    return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_pack(w1, w3, w2, E_loc, d, f, elem_bytes(dtype), w13_packed,
                                     w2_packed, stream));
}

moe_status moe_router_logits(const void* x, const float* w_gate, int T, int d, int E,
                             float* logits, void* stream) {
  if (T < 0 || d < 1 || E < 1 || E > MOE_MAX_E) return MOE_ERR_INVALID_ARG;
  if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(logits)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_router_logits(x, w_gate, T, d, E, logits, stream));
}

moe_status moe_route(const float* logits, int T, int E, int k, int gate, int32_t* topk_idx,
                     float* topk_w, void* stream) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  moe_status st = check_topk(E, k);
  if (st != MOE_OK) return st;
  if (gate != MOE_GATE_SOFTMAX_TOPK_RENORM && gate != MOE_GATE_SIGMOID_TOPK_NORM)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_route(logits, T, E, k, gate, topk_idx, topk_w, stream));
}

moe_status moe_dispatch(const int32_t* topk_idx, int T, int E, int k, int capacity,
                        int e_begin, int e_end, const void* x, int d, moe_dtype dtype,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                        int32_t* pair_pos, int32_t* n_kept, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  moe_status st = check_topk(E, k);
  if (st != MOE_OK) return st;
  if (!(0 <= e_begin && e_begin < e_end && e_end <= E)) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(T) * k > INT32_MAX) return MOE_ERR_INVALID_ARG;
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (x) {
    if (d < 1) return MOE_ERR_INVALID_ARG;
    if ((static_cast<int64_t>(d) * elem_bytes(dtype)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (!x_perm) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_MISALIGNED;
  }
  if (!counts || !offsets || !pair_pos || !n_kept || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && !sorted_pair) return MOE_ERR_INVALID_ARG;
  if (!aligned16(topk_idx) || !aligned16(counts) || !aligned16(offsets) ||
      !aligned16(sorted_pair) || !aligned16(pair_pos) || !aligned16(n_kept) || !aligned16(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < moe::dispatch_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  if (T > 0 && !topk_idx) return MOE_ERR_INVALID_ARG;
  const moe::DispatchWs w = moe::dispatch_ws(ws, T, E);
  return hip_status(moe::launch_dispatch(topk_idx, T, E, k, capacity, e_begin, e_end, x, d,
                                         elem_bytes(dtype), counts, offsets, sorted_pair,
                                         pair_pos, n_kept, x_perm, w, stream));
}

moe_status moe_ffn_up(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, moe_dtype dtype, const void* w13_packed, void* h,
                      void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_ffn(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_packed, h);
  if (st != MOE_OK) return st;
  return launch_up(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_packed, nullptr, h, stream);
}

moe_status moe_ffn_down(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, moe_dtype dtype, const void* w2_packed, void* y_perm,
                        void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  moe_status st = check_ffn(h, offsets, E_loc, max_rows, d, f, dtype, w2_packed, y_perm);
  if (st != MOE_OK) return st;
  return launch_down(h, offsets, E_loc, max_rows, d, f, dtype, w2_packed, nullptr, y_perm, stream);
}

moe_status moe_expert_ffn(const void* x_perm, const int32_t* offsets, int E_loc,
                          int64_t max_rows, int d, int f, moe_dtype dtype,
                          const void* w13_packed, const void* w2_packed, void* h, void* y_perm,
                          void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_ffn(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_packed, h);
  if (st != MOE_OK) return st;
  st = check_ffn(h, offsets, E_loc, max_rows, d, f, dtype, w2_packed, y_perm);
  if (st != MOE_OK) return st;
  st = moe_ffn_up(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_packed, h, ws, ws_bytes,
                  stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down(h, offsets, E_loc, max_rows, d, f, dtype, w2_packed, y_perm, ws, ws_bytes,
                      stream);
}

moe_status moe_quantize_fp8(const void* w_packed, int E_loc, int rows, int K, uint8_t* q,
                            float* scales, void* stream) {
  if (E_loc < 1 || rows < 1 || K < 1 || !w_packed || !q || !scales) return MOE_ERR_INVALID_ARG;
  if (rows % 128 != 0 || K % 128 != 0 || E_loc > 65535) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(w_packed) || !aligned16(q) || !aligned16(scales)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_quantize_fp8(w_packed, E_loc, rows, K, q, scales, stream));
}


moe_status moe_ffn_up_fp8(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                          int d, int f, const uint8_t* w13_q, const float* w13_s, void* h,
                          void* stream) {
  moe_status st = check_ffn_fp8(x_perm, offsets, E_loc, max_rows, d, f, w13_q, w13_s, h);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_up_fp8(x_perm, offsets, E_loc, max_rows, d, f, w13_q, w13_s,
                                           h, stream));
}

moe_status moe_ffn_down_fp8(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                            int d, int f, const uint8_t* w2_q, const float* w2_s, void* y_perm,
                            void* stream) {
  moe_status st = check_ffn_fp8(h, offsets, E_loc, max_rows, d, f, w2_q, w2_s, y_perm);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_down_fp8(h, offsets, E_loc, max_rows, d, f, w2_q, w2_s,
                                             y_perm, stream));
}

// the FP8 calls over per-expert code and scale buffers: the tables stand
// where the packed codes and scales do in the shape and pointer checks
moe_status moe_ffn_up_fp8_list(const void* x_perm, const int32_t* offsets, int E_loc,
                               int64_t max_rows, int d, int f, const void* const* w13_q_list,
                               const float* const* w13_s_list, void* h, void* stream) {
  moe_status st = check_ffn_fp8(x_perm, offsets, E_loc, max_rows, d, f, w13_q_list,
                                reinterpret_cast<const float*>(w13_s_list), h);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_up_fp8(x_perm, offsets, E_loc, max_rows, d, f, nullptr,
                                           nullptr, h, stream, w13_q_list, w13_s_list));
}

moe_status moe_ffn_down_fp8_list(const void* h, const int32_t* offsets, int E_loc,
                                 int64_t max_rows, int d, int f, const void* const* w2_q_list,
                                 const float* const* w2_s_list, void* y_perm, void* stream) {
  moe_status st = check_ffn_fp8(h, offsets, E_loc, max_rows, d, f, w2_q_list,
                                reinterpret_cast<const float*>(w2_s_list), y_perm);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_ffn_down_fp8(h, offsets, E_loc, max_rows, d, f, nullptr, nullptr,
                                             y_perm, stream, w2_q_list, w2_s_list));
}

moe_status moe_expert_ffn_fp8_list(const void* x_perm, const int32_t* offsets, int E_loc,
                                   int64_t max_rows, int d, int f,
                                   const void* const* w13_q_list, const float* const* w13_s_list,
                                   const void* const* w2_q_list, const float* const* w2_s_list,
                                   void* h, void* y_perm, void* stream) {
  moe_status st = check_ffn_fp8(x_perm, offsets, E_loc, max_rows, d, f, w13_q_list,
                                reinterpret_cast<const float*>(w13_s_list), h);
  if (st != MOE_OK) return st;
  st = check_ffn_fp8(h, offsets, E_loc, max_rows, d, f, w2_q_list,
                     reinterpret_cast<const float*>(w2_s_list), y_perm);
  if (st != MOE_OK) return st;
  st = moe_ffn_up_fp8_list(x_perm, offsets, E_loc, max_rows, d, f, w13_q_list, w13_s_list, h,
                           stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down_fp8_list(h, offsets, E_loc, max_rows, d, f, w2_q_list, w2_s_list, y_perm,
                               stream);
}

moe_status moe_expert_ffn_fp8(const void* x_perm, const int32_t* offsets, int E_loc,
                              int64_t max_rows, int d, int f, const uint8_t* w13_q,
                              const float* w13_s, const uint8_t* w2_q, const float* w2_s,
                              void* h, void* y_perm, void* stream) {
  moe_status st = check_ffn_fp8(x_perm, offsets, E_loc, max_rows, d, f, w13_q, w13_s, h);
  if (st != MOE_OK) return st;
  st = check_ffn_fp8(h, offsets, E_loc, max_rows, d, f, w2_q, w2_s, y_perm);
  if (st != MOE_OK) return st;
  st = moe_ffn_up_fp8(x_perm, offsets, E_loc, max_rows, d, f, w13_q, w13_s, h, stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down_fp8(h, offsets, E_loc, max_rows, d, f, w2_q, w2_s, y_perm, stream);
}

moe_status moe_route_reroute(const float* logits, int T, int E, int k, int gate, int capacity,
                             int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_topk(E, k);
  if (st != MOE_OK) return st;
  if (T < 0 || capacity < -1 || (gate != MOE_GATE_SOFTMAX_TOPK_RENORM &&
                                 gate != MOE_GATE_SIGMOID_TOPK_NORM))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(ws))
    return MOE_ERR_MISALIGNED;
  const size_t off = moe::dispatch_ws_bytes(T, E);
  if (ws_bytes < off + moe::reroute_ws_bytes(T, k)) return MOE_ERR_WORKSPACE;
  return launch_reroute_in(logits, T, E, k, gate, capacity, topk_idx, topk_w,
                           static_cast<char*>(ws) + off, stream);
}

moe_status moe_route_reroute_noalloc(const float* logits, int T, int E, int k, int gate,
                                     int capacity, int32_t* topk_idx, float* topk_w,
                                     void* stream) {
  moe_status st = check_topk(E, k);
  if (st != MOE_OK) return st;
  if (T < 0 || capacity < -1 || (gate != MOE_GATE_SOFTMAX_TOPK_RENORM &&
                                 gate != MOE_GATE_SIGMOID_TOPK_NORM))
    return MOE_ERR_INVALID_ARG;
  if (moe::reroute_ws_bytes(T, k) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w)) return MOE_ERR_MISALIGNED;
  void* scratch = nullptr;
  if (int e = moe::noalloc_scratch(&scratch)) return hip_status(e);
  return launch_reroute_in(logits, T, E, k, gate, capacity, topk_idx, topk_w,
                           static_cast<char*>(scratch), stream);
}

moe_status moe_ffn_up_list(const void* x_perm, const int32_t* offsets, int E_loc,
                          int64_t max_rows, int d, int f, moe_dtype dtype,
                          const void* const* w13_list, void* h, void* stream) {
  moe_status st = check_ffn(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_list, h);
  if (st != MOE_OK) return st;
  return launch_up(x_perm, offsets, E_loc, max_rows, d, f, dtype, nullptr, w13_list, h, stream);
}

moe_status moe_ffn_down_list(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                            int d, int f, moe_dtype dtype, const void* const* w2_list,
                            void* y_perm, void* stream) {
  moe_status st = check_ffn(h, offsets, E_loc, max_rows, d, f, dtype, w2_list, y_perm);
  if (st != MOE_OK) return st;
  return launch_down(h, offsets, E_loc, max_rows, d, f, dtype, nullptr, w2_list, y_perm, stream);
}

moe_status moe_expert_ffn_list(const void* x_perm, const int32_t* offsets, int E_loc,
                               int64_t max_rows, int d, int f, moe_dtype dtype,
                               const void* const* w13_list, const void* const* w2_list, void* h,
                               void* y_perm, void* stream) {
  moe_status st = check_ffn(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_list, h);
  if (st != MOE_OK) return st;
  st = check_ffn(h, offsets, E_loc, max_rows, d, f, dtype, w2_list, y_perm);
  if (st != MOE_OK) return st;
  st = moe_ffn_up_list(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_list, h, stream);
  if (st != MOE_OK) return st;
  return moe_ffn_down_list(h, offsets, E_loc, max_rows, d, f, dtype, w2_list, y_perm, stream);
}

moe_status moe_combine(const void* y_perm, const int32_t* pair_pos, const float* topk_w, int T,
                       int k, int d, moe_dtype dtype, void* y, void* stream) {
  if (T < 0 || d < 1 || k < 1 || k > MOE_MAX_K) return MOE_ERR_INVALID_ARG;
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(d) * elem_bytes(dtype)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!pair_pos || !y) return MOE_ERR_INVALID_ARG;  // topk_w null: unit weights
  if (!aligned16(y_perm) || !aligned16(pair_pos) || !aligned16(topk_w) || !aligned16(y))
    return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_combine(y_perm, pair_pos, topk_w, T, k, d, dtype == MOE_BF16, y,
                                        stream));
}

moe_status moe_check_error(void* ws, void* stream) {
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
  int flags = 0;
  int e = moe::check_error(ws, stream, &flags);
  if (e != 0) return hip_status(e);
  if (flags & (1 << MOE_ERR_INVALID_TOPK)) return MOE_ERR_INVALID_TOPK;
  if (flags & (1 << MOE_ERR_HIP)) return MOE_ERR_HIP;
  if (flags != 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------

moe_status moe_ffn_up_train(const void* x_perm, const int32_t* offsets, int E_loc,
                            int64_t max_rows, int d, int f, moe_dtype dtype,
                            const void* w13_packed, void* h, void* ab, void* stream) {
  moe_status st = check_ffn(x_perm, offsets, E_loc, max_rows, d, f, dtype, w13_packed, h);
  if (st != MOE_OK) return st;
  if (max_rows > 0 && !ab) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ab)) return MOE_ERR_MISALIGNED;
  if (dtype == MOE_BF16) {
    const double rows = static_cast<double>(max_rows);
    if (rows * d * 2 >= 4294967296.0 || rows * 2 * f * 2 >= 4294967296.0 ||
        2.0 * f * d * 2 >= 4294967296.0)
      return MOE_ERR_UNSUPPORTED;  // the pipelined GEMM addresses operands with 32-bit offsets
    return hip_status(moe::launch_ffn_up_train_bf16(x_perm, offsets, E_loc, max_rows, d, f,
                                                    w13_packed, h, ab, stream));
  }
  return hip_status(moe::launch_ffn_up_train_f32(
      static_cast<const float*>(x_perm), offsets, E_loc, max_rows, d, f,
      static_cast<const float*>(w13_packed), static_cast<float*>(h), static_cast<float*>(ab),
      stream));
}

moe_status moe_pack_weights_backward(const void* w1, const void* w3, int E_loc, int d, int f,
                                     moe_dtype dtype, void* w13_t, void* stream) {
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (E_loc < 1 || E_loc > MOE_MAX_E || d < 1 || f < 1) return MOE_ERR_INVALID_ARG;
  if ((static_cast<int64_t>(f) * elem_bytes(dtype)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (!w1 || !w3 || !w13_t) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w1) || !aligned16(w3) || !aligned16(w13_t)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_pack_backward(w1, w3, E_loc, d, f, elem_bytes(dtype), w13_t,
                                              stream));
}

moe_status moe_combine_backward(const void* dy, const void* y_perm, const int32_t* pair_pos,
                                const float* topk_w, int T, int k, int d, moe_dtype dtype,
                                void* do_perm, float* dgate, void* stream) {
  if (T < 0 || d < 1 || k < 1 || k > MOE_MAX_K) return MOE_ERR_INVALID_ARG;
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(d) * elem_bytes(dtype)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dy || !pair_pos || !topk_w || !dgate) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(y_perm) || !aligned16(pair_pos) || !aligned16(topk_w) ||
      !aligned16(do_perm) || !aligned16(dgate))
    return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_combine_backward(dy, y_perm, pair_pos, topk_w, T, k, d,
                                                 dtype == MOE_BF16, do_perm, dgate, stream));
}

moe_status moe_gate_backward(const float* logits, const int32_t* topk_idx, const float* dgate,
                             int T, int E, int k, int gate, float* dlogits, void* stream) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  moe_status st = check_topk(E, k);
  if (st != MOE_OK) return st;
  if (gate != MOE_GATE_SOFTMAX_TOPK_RENORM && gate != MOE_GATE_SIGMOID_TOPK_NORM)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !dgate || !dlogits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(dgate) || !aligned16(dlogits))
    return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_gate_backward(logits, topk_idx, dgate, T, E, k, gate, dlogits,
                                              stream));
}

moe_status moe_ffn_down_backward(const void* do_perm, const int32_t* offsets, int E_loc,
                                 int64_t max_rows, int d, int f, moe_dtype dtype,
                                 const void* w2_t, const void* ab, void* dh, void* dab,
                                 void* stream) {
  // dh = do . W2^T is the down GEMM's form with the roles of d and f swapped
  moe_status st = check_ffn(do_perm, offsets, E_loc, max_rows, f, d, dtype, w2_t, dh);
  if (st != MOE_OK) return st;
  if (max_rows > 0 && (!ab || !dab)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(ab) || !aligned16(dab)) return MOE_ERR_MISALIGNED;
  st = launch_down(do_perm, offsets, E_loc, max_rows, f, d, dtype, w2_t, nullptr, dh, stream);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_swiglu_backward(dh, ab, offsets, E_loc, max_rows, f,
                                                dtype == MOE_BF16, dab, stream));
}

moe_status moe_ffn_up_backward(const void* dab, const int32_t* offsets, int E_loc,
                               int64_t max_rows, int d, int f, moe_dtype dtype,
                               const void* w13_t, void* dx_perm, void* stream) {
  // dx = dab . [W1 | W3]^T: the down GEMM's form with K = 2f
  moe_status st = check_ffn(dab, offsets, E_loc, max_rows, d, 2 * f, dtype, w13_t, dx_perm);
  if (st != MOE_OK) return st;
  return launch_down(dab, offsets, E_loc, max_rows, d, 2 * f, dtype, w13_t, nullptr, dx_perm,
                     stream);
}

size_t moe_wgrad_workspace_bytes(int64_t max_rows, int E_loc, int d, int f, moe_dtype dtype) {
  if (max_rows < 0 || E_loc < 1 || d < 1 || f < 1) return 0;
  return moe::wgrad_ws_bytes(max_rows, E_loc, d, f, dtype == MOE_BF16);
}

moe_status moe_ffn_wgrad(const void* x_perm, const void* h, const void* do_perm, const void* dab,
                         const int32_t* offsets, int E_loc, int64_t max_rows, int d, int f,
                         moe_dtype dtype, float* dw13, float* dw2, void* ws, size_t ws_bytes,
                         void* stream) {
  moe_status st = check_ffn(x_perm, offsets, E_loc, max_rows, d, f, dtype, dw13, h);
  if (st != MOE_OK) return st;
  if (!dw2 || !ws) return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && (!do_perm || !dab)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(do_perm) || !aligned16(dab) || !aligned16(dw2) || !aligned16(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < moe::wgrad_ws_bytes(max_rows, E_loc, d, f, dtype == MOE_BF16))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_ffn_wgrad(x_perm, h, do_perm, dab, offsets, E_loc, max_rows, d,
                                          f, dtype == MOE_BF16, dw13, dw2, ws, stream));
}

size_t moe_router_backward_workspace_bytes(int T, int d, int E) {
  if (T < 0 || d < 1 || E < 1) return 0;
  return moe::router_backward_ws_bytes(T, d, E);
}

moe_status moe_router_backward(const void* x, const float* w_gate, const float* dlogits, int T,
                               int d, int E, moe_dtype dtype, void* dx, float* dw_gate, void* ws,
                               size_t ws_bytes, void* stream) {
  if (T < 0 || d < 1 || E < 1 || E > 64) return MOE_ERR_INVALID_ARG;
  if (!elem_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!w_gate || !dw_gate || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !dlogits || !dx)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(dlogits) || !aligned16(dx) ||
      !aligned16(dw_gate) || !aligned16(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < moe::router_backward_ws_bytes(T, d, E)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_router_backward(x, w_gate, dlogits, T, d, E, dtype == MOE_BF16,
                                                dx, dw_gate, static_cast<float*>(ws), stream));
}

static moe_status forward_fused_impl(const float* logits, const void* x, int T, int E, int k,
                                     int gate, int capacity, int e_begin, int e_end, int d, int f,
                                     moe_dtype dtype, const void* w13_packed,
                                     const void* w2_packed, int32_t* topk_idx, float* topk_w,
                                     int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                     int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                     void* y, void* ws, size_t ws_bytes, void* stream,
                                     bool reroute, const float* w13s = nullptr,
                                     const float* w2s = nullptr,
                                     const void* const* w13_list = nullptr,
                                     const void* const* w2_list = nullptr,
                                     const float* const* w13s_list = nullptr,
                                     const float* const* w2s_list = nullptr) {
  // w13s / w2s (or their tables) set: FP8 weights (codes in w13_packed /
  // w2_packed or the code tables, bf16 activations)
  const bool fp8 = w13s != nullptr || w2s != nullptr || w13s_list != nullptr ||
                   w2s_list != nullptr;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  moe_status st = check_topk(E, k);
  if (st != MOE_OK) return st;
  if (gate != MOE_GATE_SOFTMAX_TOPK_RENORM && gate != MOE_GATE_SIGMOID_TOPK_NORM)
    return MOE_ERR_INVALID_ARG;
  if (!(0 <= e_begin && e_begin < e_end && e_end <= E)) return MOE_ERR_INVALID_ARG;
  if (static_cast<int64_t>(T) * k > INT32_MAX) return MOE_ERR_INVALID_ARG;
  const int E_loc = e_end - e_begin;
  const int64_t max_rows = moe_max_rows(T, k, E_loc, capacity);
  // the two GEMMs' rules (shape, alignment) on the buffers they touch
  // GEMM1 reads x in place (rows gathered through sorted_pair)
  if (fp8) {
    if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    // (TensorList form: the code and scale tables stand where the packed ones do)
    const bool tables = w13s_list != nullptr || w2s_list != nullptr;
    if (tables && (!w13_list || !w2_list || !w13s_list || !w2s_list)) return MOE_ERR_INVALID_ARG;
    st = check_ffn_fp8(x, offsets, E_loc, max_rows, d, f, tables ? w13_list : w13_packed,
                       tables ? reinterpret_cast<const float*>(w13s_list) : w13s, h);
    if (st != MOE_OK) return st;
    st = check_ffn_fp8(h, offsets, E_loc, max_rows, d, f, tables ? w2_list : w2_packed,
                       tables ? reinterpret_cast<const float*>(w2s_list) : w2s, y_perm);
    if (st != MOE_OK) return st;
    // the pipelined FP8 body's depth
    if (d < moe::fp8_pipe_min_k() || f < moe::fp8_pipe_min_k()) return MOE_ERR_UNSUPPORTED;
  } else {
    // (TensorList form: the tables stand where the packed weights do)
    if (w13_list != nullptr) w13_packed = w13_list;
    if (w2_list != nullptr) w2_packed = w2_list;
    st = check_ffn(x, offsets, E_loc, max_rows, d, f, dtype, w13_packed, h);
    if (st != MOE_OK) return st;
    st = check_ffn(h, offsets, E_loc, max_rows, d, f, dtype, w2_packed, y_perm);
    if (st != MOE_OK) return st;
  }
  const double big = static_cast<double>(max_rows > T ? max_rows : T);
  if (dtype == MOE_BF16 && (big * (d > f ? d : f) * 2 >= 4294967296.0 ||
                            static_cast<double>(2) * f * d * 2 >= 4294967296.0))
    return MOE_ERR_UNSUPPORTED;  // the fused GEMMs address operands with 32-bit offsets
  if (!ws || !counts || !n_kept || !y) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !x || !topk_idx || !topk_w || !sorted_pair || !pair_pos))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(x) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      !aligned16(counts) || !aligned16(sorted_pair) || !aligned16(pair_pos) ||
      !aligned16(n_kept) || !aligned16(y) || !aligned16(ws))
    return MOE_ERR_MISALIGNED;
  if (ws_bytes < moe::dispatch_ws_bytes(T, E) + (reroute ? moe::reroute_ws_bytes(T, k) : 0))
    return MOE_ERR_WORKSPACE;
  const moe::DispatchWs w = moe::dispatch_ws(ws, T, E);
  moe::FusedArgs a;
  a.reroute = reroute ? 1 : 0;
  a.cand_e = nullptr;
  a.cand_v = nullptr;
  a.rerouted = nullptr;
  if (reroute) {  // the same workspace layout as moe_route_reroute
    char* c = static_cast<char*>(ws) + moe::dispatch_ws_bytes(T, E);
    const size_t cand_bytes =
        (static_cast<size_t>(T) * (k + 1) * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
    a.cand_e = reinterpret_cast<int32_t*>(c);
    a.cand_v = reinterpret_cast<float*>(c + cand_bytes);
    a.rerouted = reinterpret_cast<uint64_t*>(c + 2 * cand_bytes);
  }
  a.logits = logits;
  a.x = x;
  a.w13 = w13_list != nullptr ? nullptr : w13_packed;
  a.w2 = w2_list != nullptr ? nullptr : w2_packed;
  a.w13_list = w13_list;
  a.w2_list = w2_list;
  a.w13s = w13s;
  a.w2s = w2s;
  a.w13s_list = w13s_list;
  a.w2s_list = w2s_list;
  a.T = T;
  a.E = E;
  a.k = k;
  a.gate = gate;
  a.capacity = capacity;
  a.e_begin = e_begin;
  a.e_end = e_end;
  a.d = d;
  a.f = f;
  a.ffn_all_rows = max_rows / E_loc <= 48 ? 1 : 0;
  // the row splits of the separate FFN calls
  const int64_t avg_rows = max_rows / E_loc;
  const int cu = moe::device_cu_count();
  if (!moe::few_gemm_tiles(E_loc, f, true, cu))
    a.rows_up = moe::kFusedRide;
  else if (avg_rows <= moe::kWideRows)
    a.rows_up = moe::kFusedWide;
  else
    a.rows_up = moe::remainders_with_big_tiles(E_loc, f, d, true, cu) ? moe::kFusedAllBig
                                                                      : moe::kFusedBigTail;
  if (!moe::few_gemm_tiles(E_loc, d, false, cu))
    a.rows_down = moe::kFusedRide;
  else
    a.rows_down = moe::remainders_with_big_tiles(E_loc, d, f, false, cu) ? moe::kFusedAllBig
                                                                         : moe::kFusedBigTail;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.counts = counts;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.pair_pos = pair_pos;
  a.n_kept = n_kept;
  a.h = h;
  a.y_perm = y_perm;
  a.y = y;
  a.err = w.err;
  a.block_counts = w.block_counts;
  a.bar_gen = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + moe::kWsBarGen);
  a.bar_count = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + moe::kWsBarCount);
  a.bar_group = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + moe::kWsBarGroup);
  // GEMM1 -> GEMM2 per expert instead of a barrier.  Possible when both
  // phases run the pipelined body (bf16; FP8 unless its code-streaming body
  // runs), the workspace holds the counters and their largest value,
  // max_rows * f / 32, fits 32 bits.  Chosen (auto) when every row goes to
  // 128-row tiles: each expert is one M-tile, so no weight tile is shared
  // between tiles and the consumer's acquire (which invalidates the L2)
  // costs no re-fetch; with several M-tiles per expert it measured slower
  // than the barrier.
  const size_t ready_at = moe::dispatch_ws_bytes(T, E) + moe::reroute_ws_bytes(T, k);
  const bool can_overlap = dtype == MOE_BF16 && !(fp8 && a.ffn_all_rows) &&
                           ws_bytes >= ready_at + moe::ready_ws_bytes(E_loc) &&
                           static_cast<double>(max_rows) * (f / 32) < 4294967296.0;
  const int mode = g_fused_overlap.load(std::memory_order_relaxed);
  a.overlap = can_overlap && (mode == MOE_OVERLAP_ALWAYS ||
                              (mode == MOE_OVERLAP_AUTO && a.ffn_all_rows != 0));
  a.up_ready = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + ready_at);
  return hip_status(moe::launch_fused(a, dtype == MOE_BF16, max_rows, stream, fp8));
}

moe_status moe_set_fused_overlap(int mode) {
  if (mode != MOE_OVERLAP_NEVER && mode != MOE_OVERLAP_AUTO && mode != MOE_OVERLAP_ALWAYS)
    return MOE_ERR_INVALID_ARG;
  g_fused_overlap.store(mode, std::memory_order_relaxed);
  return MOE_OK;
}

moe_status moe_forward_fused(const float* logits, const void* x, int T, int E, int k, int gate,
                             int capacity, int e_begin, int e_end, int d, int f, moe_dtype dtype,
                             const void* w13_packed, const void* w2_packed, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos, int32_t* n_kept,
                             void* h, void* y_perm, void* y, void* ws, size_t ws_bytes,
                             void* stream) {
  return forward_fused_impl(logits, x, T, E, k, gate, capacity, e_begin, e_end, d, f, dtype,
                            w13_packed, w2_packed, topk_idx, topk_w, counts, offsets, sorted_pair,
                            pair_pos, n_kept, h, y_perm, y, ws, ws_bytes, stream, false);
}

moe_status moe_forward_fused_reroute(const float* logits, const void* x, int T, int E, int k,
                                     int gate, int capacity, int e_begin, int e_end, int d, int f,
                                     moe_dtype dtype, const void* w13_packed,
                                     const void* w2_packed, int32_t* topk_idx, float* topk_w,
                                     int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                     int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                     void* y, void* ws, size_t ws_bytes, void* stream) {
  return forward_fused_impl(logits, x, T, E, k, gate, capacity, e_begin, e_end, d, f, dtype,
                            w13_packed, w2_packed, topk_idx, topk_w, counts, offsets, sorted_pair,
                            pair_pos, n_kept, h, y_perm, y, ws, ws_bytes, stream, true);
}

moe_status moe_forward_fused_list(const float* logits, const void* x, int T, int E, int k,
                                  int gate, int capacity, int e_begin, int e_end, int d, int f,
                                  moe_dtype dtype, const void* const* w13_list,
                                  const void* const* w2_list, int32_t* topk_idx, float* topk_w,
                                  int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                  int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                  void* y, void* ws, size_t ws_bytes, void* stream) {
  if (!w13_list || !w2_list) return MOE_ERR_INVALID_ARG;
  return forward_fused_impl(logits, x, T, E, k, gate, capacity, e_begin, e_end, d, f, dtype,
                            nullptr, nullptr, topk_idx, topk_w, counts, offsets, sorted_pair,
                            pair_pos, n_kept, h, y_perm, y, ws, ws_bytes, stream, false, nullptr,
                            nullptr, w13_list, w2_list);
}

moe_status moe_forward_fused_fp8(const float* logits, const void* x, int T, int E, int k,
                                 int gate, int capacity, int e_begin, int e_end, int d, int f,
                                 const uint8_t* w13_q, const float* w13_s, const uint8_t* w2_q,
                                 const float* w2_s, int32_t* topk_idx, float* topk_w,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                 int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                 void* y, void* ws, size_t ws_bytes, void* stream) {
  if (!w13_s || !w2_s) return MOE_ERR_INVALID_ARG;
  return forward_fused_impl(logits, x, T, E, k, gate, capacity, e_begin, e_end, d, f, MOE_BF16,
                            w13_q, w2_q, topk_idx, topk_w, counts, offsets, sorted_pair, pair_pos,
                            n_kept, h, y_perm, y, ws, ws_bytes, stream, false, w13_s, w2_s);
}

moe_status moe_forward_fused_fp8_list(const float* logits, const void* x, int T, int E, int k,
                                      int gate, int capacity, int e_begin, int e_end, int d,
                                      int f, const void* const* w13_q_list,
                                      const float* const* w13_s_list,
                                      const void* const* w2_q_list,
                                      const float* const* w2_s_list, int32_t* topk_idx,
                                      float* topk_w, int32_t* counts, int32_t* offsets,
                                      int32_t* sorted_pair, int32_t* pair_pos, int32_t* n_kept,
                                      void* h, void* y_perm, void* y, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!w13_q_list || !w13_s_list || !w2_q_list || !w2_s_list) return MOE_ERR_INVALID_ARG;
  return forward_fused_impl(logits, x, T, E, k, gate, capacity, e_begin, e_end, d, f, MOE_BF16,
                            nullptr, nullptr, topk_idx, topk_w, counts, offsets, sorted_pair,
                            pair_pos, n_kept, h, y_perm, y, ws, ws_bytes, stream, false, nullptr,
                            nullptr, w13_q_list, w2_q_list, w13_s_list, w2_s_list);
}

}  // extern "C"
