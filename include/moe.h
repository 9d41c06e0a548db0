/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts expert path.
 *
 * One MoE layer on one GPU, as four asynchronous calls on one HIP stream:
 *
 *   moe_router_logits -> moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine
 *
 * plus moe_pack_weights (one-time weight re-layout) and moe_check_error, and
 * moe_forward_fused: route -> dispatch -> expert FFN -> combine in one launch.
 *
 * Sources of the operations (cited by page title and section):
 *   - MoE sparse-activation page ("大模型MoE稀疏激活原理与硬件适配实战"):
 *     §2.2 the three levels (route, load the chosen experts' weights, compute
 *     locally); §2.3 per-expert load / capacity; §3.1 router row of the table
 *     (logits in, top-k indices out); §3.2 stage 2 (rank the logits, take the
 *     top k); §5.3 scenario 3 (router kept in fp32).
 *   - NCCL EP page ("NCCL EP架构解析"): §1 long-lived group resources vs a
 *     per-batch handle (here: caller-owned workspace vs the dispatch plan that
 *     moe_combine reuses); §2.1 LL combine (weighted sum over the k experts);
 *     §2.2 layout table (compact expert-major rows); §5.1 error codes
 *     (invalid top-k index, runtime error).
 *   - DWDP page ("DWDP: 在NVL72上的高性能分布式权重数据并行"): key
 *     optimisations -- one grouped GEMM over all local experts with the row
 *     gather and SwiGLU fused, then a second grouped GEMM; W3/W1 packed as one
 *     first-layer operand; the operator takes the selected experts [T x k] and
 *     their final scales [T x k].
 *   - ThunderEP page (PCIe all-to-all scheduling on consumer GPUs): §2.1 pack
 *     every row bound for one owner into one contiguous buffer; §4.4 MoE
 *     tensors must be contiguous (misaligned addresses fault).
 *   - MegaMoE comparison page ("细粒度专家并行方案对比"): core differences §1,
 *     the single fused kernel with a wave pipeline (moe_forward_fused).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a device pointer owned by the caller (the
 *     library never allocates or frees on these paths), unless stated.
 *     Every pointer must be 16-byte aligned; tensors are dense row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return after host-side validation; the
 *     only call that waits is moe_check_error.
 *   - Validation failures return an error code and enqueue nothing.
 *     MOE_ERR_HIP means a launch failed; moe_last_hip_error() gives the code.
 *   - Element types: MOE_F32 (fp32 everywhere) or MOE_BF16 (bf16 storage,
 *     fp32 accumulation).  Router logits and gates are always fp32.
 *   - Results are bitwise reproducible run to run: no floating-point atomics
 *     are used anywhere; integer atomics only where order cannot matter.
 *   - Calls on one stream that share a workspace must not overlap in time
 *     with calls on other streams using the same workspace.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* a size, range or pointer argument is invalid        */
  MOE_ERR_INVALID_TOPK = 2,  /* k < 1, k > E, k > MOE_MAX_K, or (device-detected)
                                an expert index outside [0, E) or repeated in a row */
  MOE_ERR_UNSUPPORTED = 3,   /* a dtype / shape combination this build does not run */
  MOE_ERR_MISALIGNED = 4,    /* a pointer is not 16-byte aligned                    */
  MOE_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than moe_workspace_bytes  */
  MOE_ERR_HIP = 6            /* a HIP launch or runtime call failed                 */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  /* softmax over all experts, keep the top k, renormalise over the k; equal to
     a softmax over the k chosen logits (sparse-activation page §3.2 stage 2) */
  MOE_GATE_SOFTMAX_TOPK_RENORM = 0,
  /* sigmoid of each chosen logit, normalised to sum to 1 over the k chosen   */
  MOE_GATE_SIGMOID_TOPK_NORM = 1
} moe_gate;

#define MOE_MAX_K 8     /* largest top-k supported                          */
#define MOE_MAX_E 1024  /* largest number of (global) experts supported     */

/* Human-readable name of a status code (static storage, never NULL). */
const char* moe_status_string(int status);

/* hipError_t code of the last failed HIP call made by this library on the
 * calling host thread (0 if none). */
int moe_last_hip_error(void);

/* Bytes of workspace needed by moe_dispatch and moe_expert_ffn (and the
 * device error word read by moe_check_error) for T tokens, E global experts,
 * top-k k and E_loc local experts; it also holds the rerouting scratch and
 * the fused launch's per-expert readiness counters (E_loc words).  Returns 0
 * if the sizes are invalid.
 * The workspace must be zero-filled once before its first use; the library
 * keeps it consistent afterwards. */
size_t moe_workspace_bytes(int T, int E, int k, int E_loc);

/* Per-expert capacity C = ceil(cf * T * k / E) for a capacity factor given as
 * the exact fraction cf = cf_num / cf_den (MoE sparse-activation page §2.3:
 * per-expert load (Batch x SeqLen x K) / E, scaled by the capacity factor).
 * Returns -1 (no limit) if cf_num < 0, and -2 if an argument is invalid. */
int64_t moe_capacity(int T, int k, int E, int64_t cf_num, int64_t cf_den);

/* Number of rows that x_perm / h / y_perm must provide: min(T*k, E_loc*C)
 * when capacity C >= 0, else T*k. */
int64_t moe_max_rows(int T, int k, int E_loc, int capacity);

/* One-time re-layout of expert weights from the logical x.W layout
 *   w1, w3: [E_loc][d][f]      w2: [E_loc][f][d]
 * into the K-contiguous packed layout used by moe_expert_ffn:
 *   w13_packed: [E_loc][2f][d]  (rows 0..f-1: W1 transposed; f..2f-1: W3 transposed)
 *   w2_packed:  [E_loc][d][f]   (W2 transposed)
 * (DWDP page, key optimisations: W3 and W1 form one fused first-layer
 * operand; sparse-activation page §4.2 layer 2: each expert's weights
 * contiguous, re-ordered once at load.)  Outputs must not alias inputs. */
moe_status moe_pack_weights(const void* w1, const void* w3, const void* w2, int E_loc, int d,
                            int f, moe_dtype dtype, void* w13_packed, void* w2_packed,
                            void* stream);

/* Router logits (sparse-activation page §3.1 router row, §5.3 fp32 router):
 *   logits[t][e] = sum_i x[t][i] * w_gate[i][e]
 * x: [T][d] bf16; w_gate: [d][E] fp32; logits: [T][E] fp32 (output).
 * fp32 products and accumulation, each logit one fixed-order sum
 * (deterministic).  Requires d % 8 == 0, 1 <= E <= MOE_MAX_E. */
moe_status moe_router_logits(const void* x, const float* w_gate, int T, int d, int E,
                             float* logits, void* stream);

/* Top-k routing and gates (sparse-activation page §3.2 stage 2).
 * logits: [T][E] fp32, finite.  Outputs topk_idx [T][k] int32 (best first,
 * equal logits ordered by lower expert index, -0.0 == +0.0) and topk_w [T][k]
 * fp32 gate weights per `gate`.  Selection compares the fp32 logits exactly. */
moe_status moe_route(const float* logits, int T, int E, int k, int gate, int32_t* topk_idx,
                     float* topk_w, void* stream);

/* Top-k routing with capacity-overflow rerouting (sparse-activation page
 * §3.2, stage 3: when a token's best expert is already at its capacity
 * limit, the token takes the next expert after its k instead).  Tokens are
 * taken in index order; the load of an expert is the number of earlier
 * tokens whose final choice holds it.  If capacity >= 0, k < E and the best
 * expert's load has reached capacity, the best expert is replaced by the
 * (k+1)-th best and the other k - 1 stay.  Outputs as moe_route (final
 * experts best first, gates over the final k).  capacity = -1: plain routing.
 * Pass the same capacity to moe_dispatch, whose rule still drops pairs whose
 * expert is full (a replacement can be).  ws: moe_workspace_bytes(T, E, k, .)
 * bytes (the k + 1 candidates per token and a bit per token are kept there).
 * The rule is sequential in token order: one wave decides the tokens 64 at a
 * time; candidates and gates are computed for all tokens in parallel. */
moe_status moe_route_reroute(const float* logits, int T, int E, int k, int gate, int capacity,
                             int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                             void* stream);

/* Bytes of the library's fixed device scratch array (one per GPU, held until
 * the process ends) used by moe_route_reroute_noalloc. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)

/* moe_route_reroute for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, outputs and bits, with the rerouting
 * scratch (the k + 1 candidates per token and a bit per token) in the
 * library's fixed device array instead of a workspace.  It allocates nothing
 * and calls no allocating routine.  The scratch it needs,
 * 2 * ceil256(4 T (k + 1)) + ceil256(8 ceil(T / 64)) bytes, must not exceed
 * MOE_NOALLOC_SCRATCH_BYTES (about T (k + 1) <= 524000), else
 * MOE_ERR_WORKSPACE with nothing enqueued.  The array needs no clearing
 * (every call writes the scratch it reads before reading it), but every call
 * on one GPU uses that GPU's one array: calls that overlap in time on one GPU
 * (on different streams, or from different host threads) race and must be
 * serialised by the caller.  The first call on a device looks the array's
 * address up there (with that device current). */
moe_status moe_route_reroute_noalloc(const float* logits, int T, int E, int k, int gate,
                                     int capacity, int32_t* topk_idx, float* topk_w,
                                     void* stream);

/* Dispatch plan and permutation (ThunderEP page §2.1/§2.2: rows packed per
 * owner, per-expert index lists; NCCL EP page §2.2: compact expert-major
 * layout; sparse-activation page §2.3: capacity).
 * Pair p = t*k + j is token t's j-th choice e = topk_idx[t][j].  Its position
 * pos(p) is the number of tokens t' < t that chose e.  It is kept iff
 * capacity < 0 or pos(p) < capacity, and local iff e_begin <= e < e_end.
 * Outputs (int32, device):
 *   counts[E]            pairs per expert before any drop
 *   offsets[E_loc + 1]   exclusive scan of min(counts, capacity) over local experts
 *   sorted_pair[rows]    sorted_pair[offsets[e - e_begin] + pos(p)] = p for kept local p
 *                        (entries past n_kept are left untouched)
 *   pair_pos[T*k]        that row, -1 if dropped, -2 if kept but not local
 *   n_kept[1]            offsets[E_loc]
 *   x_perm[rows][d]      x_perm[row] = x[sorted_pair[row] / k] (skipped if x == NULL)
 * x / x_perm hold `dtype` elements; rows = moe_max_rows(T, k, E_loc, capacity).
 * An index outside [0, E) or repeated within a row sets the device error word
 * (see moe_check_error); such pairs are ignored. */
moe_status moe_dispatch(const int32_t* topk_idx, int T, int E, int k, int capacity,
                        int e_begin, int e_end, const void* x, int d, moe_dtype dtype,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                        int32_t* pair_pos, int32_t* n_kept, void* x_perm, void* ws,
                        size_t ws_bytes, void* stream);

/* Per-expert SwiGLU FFN as two grouped GEMMs over the expert-major rows
 * (DWDP page key optimisations: gather + grouped GEMM + SwiGLU, then grouped
 * GEMM; MegaMoE comparison page §1: two linear layers and SwiGLU):
 *   h[r]      = silu(x_perm[r] . W1_e) * (x_perm[r] . W3_e)   silu(a) = a*sigmoid(a)
 *   y_perm[r] = h[r] . W2_e          for rows r in [offsets[i], offsets[i+1]), e = local i
 * x_perm: [rows][d]; h: [rows][f] (output, scratch for the second GEMM);
 * y_perm: [rows][d] (output, not yet weighted); weights packed by
 * moe_pack_weights.  max_rows bounds offsets[E_loc] (moe_max_rows).
 * Requires d % 64 == 0 and f % 64 == 0 (bf16) or d % 4 == 0, f % 4 == 0 (f32).
 * Row counts are read on the device; nothing is synchronised with the host.
 * moe_ffn_up and moe_ffn_down are the two halves of moe_expert_ffn. */
moe_status moe_expert_ffn(const void* x_perm, const int32_t* offsets, int E_loc,
                          int64_t max_rows, int d, int f, moe_dtype dtype,
                          const void* w13_packed, const void* w2_packed, void* h, void* y_perm,
                          void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_up(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                      int d, int f, moe_dtype dtype, const void* w13_packed, void* h,
                      void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_down(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                        int d, int f, moe_dtype dtype, const void* w2_packed, void* y_perm,
                        void* ws, size_t ws_bytes, void* stream);

/* Kernels that one FFN half launches (DWDP page, key optimisations: one
 * grouped GEMM over all local experts, whose per-expert loads differ).  The
 * choice depends only on the sizes (row counts stay on the device): */
typedef enum {
  MOE_FFN_PLAN_NONE = 0,      /* max_rows == 0: nothing is launched                     */
  MOE_FFN_PLAN_F32 = 1,       /* fp32 grouped GEMM                                      */
  MOE_FFN_PLAN_STREAM = 2,    /* 32-row tiles over every row: few rows per expert       */
                              /* (at most 48 on average by max_rows / E_loc)            */
  MOE_FFN_PLAN_STREAM_WIDE_OPERANDS = 3, /* the same kernel because an operand --      */
                              /* max_rows x max(d, f) or one expert's weights, in bf16 -- */
                              /* reaches 4 GiB (the other kernels use 32-bit offsets)     */
  MOE_FFN_PLAN_WIDE = 4,      /* first half only: 128-row tiles of 256 weight rows over */
                              /* every row (few tiles, at most 512 rows per expert)     */
  MOE_FFN_PLAN_BIG_ALL = 5,   /* 256-row tiles over every row (few, short tiles)        */
  MOE_FFN_PLAN_BIG_TAIL = 6,  /* 256-row tiles over each expert's full blocks, 128-row  */
                              /* tiles over the remainders below 128 rows (few tiles,   */
                              /* K > 4096)                                              */
  MOE_FFN_PLAN_BIG_RIDE = 7   /* many tiles: 256-row tiles over every row of the experts */
                              /* with a full block, 128-row tiles over the experts with */
                              /* fewer than 128 rows                                    */
} moe_ffn_plan_t;

/* Host-only query (no GPU needed): the moe_ffn_plan_t value that moe_ffn_up
 * (half = 0) or moe_ffn_down / the backward dgrad GEMMs on the same sizes
 * (half = 1) use for max_rows rows, E_loc experts, d, f and dtype on a device
 * with cu_count compute units.  -1 if an argument is invalid. */
int moe_ffn_plan(int half, int64_t max_rows, int E_loc, int d, int f, int dtype, int cu_count);

/* moe_expert_ffn over a table of per-expert weight buffers instead of one
 * packed tensor (DWDP page, key optimisations and TensorList: the grouped
 * GEMM takes a list of weight buffers -- locally resident ones and ones
 * fetched from elsewhere -- so nothing is copied into one contiguous tensor).
 * w13_list / w2_list: device arrays of E_loc device pointers; entry i points
 * to local expert i's weights in the packed layout of moe_pack_weights
 * ([2f][d] for w13, [d][f] for w2), each buffer 16-byte aligned and alive
 * until the call's kernels have run.  The tables themselves are 16-byte
 * aligned.  Same operation, kernels and bits as moe_expert_ffn on packed
 * weights.  No workspace. */
moe_status moe_expert_ffn_list(const void* x_perm, const int32_t* offsets, int E_loc,
                               int64_t max_rows, int d, int f, moe_dtype dtype,
                               const void* const* w13_list, const void* const* w2_list, void* h,
                               void* y_perm, void* stream);
moe_status moe_ffn_up_list(const void* x_perm, const int32_t* offsets, int E_loc,
                           int64_t max_rows, int d, int f, moe_dtype dtype,
                           const void* const* w13_list, void* h, void* stream);
moe_status moe_ffn_down_list(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                             int d, int f, moe_dtype dtype, const void* const* w2_list,
                             void* y_perm, void* stream);

/* FP8 expert weights (NCCL EP page §2.1, expert-compute stage: FP8 compute
 * with a scale tensor).  The page fixes neither format nor scale shape; this
 * library uses E4M3-FN codes (OCP FP8, gfx950's FP8 type: bias 7, 3 mantissa
 * bits, largest magnitude 448, no infinities) and one fp32 scale per block of
 * 128 rows x 128 K-columns of each expert's packed weight matrix.
 *
 * moe_quantize_fp8: packed bf16 weights w_packed [E_loc][rows][K] (the
 * moe_pack_weights layout: rows = 2f, K = d for w13; rows = d, K = f for w2)
 * -> codes q [E_loc][rows][K] (uint8) and scales [E_loc][rows/128][K/128]
 * (fp32).  Per block: amax = max |w|; scale = the smallest power of two 2^e
 * with amax <= 448 * 2^e (1 for an all-zero block), so code * scale is
 * exactly a bf16 value and the block's largest code lies in [224, 448];
 * q = E4M3(w / scale) rounded to nearest even (saturating at +-448, which no
 * weight reaches).  rows and K must be multiples of 128
 * (MOE_ERR_UNSUPPORTED); pointers 16-byte aligned; outputs must not alias the
 * input.  One-time, like moe_pack_weights. */
moe_status moe_quantize_fp8(const void* w_packed, int E_loc, int rows, int K, uint8_t* q,
                            float* scales, void* stream);

/* moe_expert_ffn with FP8 weights: the same operation and row layout, bf16
 * activations (x_perm, h, y_perm) and fp32 accumulation, the weights being
 * code value * block scale (each turned into bf16 as the weight tile is
 * staged).  d and f must be multiples of 128.  No workspace. */
moe_status moe_expert_ffn_fp8(const void* x_perm, const int32_t* offsets, int E_loc,
                              int64_t max_rows, int d, int f, const uint8_t* w13_q,
                              const float* w13_s, const uint8_t* w2_q, const float* w2_s,
                              void* h, void* y_perm, void* stream);
moe_status moe_ffn_up_fp8(const void* x_perm, const int32_t* offsets, int E_loc, int64_t max_rows,
                          int d, int f, const uint8_t* w13_q, const float* w13_s, void* h,
                          void* stream);
moe_status moe_ffn_down_fp8(const void* h, const int32_t* offsets, int E_loc, int64_t max_rows,
                            int d, int f, const uint8_t* w2_q, const float* w2_s, void* y_perm,
                            void* stream);

/* The FP8 calls over per-expert buffers (DWDP page, key optimisations and
 * TensorList: the grouped GEMM takes a list of weight buffers, so experts
 * need not be one packed tensor; NCCL EP page §2.1: FP8 expert compute with
 * a scale tensor).  *_q_list and *_s_list: device tables of E_loc device
 * pointers; entry i of a code table points to expert i of moe_quantize_fp8's
 * codes ([2f][d] for w13, [d][f] for w2, uint8), entry i of a scale table to
 * expert i of its scales ([2f/128][d/128] resp. [d/128][f/128], fp32); every
 * buffer and table 16-byte aligned and alive until the call's kernels have
 * run.  Same kernels and bits as the packed FP8 calls.  A NULL table is
 * MOE_ERR_INVALID_ARG; other rules and errors as moe_expert_ffn_fp8.  No
 * workspace. */
moe_status moe_expert_ffn_fp8_list(const void* x_perm, const int32_t* offsets, int E_loc,
                                   int64_t max_rows, int d, int f,
                                   const void* const* w13_q_list, const float* const* w13_s_list,
                                   const void* const* w2_q_list, const float* const* w2_s_list,
                                   void* h, void* y_perm, void* stream);
moe_status moe_ffn_up_fp8_list(const void* x_perm, const int32_t* offsets, int E_loc,
                               int64_t max_rows, int d, int f, const void* const* w13_q_list,
                               const float* const* w13_s_list, void* h, void* stream);
moe_status moe_ffn_down_fp8_list(const void* h, const int32_t* offsets, int E_loc,
                                 int64_t max_rows, int d, int f, const void* const* w2_q_list,
                                 const float* const* w2_s_list, void* y_perm, void* stream);

/* Weighted combine (NCCL EP page §2.1, LL combine):
 *   y[t] = sum_{j=0..k-1, pair_pos[t*k+j] >= 0} topk_w[t][j] * y_perm[pair_pos[t*k+j]]
 * accumulated in fp32 in ascending j, rounded once to `dtype`; tokens with no
 * local kept pair get zero rows.  y: [T][d] (output).  topk_w may be NULL:
 * every weight is then 1 (the backward pass sums a token's input-gradient
 * rows this way). */
moe_status moe_combine(const void* y_perm, const int32_t* pair_pos, const float* topk_w, int T,
                       int k, int d, moe_dtype dtype, void* y, void* stream);

/* Waits for `stream`, then returns MOE_ERR_INVALID_TOPK if a kernel since the
 * last check saw an invalid expert index, MOE_ERR_HIP if the stream reported
 * an error or a moe_forward_fused barrier timed out, else MOE_OK.  Clears the
 * device flags it reports (and re-arms the fused barrier after a time-out). */
moe_status moe_check_error(void* ws, void* stream);

/* The whole layer -- moe_route, moe_dispatch, moe_expert_ffn, moe_combine --
 * as ONE persistent cooperative launch (MegaMoE comparison page, core
 * differences §1 and summary: one fused kernel for the MoE layer instead of a
 * chain of kernels; sparse-activation page §4.2 layer 1: router, top-k and
 * expert compute fused).  Every argument means what it means in those four
 * calls, and every output (topk_idx, topk_w, counts, offsets, sorted_pair,
 * pair_pos, n_kept, h, y_perm, y) is written with the same bits the four
 * calls produce.  No permuted copy of x is made: the first GEMM reads each row
 * of x in place through sorted_pair (DWDP page, key optimisations: the row
 * gather fused into the grouped GEMM), so there is no x_perm argument.
 * logits: [T][E] fp32 (moe_router_logits stays a separate call).  d, f and
 * the pointers obey the union of the four calls' rules; bf16 additionally
 * needs max(max_rows, T) * max(d, f) * 2 and 4 * f * d below 2^32 (else
 * MOE_ERR_UNSUPPORTED).  One workgroup per CU at most; phases are
 * separated by device-wide barriers whose words live in the workspace header
 * (zero-filled once, as for every call), so two fused calls that share a
 * workspace must not run concurrently.  The two GEMM phases may instead
 * overlap per expert (see moe_set_fused_overlap): a second-GEMM tile of
 * expert e starts once every first-GEMM tile of e is stored (a per-expert
 * counter in the workspace, released and acquired at device scope); that
 * needs a workspace of moe_workspace_bytes(T, E, k, e_end - e_begin) bytes,
 * and with a smaller one (at least the dispatch scratch) a barrier separates
 * them.  Both orders give the same bits.  A barrier or wait that does not
 * complete within seconds sets the device error word (see moe_check_error)
 * instead of hanging the GPU. */
moe_status moe_forward_fused(const float* logits, const void* x, int T, int E, int k, int gate,
                             int capacity, int e_begin, int e_end, int d, int f, moe_dtype dtype,
                             const void* w13_packed, const void* w2_packed, int32_t* topk_idx,
                             float* topk_w, int32_t* counts, int32_t* offsets,
                             int32_t* sorted_pair, int32_t* pair_pos, int32_t* n_kept,
                             void* h, void* y_perm, void* y, void* ws, size_t ws_bytes,
                             void* stream);

/* moe_forward_fused with the expert weights as per-expert buffers (DWDP page,
 * key optimisations: the grouped GEMM reads each expert's weights through a
 * TensorList, so experts need not be one packed tensor; MegaMoE comparison
 * page, core differences §1: the layer as one kernel).  w13_list and w2_list
 * are device tables of E_loc device pointers (the moe_expert_ffn_list
 * tables): expert i's buffers hold expert i of moe_pack_weights' outputs,
 * w13 [2f][d] and w2 [d][f], each 16-byte aligned.  Every output has the same
 * bits as moe_forward_fused on the same weights packed.  Other arguments,
 * rules and errors as moe_forward_fused; a NULL table is
 * MOE_ERR_INVALID_ARG. */
moe_status moe_forward_fused_list(const float* logits, const void* x, int T, int E, int k,
                                  int gate, int capacity, int e_begin, int e_end, int d, int f,
                                  moe_dtype dtype, const void* const* w13_list,
                                  const void* const* w2_list, int32_t* topk_idx, float* topk_w,
                                  int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                  int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                  void* y, void* ws, size_t ws_bytes, void* stream);

/* How moe_forward_fused (and its rerouting, FP8 and TensorList forms) orders its two GEMM
 * phases, for every later call in the process (default MOE_OVERLAP_AUTO):
 *   MOE_OVERLAP_NEVER   a device-wide barrier between them;
 *   MOE_OVERLAP_AUTO    per-expert waits where they measured faster: when
 *                       every row runs in 128-row tiles (at most 48 rows per
 *                       local expert on average), else the barrier;
 *   MOE_OVERLAP_ALWAYS  per-expert waits wherever they are possible (bf16,
 *                       both GEMM phases on the pipelined tiles, a workspace
 *                       of moe_workspace_bytes).
 * The waits let a second-GEMM tile start once its expert's first-GEMM tiles
 * are all stored (MegaMoE comparison page, core differences §1: the stages
 * of different experts overlap).  Every mode gives the same bits.  Returns
 * MOE_ERR_INVALID_ARG for any other value. */
#define MOE_OVERLAP_NEVER 0
#define MOE_OVERLAP_AUTO 1
#define MOE_OVERLAP_ALWAYS 2
moe_status moe_set_fused_overlap(int mode);

/* moe_forward_fused with moe_route_reroute's routing (sparse-activation page
 * §3.2 stage 3, capacity-overflow rerouting in token order) in place of
 * moe_route's: the same arguments (capacity drives both the rerouting and the
 * dispatch's drops) and the same bits as moe_route_reroute -> moe_dispatch ->
 * moe_expert_ffn -> moe_combine.  Inside the launch the candidates are taken
 * by every workgroup, workgroup 0 resolves who reroutes (the rule is
 * sequential) while the others wait at the next barrier, and the gates
 * follow.  ws: moe_workspace_bytes(T, E, k, .) bytes (it holds the rerouting
 * scratch after the dispatch scratch). */
moe_status moe_forward_fused_reroute(const float* logits, const void* x, int T, int E, int k,
                                     int gate, int capacity, int e_begin, int e_end, int d, int f,
                                     moe_dtype dtype, const void* w13_packed,
                                     const void* w2_packed, int32_t* topk_idx, float* topk_w,
                                     int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                     int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                     void* y, void* ws, size_t ws_bytes, void* stream);

/* moe_forward_fused with FP8 expert weights (NCCL EP page §2.1: FP8 expert
 * compute with a scale tensor; MegaMoE comparison page, core differences §1:
 * the layer as one kernel): w13_q / w2_q are the E4M3-FN codes and w13_s /
 * w2_s the fp32 128 x 128 block scales that moe_quantize_fp8 makes from
 * w13_packed / w2_packed; x, h, y_perm and y are bf16.  The GEMM phases run
 * the FP8 pipelined body of moe_expert_ffn_fp8 (codes in LDS, each MFMA
 * operand converted to its dequantised bf16 weights with the block's scale),
 * so the result has the same bits as moe_route -> moe_dispatch ->
 * moe_expert_ffn_fp8 -> moe_combine wherever those calls run their
 * pipelined kernels (more than 48 rows per expert on average).  Requires d
 * and f multiples of 128 and at least 256 (the pipeline's depth), else
 * MOE_ERR_UNSUPPORTED; the other arguments and errors as moe_forward_fused. */
moe_status moe_forward_fused_fp8(const float* logits, const void* x, int T, int E, int k,
                                 int gate, int capacity, int e_begin, int e_end, int d, int f,
                                 const uint8_t* w13_q, const float* w13_s, const uint8_t* w2_q,
                                 const float* w2_s, int32_t* topk_idx, float* topk_w,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                                 int32_t* pair_pos, int32_t* n_kept, void* h, void* y_perm,
                                 void* y, void* ws, size_t ws_bytes, void* stream);

/* moe_forward_fused_fp8 with the codes and block scales as per-expert
 * buffers (DWDP page, key optimisations and TensorList; the tables as in
 * moe_expert_ffn_fp8_list: entry i of w13_q_list / w13_s_list / w2_q_list /
 * w2_s_list points to expert i of moe_quantize_fp8's codes or scales, each
 * 16-byte aligned).  Same bits as moe_forward_fused_fp8 on the packed codes
 * and scales; a NULL table is MOE_ERR_INVALID_ARG, other rules and errors as
 * moe_forward_fused_fp8. */
moe_status moe_forward_fused_fp8_list(const float* logits, const void* x, int T, int E, int k,
                                      int gate, int capacity, int e_begin, int e_end, int d,
                                      int f, const void* const* w13_q_list,
                                      const float* const* w13_s_list,
                                      const void* const* w2_q_list,
                                      const float* const* w2_s_list, int32_t* topk_idx,
                                      float* topk_w, int32_t* counts, int32_t* offsets,
                                      int32_t* sorted_pair, int32_t* pair_pos, int32_t* n_kept,
                                      void* h, void* y_perm, void* y, void* ws, size_t ws_bytes,
                                      void* stream);

/* ------------------------------------------------------------------------
 * Backward pass (NCCL EP page §3.2, training adaptation: the backward step
 * reuses the forward's routing handle, sends the output gradient to the
 * experts through it, runs the experts' backward and brings the input
 * gradients back through the same handle).  Here the handle is the forward's
 * dispatch plan (offsets, pair_pos) and its saved tensors (x_perm, the
 * pre-activations ab, h, y_perm, topk_idx, topk_w).  What is computed is the
 * exact gradient of the forward layer at the given point with the routing
 * decisions (top-k sets, capacity drops, local/remote split) held fixed.
 * One training step on one stream:
 *
 *   forward : router_logits -> route -> dispatch -> ffn_up_train -> ffn_down -> combine
 *   backward: combine_backward -> gate_backward -> [router_backward]
 *             ffn_down_backward -> ffn_up_backward -> combine(topk_w = NULL) -> dx
 *             ffn_wgrad (dW13, dW2)
 *
 * Rounding points: do_perm, dh, dab, dx_perm and dx are stored in the layer
 * dtype (fp32 accumulation inside each call); dgate, dlogits, the weight
 * gradients and dW_g are fp32.  Conventions as above (caller-owned, 16-byte
 * aligned device buffers; nothing is allocated; host validation first).
 * ------------------------------------------------------------------------ */

/* moe_ffn_up with the pre-activations kept for the backward pass: h as
 * moe_ffn_up, and ab [max_rows][2f] (layer dtype): row r holds a = x W1 in
 * columns [0, f) and g = x W3 in [f, 2f) (before SwiGLU; bf16: rounded from
 * the same fp32 sums that h is computed from).  bf16 needs max_rows * 2f * 2,
 * max_rows * d * 2 and 4 * f * d below 2^32 (else MOE_ERR_UNSUPPORTED). */
moe_status moe_ffn_up_train(const void* x_perm, const int32_t* offsets, int E_loc,
                            int64_t max_rows, int d, int f, moe_dtype dtype,
                            const void* w13_packed, void* h, void* ab, void* stream);

/* The first FFN half's backward operand: w13_t [E_loc][d][2f] with row c =
 * W1[e][c][0..f) followed by W3[e][c][0..f) (w1, w3: [E_loc][d][f], the
 * layout moe_pack_weights reads).  The second half's backward operand is W2
 * itself, [E_loc][f][d], so it needs no re-layout.  f * elem_bytes must be a
 * multiple of 16. */
moe_status moe_pack_weights_backward(const void* w1, const void* w3, int E_loc, int d, int f,
                                     moe_dtype dtype, void* w13_t, void* stream);

/* Backward of moe_combine.  dy: [T][d] (layer dtype).  For every pair p =
 * t*k + j with a local row r = pair_pos[p] >= 0:
 *   do_perm[r]  = topk_w[t][j] * dy[t]            (rounded once to dtype)
 *   dgate[t][j] = sum_c dy[t][c] * y_perm[r][c]    (fp32)
 * Pairs without a local row get dgate 0 (their gradient, if remote, comes
 * from the rank that holds the expert) and no do_perm row.  y_perm: the
 * forward's unweighted expert outputs.  do_perm rows not named by pair_pos
 * are left untouched. */
moe_status moe_combine_backward(const void* dy, const void* y_perm, const int32_t* pair_pos,
                                const float* topk_w, int T, int k, int d, moe_dtype dtype,
                                void* do_perm, float* dgate, void* stream);

/* Backward of the gate functions of moe_route / moe_route_reroute: dlogits
 * [T][E] fp32 from dgate [T][k], with the gates recomputed from the chosen
 * logits (the experts in topk_idx):
 *   softmax-renorm: dl_j = w_j (dg_j - sum_i w_i dg_i)
 *   sigmoid-norm:   dl_j = s_j (1 - s_j) (dg_j - sum_i w_i dg_i) / sum_i s_i
 * and 0 for every expert not chosen (the selection is piecewise constant). */
moe_status moe_gate_backward(const float* logits, const int32_t* topk_idx, const float* dgate,
                             int T, int E, int k, int gate, float* dlogits, void* stream);

/* Backward through the second FFN half and SwiGLU: dh = do_perm . W2^T per
 * expert segment (the down GEMM with the roles of d and f swapped; w2_t =
 * W2 in its logical layout [E_loc][f][d]), then from the saved
 * pre-activations ab (moe_ffn_up_train), with s = sigmoid(a):
 *   da = dh * g * s * (1 + a (1 - s)),   dg = dh * a * s
 * written as dab [max_rows][2f] (da then dg).  dh: [max_rows][f] (output).
 * Shape rules as moe_ffn_down. */
moe_status moe_ffn_down_backward(const void* do_perm, const int32_t* offsets, int E_loc,
                                 int64_t max_rows, int d, int f, moe_dtype dtype,
                                 const void* w2_t, const void* ab, void* dh, void* dab,
                                 void* stream);

/* Input gradient of the first FFN half: dx_perm = dab . [W1 | W3]^T per expert
 * segment, i.e. da W1^T + dg W3^T (w13_t from moe_pack_weights_backward).
 * dx_perm: [max_rows][d] (output).  moe_combine(dx_perm, pair_pos, NULL, ...)
 * then gives each token's dx. */
moe_status moe_ffn_up_backward(const void* dab, const int32_t* offsets, int E_loc,
                               int64_t max_rows, int d, int f, moe_dtype dtype,
                               const void* w13_t, void* dx_perm, void* stream);

/* Expert weight gradients, in the packed layouts of the forward weights, fp32:
 *   dw13[e] [2f][d]: rows n < f are dW1^T (dW1 = x_perm_e^T da_e), rows
 *                    f + n are dW3^T (dW3 = x_perm_e^T dg_e)
 *   dw2[e]  [d][f]:  dW2^T (dW2 = h_e^T do_e)
 * summed over each expert's rows (offsets); an expert with no rows gets
 * zeros.  x_perm [max_rows][d], h [max_rows][f], do_perm [max_rows][d], dab
 * [max_rows][2f] in the layer dtype.  ws: moe_wgrad_workspace_bytes bytes
 * (bf16: the operands transposed so the reduction over rows runs along
 * memory; fp32: a small segment table).  Shape rules as moe_expert_ffn. */
size_t moe_wgrad_workspace_bytes(int64_t max_rows, int E_loc, int d, int f, moe_dtype dtype);
moe_status moe_ffn_wgrad(const void* x_perm, const void* h, const void* do_perm, const void* dab,
                         const int32_t* offsets, int E_loc, int64_t max_rows, int d, int f,
                         moe_dtype dtype, float* dw13, float* dw2, void* ws, size_t ws_bytes,
                         void* stream);

/* Backward of moe_router_logits (sparse-activation page §3.1 router row, §5.3
 * fp32 router): with dlogits [T][E] fp32,
 *   dx[t][c]   += sum_e dlogits[t][e] * w_gate[c][e]   (fp32 sum added to dx's
 *                 value, rounded once more to dtype)
 *   dw_gate[c][e] = sum_t x[t][c] * dlogits[t][e]      (fp32, fixed order)
 * E <= 64, d a multiple of 8.  ws: moe_router_backward_workspace_bytes bytes
 * (per-64-token partial sums of dw_gate, added in order: no atomics). */
size_t moe_router_backward_workspace_bytes(int T, int d, int E);
moe_status moe_router_backward(const void* x, const float* w_gate, const float* dlogits, int T,
                               int d, int E, moe_dtype dtype, void* dx, float* dw_gate, void* ws,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
