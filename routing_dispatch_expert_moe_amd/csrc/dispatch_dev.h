// Dispatch plan (histogram, scan, stable positions, capacity) and the row
// permutation into the compact expert-major layout.
//
// ThunderEP page §2.1 and §2.2: every row bound for one owner is packed into
// one contiguous buffer, and each owner keeps the index list of its rows.
// NCCL EP page §2.2, layout table: compact [sum of rows x H] form.
// MoE sparse-activation page §2.3: per-expert load / capacity.
//
// Positions must be the stable (token-order) rank of each pair within its
// expert, bit-exactly.  Tokens are cut into blocks of 256; inside a block,
// each expert gets a 256-bit LDS bitmap of the tokens that chose it (LDS
// atomic OR: the result does not depend on arrival order).  A pair's rank in
// its block is the popcount of its expert's bitmap below the token, and the
// block's base for that expert comes from an expert-major scan over blocks.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kTB = kDispatchTokensPerBlock;  // tokens per block (256)
constexpr int kWords = kTB / 64;              // bitmap words per expert

// Build the block's bitmaps: bits[e * kWords + w] bit b <=> token t0 + 64w + b chose e.
// Invalid (out of range or repeated) entries raise the error word and are skipped.
__device__ __forceinline__ void build_bitmaps(unsigned long long* bits, const int32_t* idx, int T,
                                              int E, int k, int t0, int* err) {
  for (int i = threadIdx.x; i < E * kWords; i += blockDim.x) bits[i] = 0ull;
  __syncthreads();
  const int t1 = min(T, t0 + kTB);
  const int p0 = t0 * k, p1 = t1 * k;
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = idx[p];
    if (e < 0 || e >= E) {
      raise_error(err, MOE_ERR_INVALID_TOPK);
      continue;
    }
    const int lt = p / k - t0;
    const unsigned long long bit = 1ull << (lt & 63);
    const unsigned long long old = atomicOr(&bits[e * kWords + (lt >> 6)], bit);
    if (old & bit) raise_error(err, MOE_ERR_INVALID_TOPK);  // expert repeated in one row
  }
  __syncthreads();
}

// Count pass of token block vb: pairs per expert among the block's tokens.
// bits: LDS, E * kWords words.
__device__ __forceinline__ void dispatch_count_block(int vb, unsigned long long* bits,
                                                     const int32_t* __restrict__ idx, int T, int E,
                                                     int k, int* __restrict__ block_counts,
                                                     int* err) {
  const int t0 = vb * kTB;
  build_bitmaps(bits, idx, T, E, k, t0, err);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popcll(bits[e * kWords + w]);
    block_counts[(size_t)vb * E + e] = c;
  }
  __syncthreads();  // bits are rebuilt by the caller's next block
}

// Place pass of token block vb: each pair's row (or -1 dropped / -2 remote),
// for the block's tokens in [t_lo, t_hi) (the whole block by default).
// base[e]: pairs of expert e in the blocks before vb; offsets: local segment
// starts.  bits: LDS, E * kWords words.
__device__ __forceinline__ void dispatch_place_block(
    int vb, unsigned long long* bits, const int32_t* __restrict__ idx, int T, int E, int k,
    int capacity, int e_begin, int e_end, const int* base, const int32_t* offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos, int t_lo = 0,
    int t_hi = 0x7fffffff) {
  const int t0 = vb * kTB;
  // errors were already reported by the count pass; do not report twice
  build_bitmaps(bits, idx, T, E, k, t0, nullptr);
  const int p_lo = max(t0, t_lo) * k;
  const int p_hi = min(min(T, t0 + kTB), t_hi) * k;
  for (int p = p_lo + threadIdx.x; p < p_hi; p += blockDim.x) {
    const int e = idx[p];
    if (e < 0 || e >= E) {
      pair_pos[p] = -1;
      continue;
    }
    const int lt = p / k - t0;
    const int w = lt >> 6;
    int below = 0;
    for (int i = 0; i < w; ++i) below += __popcll(bits[e * kWords + i]);
    const unsigned long long lowmask = (lt & 63) ? ((1ull << (lt & 63)) - 1ull) : 0ull;
    below += __popcll(bits[e * kWords + w] & lowmask);
    const int pos = base[e] + below;
    const bool kept = capacity < 0 || pos < capacity;
    int out;
    if (!kept) {
      out = -1;
    } else if (e >= e_begin && e < e_end) {
      out = offsets[e - e_begin] + pos;
      sorted_pair[out] = p;
    } else {
      out = -2;
    }
    pair_pos[p] = out;
  }
  __syncthreads();  // bits are rebuilt by the caller's next block
}

// x_perm[row] = x[t] for every kept local pair of token t: one wave per token
// reads the token's row once (16-byte loads) and writes it to its <= k rows.
// U: 16-byte chunks per lane loaded before their stores; NT: streaming
// (non-temporal) stores
template <int U = 4, bool NT = false>
__device__ __forceinline__ void permute_token(const uint4* __restrict__ x, int t, int k, int chunks,
                                              const int32_t* __restrict__ pair_pos,
                                              uint4* __restrict__ x_perm) {
  const int lane = lane_id();
  int rows[MOE_MAX_K];
  bool any = false;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    rows[j] = j < k ? pair_pos[(size_t)t * k + j] : -1;
    any |= rows[j] >= 0;
  }
  if (!any) return;
  const uint4* src = x + (size_t)t * chunks;
  for (int c0 = lane; c0 < chunks; c0 += U * kWave) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * kWave < chunks) v[u] = src[c0 + u * kWave];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c >= chunks) break;
#pragma unroll
      for (int j = 0; j < MOE_MAX_K; ++j) {
        if (rows[j] < 0) continue;
        uint4* dst = x_perm + (size_t)rows[j] * chunks + c;
        if constexpr (NT) {
          typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(u32x4_nt{v[u].x, v[u].y, v[u].z, v[u].w},
                                      reinterpret_cast<u32x4_nt*>(dst));
        } else {
          *dst = v[u];
        }
      }
    }
  }
}

}  // namespace moe
