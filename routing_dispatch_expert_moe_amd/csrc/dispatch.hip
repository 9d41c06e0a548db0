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
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kTB = kDispatchTokensPerBlock;  // tokens per block (256)
constexpr int kWords = kTB / 64;              // bitmap words per expert

size_t dispatch_ws_bytes(int T, int E) {
  const size_t nb = (static_cast<size_t>(T) + kTB - 1) / kTB;
  size_t b = kWsHeader + 2 * nb * static_cast<size_t>(E) * sizeof(int);
  return (b + 255) & ~static_cast<size_t>(255);
}

DispatchWs dispatch_ws(void* ws, int T, int E) {
  const size_t nb = (static_cast<size_t>(T) + kTB - 1) / kTB;
  char* p = static_cast<char*>(ws);
  DispatchWs w;
  w.err = reinterpret_cast<int*>(p);
  w.block_counts = reinterpret_cast<int*>(p + kWsHeader);
  w.block_base = w.block_counts + nb * E;
  return w;
}

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

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int T, int E, int k,
                                                             int* __restrict__ block_counts,
                                                             int* err) {
  extern __shared__ unsigned long long bits[];
  const int t0 = blockIdx.x * kTB;
  build_bitmaps(bits, idx, T, E, k, t0, err);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWords; ++w) c += __popcll(bits[e * kWords + w]);
    block_counts[(size_t)blockIdx.x * E + e] = c;
  }
}

// One workgroup: expert-major scan over blocks, capacity, local offsets.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int* __restrict__ block_counts,
                                                             int nb, int E, int capacity,
                                                             int e_begin, int e_end,
                                                             int* __restrict__ block_base,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ n_kept) {
  __shared__ int kept_s[MOE_MAX_E];
  __shared__ int scan_s[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nb; ++b) {
      block_base[(size_t)b * E + e] = run;
      run += block_counts[(size_t)b * E + e];
    }
    counts[e] = run;
    kept_s[e] = capacity < 0 ? run : min(run, capacity);
  }
  __syncthreads();
  // exclusive scan of kept_s[e_begin, e_end): each thread owns a contiguous run
  const int E_loc = e_end - e_begin;
  const int per = (E_loc + blockDim.x - 1) / blockDim.x;
  const int lo = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < E_loc) local += kept_s[e_begin + lo + i];
  scan_s[threadIdx.x] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums (integers: exact)
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    int v = threadIdx.x >= off ? scan_s[threadIdx.x - off] : 0;
    __syncthreads();
    scan_s[threadIdx.x] += v;
    __syncthreads();
  }
  int run = scan_s[threadIdx.x] - local;
  for (int i = 0; i < per; ++i) {
    if (lo + i < E_loc) {
      offsets[lo + i] = run;
      run += kept_s[e_begin + lo + i];
    }
  }
  if (threadIdx.x == blockDim.x - 1) {
    offsets[E_loc] = scan_s[threadIdx.x];
    *n_kept = scan_s[threadIdx.x];
  }
}

__global__ __launch_bounds__(256) void dispatch_place_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int capacity, int e_begin, int e_end,
    const int* __restrict__ block_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos, int* err) {
  extern __shared__ unsigned long long bits[];
  const int t0 = blockIdx.x * kTB;
  // errors were already reported by the count pass; do not report twice
  build_bitmaps(bits, idx, T, E, k, t0, nullptr);
  const int t1 = min(T, t0 + kTB);
  const int* base = block_base + (size_t)blockIdx.x * E;
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += blockDim.x) {
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
}

// x_perm[row] = x[t] for every kept local pair of token t: one wave per token
// reads the token's row once (16-byte loads) and writes it to its <= k rows.
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint4* __restrict__ x, int T,
                                                           int k, int chunks,
                                                           const int32_t* __restrict__ pair_pos,
                                                           uint4* __restrict__ x_perm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
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
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 v = src[c];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j)
      if (rows[j] >= 0) x_perm[(size_t)rows[j] * chunks + c] = v;
  }
}

int launch_dispatch(const int32_t* idx, int T, int E, int k, int capacity, int e_begin,
                    int e_end, const void* x, int d, int elem_bytes, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, int32_t* n_kept,
                    void* x_perm, const DispatchWs& ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = (T + kTB - 1) / kTB;
  const size_t lds = static_cast<size_t>(E) * kWords * sizeof(unsigned long long);
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nb), dim3(256), lds, s, idx, T, E, k,
                     ws.block_counts, ws.err);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, ws.block_counts, nb, E,
                     capacity, e_begin, e_end, ws.block_base, counts, offsets, n_kept);
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(nb), dim3(256), lds, s, idx, T, E, k, capacity,
                     e_begin, e_end, ws.block_base, offsets, sorted_pair, pair_pos, ws.err);
  if (x != nullptr) {
    const int chunks = static_cast<int>((static_cast<size_t>(d) * elem_bytes) / 16);
    hipLaunchKernelGGL(permute_rows_kernel, dim3((T + 3) / 4), dim3(256), 0, s,
                       static_cast<const uint4*>(x), T, k, chunks, pair_pos,
                       static_cast<uint4*>(x_perm));
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
