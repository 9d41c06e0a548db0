// Stand-alone launchers of the dispatch passes (dispatch_dev.h): count,
// expert-major scan (one workgroup), place, permute.
#include "dispatch_dev.h"

namespace moe {

size_t dispatch_ws_bytes(int T, int E) {
  const size_t nb = (static_cast<size_t>(T) + kTB - 1) / kTB;
  size_t b = kWsHeader + 2 * nb * static_cast<size_t>(E) * sizeof(int);
  return (b + 255) & ~static_cast<size_t>(255);
}

size_t reroute_ws_bytes(int T, int k) {
  const size_t n = static_cast<size_t>(T) * (k + 1);
  const size_t masks = (static_cast<size_t>(T) + 63) / 64 * sizeof(uint64_t);
  return 2 * ((n * 4 + 255) & ~static_cast<size_t>(255)) + ((masks + 255) & ~static_cast<size_t>(255));
}

size_t ready_ws_bytes(int E_loc) {
  return (static_cast<size_t>(E_loc) * sizeof(uint32_t) + 255) & ~static_cast<size_t>(255);
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

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int T, int E, int k,
                                                             int* __restrict__ block_counts,
                                                             int* err) {
  extern __shared__ unsigned long long bits[];
  dispatch_count_block(blockIdx.x, bits, idx, T, E, k, block_counts, err);
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
  constexpr int U = 4;  // block counts in flight per thread
  // P threads per expert each take a contiguous range of blocks: a first pass
  // sums each range (parts in scan_s), a second writes the running bases from
  // the sum of the ranges before it (integer sums: the same values in any order)
  const int P = E <= 512 ? min(16, static_cast<int>(blockDim.x) / E) : 1;
  const int e_t = threadIdx.x % E, p_t = threadIdx.x / E;
  const int per_b = (nb + P - 1) / P;
  const int b0 = p_t * per_b, b1 = min(nb, b0 + per_b);
  if (P > 1) {
    if (p_t < P) {
      int sum = 0;
      for (int b = b0; b < b1; b += U) {
        int c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) c[u] = b + u < b1 ? block_counts[(size_t)(b + u) * E + e_t] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) sum += c[u];
      }
      scan_s[p_t * E + e_t] = sum;
    }
    __syncthreads();
  }
  for (int e = P > 1 ? e_t : threadIdx.x; e < E && p_t < P; e += P > 1 ? E : blockDim.x) {
    const int lo = P > 1 ? b0 : 0, hi = P > 1 ? b1 : nb;
    int run = 0;
    for (int q = 0; q < p_t && P > 1; ++q) run += scan_s[q * E + e];
    for (int b = lo; b < hi; b += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = b + u < hi ? block_counts[(size_t)(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b + u < hi) {
          block_base[(size_t)(b + u) * E + e] = run;
          run += c[u];
        }
      }
    }
    if (P == 1 || p_t == P - 1) {  // the last part ends with the expert's total
      counts[e] = run;
      kept_s[e] = capacity < 0 ? run : min(run, capacity);
    }
  }
  __syncthreads();  // kept_s complete; scan_s free again
  // exclusive scan of kept_s[e_begin, e_end): each thread owns a contiguous run
  const int E_loc = e_end - e_begin;
  const int per = (E_loc + blockDim.x - 1) / blockDim.x;
  const int lo = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < E_loc) local += kept_s[e_begin + lo + i];
  // wave-level inclusive prefix sums of the per-thread sums (lane shuffles,
  // no barrier), then each wave adds the totals of the waves before it
  // (integers: exact)
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) scan_s[wv] = incl;  // wave totals
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += scan_s[w];
  int run = before + incl - local;
  for (int i = 0; i < per; ++i) {
    if (lo + i < E_loc) {
      offsets[lo + i] = run;
      run += kept_s[e_begin + lo + i];
    }
  }
  if (threadIdx.x == blockDim.x - 1) {
    offsets[E_loc] = before + incl;
    *n_kept = before + incl;
  }
}

__global__ __launch_bounds__(256) void dispatch_place_kernel(
    const int32_t* __restrict__ idx, int T, int E, int k, int capacity, int e_begin, int e_end,
    const int* __restrict__ block_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  extern __shared__ unsigned long long bits[];
  dispatch_place_block(blockIdx.x, bits, idx, T, E, k, capacity, e_begin, e_end,
                       block_base + (size_t)blockIdx.x * E, offsets, sorted_pair, pair_pos);
}

__global__ __launch_bounds__(256) void permute_rows_kernel(const uint4* __restrict__ x, int T,
                                                           int k, int chunks,
                                                           const int32_t* __restrict__ pair_pos,
                                                           uint4* __restrict__ x_perm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  permute_token<8, true>(x, t, k, chunks, pair_pos, x_perm);
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
                     e_begin, e_end, ws.block_base, offsets, sorted_pair, pair_pos);
  if (x != nullptr) {
    const int chunks = static_cast<int>((static_cast<size_t>(d) * elem_bytes) / 16);
    hipLaunchKernelGGL(permute_rows_kernel, dim3((T + 3) / 4), dim3(256), 0, s,
                       static_cast<const uint4*>(x), T, k, chunks, pair_pos,
                       static_cast<uint4*>(x_perm));
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
