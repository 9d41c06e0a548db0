// Persistent per-expert tile scheduling shared by the grouped GEMMs.
#pragma once

#include "common.h"

namespace moe {

// prefix[e] = number of M-tiles of experts before e (exclusive), prefix[E_loc] = total.
// Wave 0 does the scan; lanes own contiguous runs.
template <int BM>
__device__ __forceinline__ void mtile_prefix(const int32_t* __restrict__ offsets, int E_loc, int* prefix) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (E_loc + kWave - 1) / kWave;
    const int lo = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = lo + i;
      if (e < E_loc) {
        const int n = offsets[e + 1] - offsets[e];
        local += (n + BM - 1) / BM;
      }
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int v = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += v;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int e = lo + i;
      if (e < E_loc) {
        prefix[e] = run;
        const int n = offsets[e + 1] - offsets[e];
        run += (n + BM - 1) / BM;
      }
    }
    if (lane == kWave - 1) prefix[E_loc] = incl;
  }
  __syncthreads();
}

__device__ __forceinline__ int find_expert(const int* prefix, int E_loc, int mt) {
  // largest e with prefix[e] <= mt (prefix is non-decreasing; empty experts repeat values)
  int lo = 0, hi = E_loc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
