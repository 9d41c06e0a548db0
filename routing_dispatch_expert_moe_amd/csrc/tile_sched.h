// Persistent per-expert tile scheduling shared by the grouped GEMMs.
//
// Every expert's rows form one segment of the expert-major activations.  The
// rows of a segment are split between the kernels that run them:
//   ROWS_ALL   every row (one kernel does the whole FFN half),
//   ROWS_BIG   the full 256-row blocks, plus a last partial block when it is
//              at least half full (large-tile kernel),
//   ROWS_TAIL  whatever ROWS_BIG leaves: a last block of fewer than 128 rows,
//              or all rows of an expert with fewer than 128 (small-tile kernel);
//   ROWS_BIGR / ROWS_TAILR  the same split for passes with many tiles, except
//              that an expert with at least one full block also takes its
//              short last block in the large tiles: that tile reads the weight
//              tiles the expert's full blocks stream anyway, where the
//              small-tile kernel would stream the expert's weights a second
//              time; the small tiles keep the experts with fewer than 128 rows.
// With this split no large tile runs less than half full, and skewed expert
// loads (a few experts with thousands of rows, most with tens) keep both
// kernels busy on useful rows.
#pragma once

#include "common.h"

namespace moe {

constexpr int kBigM = 256;     // rows per large tile
constexpr int kTailMax = 128;  // a last block below this many rows goes to the small tiles

enum RowClass { ROWS_ALL = 0, ROWS_BIG = 1, ROWS_TAIL = 2, ROWS_BIGR = 3, ROWS_TAILR = 4 };

constexpr bool is_tail_class(int c) { return c == ROWS_TAIL || c == ROWS_TAILR; }

// rows [first, first + count) of an n-row segment belong to class CLASS
template <int CLASS>
__device__ __forceinline__ void class_rows(int n, int& first, int& count) {
  if constexpr (CLASS == ROWS_ALL) {
    first = 0;
    count = n;
  } else {
    const int full = (n / kBigM) * kBigM;
    const int rem = n - full;
    constexpr bool ride = CLASS == ROWS_BIGR || CLASS == ROWS_TAILR;
    // rows [0, split) are large-tile rows
    const int split = (rem >= kTailMax || (ride && n >= kBigM)) ? n : full;
    if constexpr (!is_tail_class(CLASS)) {
      first = 0;
      count = split;
    } else {
      first = split;
      count = n - split;
    }
  }
}

// prefix[e] = number of M-tiles (BM rows of class CLASS) of experts before e,
// prefix[E_loc] = total.  Wave 0 does the scan; lanes own contiguous runs.
// Ends with a workgroup barrier.
template <int BM, int CLASS = ROWS_ALL>
__device__ __forceinline__ void mtile_prefix(const int32_t* __restrict__ offsets, int E_loc, int* prefix) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (E_loc + kWave - 1) / kWave;
    const int lo = lane * per;
    auto tiles = [&](int e) {
      int first, count;
      class_rows<CLASS>(offsets[e + 1] - offsets[e], first, count);
      return (count + BM - 1) / BM;
    };
    int local = 0;
    for (int i = 0; i < per; ++i)
      if (lo + i < E_loc) local += tiles(lo + i);
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
        run += tiles(e);
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
