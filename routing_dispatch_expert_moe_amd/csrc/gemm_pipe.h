// Pipelined grouped GEMM (bf16 in, fp32 accumulation, v_mfma_f32_32x32x16_bf16)
// for the expert FFN halves.
//
// DWDP page, key optimisations: the first grouped GEMM takes every local
// expert's rows against its fused [W1 | W3] operand with SwiGLU in the
// epilogue; the second grouped GEMM applies W2.
//
// Tile: BM activation rows x BNW weight rows (SwiGLU: BNW/2 W1 rows + the
// matching W3 rows -> BNW/2 h columns).  NW waves split the tile 2 x NW/2;
// each wave owns (BM / 2) x (BNW / (NW/2)) in 32 x 32 MFMA tiles.
//   BM = BNW = 256, NW = 8: experts with many rows (MFMA-bound; two waves per
//             SIMD with 128 accumulators each, so one wave's waits are
//             covered by the other's MFMAs);
//   BM = 128, NW = 4: the short remainders, where the weights stream from
//             HBM and the smaller tile leaves LDS for a deeper pipeline.
//
// Memory pipeline: operands go HBM/L2 -> LDS directly (global_load_lds_dwordx4,
// no staging registers) in K-steps of 32 through STAGES LDS buffers, so loads
// run STAGES - 1 steps ahead of the MFMAs.  A step's loads are spread over the
// MFMAs of the step before; MFMA operands are double buffered in registers
// (the next 16-deep substep's LDS reads overlap the current substep's MFMAs),
// and each step's barrier sits under the last substep's MFMAs.  The load
// stream runs across tile boundaries, so the next tile's operands are in
// flight during the current tile's epilogue.  Rows are 64 bytes (4 chunks of
// 16 B); chunk c of row r sits at chunk c ^ ((r >> 2) & 3), so each 16-lane
// phase of a ds_read_b128 touches 16 distinct bank groups; the direct loads
// realise this by choosing which global chunk each lane fetches.
//
// Rows: the rows of row class CLASS of each expert (tile_sched.h).
//
// Scheduling: persistent grid (one workgroup per CU); tiles in expert order,
// M-tiles fastest so consecutive tiles share a weight tile; workgroup ids
// remapped so each XCD (ids dealt round-robin over 8 XCDs) owns contiguous
// tile ranges and shares weight tiles in its own L2.
#pragma once

#include <type_traits>

#include "common.h"
#include "tile_sched.h"

namespace moe {

namespace pipe {

constexpr int kBK = 32;          // K depth of one pipeline step
constexpr int kKC = kBK / 8;     // 16-byte chunks per 64-byte row
constexpr int kRPI = 64 / kKC;   // rows covered by one 64-lane 16-byte load (16)
constexpr int kSUB = kBK / 16;   // MFMA K-substeps per step (2)

__device__ __forceinline__ float silu_fast(float a) {
  return a * __builtin_amdgcn_rcpf(1.f + __expf(-a));
}

// s_waitcnt vmcnt(N) (N < 64) with the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// scheduling groups of one substep: MFMA g is followed by its share of the NDS
// LDS reads and of the NVM global loads (both evenly spread; the substep opens
// with an MFMA so the wait for its own operands never covers the new reads)
template <int G, int NMF, int NDS, int NVM>
__device__ __forceinline__ void interleave() {
  if constexpr (G < NMF) {
    constexpr int nds = ((G + 1) * NDS) / NMF - (G * NDS) / NMF;
    constexpr int nvm = ((G + 2) * NVM) / NMF - ((G + 1) * NVM) / NMF;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (nds > 0) __builtin_amdgcn_sched_group_barrier(0x100, nds, 0);
    if constexpr (nvm > 0) __builtin_amdgcn_sched_group_barrier(0x020, nvm, 0);
    interleave<G + 1, NMF, NDS, NVM>();
  }
}

struct Tile {
  int e, m0, seg1, n0;
};

template <int BM, int BN, int CLASS>
__device__ __forceinline__ Tile decode_tile(int t, int NT, const int* prefix, const int* segs,
                                            int E_loc) {
  Tile r;
  r.e = find_expert(prefix, E_loc, t / NT);
  const int mt_e = prefix[r.e + 1] - prefix[r.e];
  const int local = t - prefix[r.e] * NT;
  const int nt = local / mt_e, mti = local % mt_e;
  int first, count;
  class_rows<CLASS>(segs[r.e + 1] - segs[r.e], first, count);
  r.m0 = segs[r.e] + first + mti * BM;
  r.seg1 = segs[r.e] + first + count;
  r.n0 = nt * BN;
  // the tile is the same for the whole wave: keep its fields in scalar registers
  r.e = __builtin_amdgcn_readfirstlane(r.e);
  r.m0 = __builtin_amdgcn_readfirstlane(r.m0);
  r.seg1 = __builtin_amdgcn_readfirstlane(r.seg1);
  r.n0 = __builtin_amdgcn_readfirstlane(r.n0);
  return r;
}

}  // namespace pipe

using namespace pipe;

// dynamic LDS bytes of gemm_pipe_body<..., BM, BNW, STAGES, ...>
constexpr size_t pipe_lds_bytes(int BM, int BNW, int STAGES) {
  return static_cast<size_t>(STAGES) * (BM + BNW) * kBK * sizeof(uint16_t);
}

// One workgroup's share of the grouped GEMM: workgroup `bid` of `G` walks its
// tiles.  lds: pipe_lds_bytes(BM, BNW, STAGES); prefix, segs: E_loc + 1 ints
// of LDS each.  Every thread of the workgroup must call it (it has barriers).
// BNW weight rows per tile (256 or 128; SwiGLU: half W1, half W3).  NW waves
// (4 or 8: one or two per SIMD) split the tile 2 x NW/2.
// gather: if not null, activation row r is row gather[r] / gk of A (A rows
// read in place through the dispatch permutation instead of a permuted copy).
// wlist: if not null, expert e's packed weights start at wlist[e] (a table of
// per-expert buffers) instead of W + e * (weight rows * K).
// SAVE (SwiGLU only): the pre-activations are also stored, a = A W1 at
// AB[row][col] and g = A W3 at AB[row][N + col] (row pitch 2N), rounded to
// bf16, for the backward pass.
template <bool SWIGLU, int BM, int BNW, int STAGES, int CLASS, int NW = 4, bool SAVE = false>
__device__ __forceinline__ void gemm_pipe_body(const uint16_t* __restrict__ A,
                                               const int32_t* __restrict__ offsets, int E_loc,
                                               const uint16_t* __restrict__ W,
                                               uint16_t* __restrict__ C, int N, int K, int bid,
                                               int G, uint4* lds, int* prefix, int* segs,
                                               const int32_t* __restrict__ gather = nullptr,
                                               int gk = 1,
                                               const uint16_t* const* __restrict__ wlist = nullptr,
                                               uint16_t* __restrict__ AB = nullptr) {
  static_assert(SWIGLU || !SAVE, "pre-activations exist only with SwiGLU");
  constexpr int BN = SWIGLU ? BNW / 2 : BNW;  // output columns per tile
  constexpr int HALF = BNW / 2;               // SwiGLU: W1 rows (then as many W3 rows)
  constexpr int FM = BM / 64;                 // 32-row MFMA blocks per wave
  constexpr int WN = NW / 2;                  // waves along the weight rows (2 along M)
  constexpr int NQ = BNW / WN / 32;           // 32-column MFMA blocks per wave
  constexpr int LA = BM / kRPI / NW;          // A loads per wave per step
  constexpr int LB = BNW / kRPI / NW;         // B loads per wave per step
  constexpr int LSTEP = LA + LB;
  constexpr int STAGE_U4 = (BM + BNW) * kKC;
  static_assert(FM >= 1 && NQ >= 2 && LB % kSUB == 0, "unsupported tile");
  for (int i = threadIdx.x; i <= E_loc; i += blockDim.x) segs[i] = offsets[i];
  mtile_prefix<BM, CLASS>(offsets, E_loc, prefix);  // ends with a barrier
  const int NT = (N + BN - 1) / BN;
  const int total = prefix[E_loc] * NT;
  int vb = bid;
  if ((G & 7) == 0) vb = (bid & 7) * (G >> 3) + (bid >> 3);
  if (vb >= total) {
    __syncthreads();  // prefix / segs may be rewritten by the caller's next phase
    return;
  }
  const int ntiles = (total - vb + G - 1) / G;
  const int KT = K / kBK;
  const int S = ntiles * KT;  // this workgroup's K-steps over all its tiles

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and everything derived from it, such
  // as the M0 bases of the direct loads) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;
  // LDS swizzle: chunk c of row r is stored at c ^ swz(r); swz spreads the 16
  // rows read by one 16-lane ds_read_b128 phase over all bank groups
  auto swz = [](int r) { return (r >> 2) & 3; };
  // the chunk this lane fetches in every 16-row group it loads (row = g * 16 +
  // lane / 4, so swz(row) depends only on the lane)
  const int lkc = (lane % kKC) ^ swz(lane / kKC);
  const char* Ab = reinterpret_cast<const char*>(A);

  // ---- issue side: the tile whose operands are being fetched
  int it_tile = -1;
  const char* iWb = nullptr;
  uint32_t aoff[LA], boff[LB];
  auto set_issue_tile = [&](int j) {
    const Tile t = decode_tile<BM, BN, CLASS>(vb + j * G, NT, prefix, segs, E_loc);
    iWb = reinterpret_cast<const char*>(wlist != nullptr ? wlist[t.e] : W + t.e * wstride);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int rt = (i * NW + wave) * kRPI + lane / kKC;  // row within the tile
      int arow = min(t.m0 + rt, t.seg1 - 1);
      if (gather != nullptr) arow = gather[arow] / gk;
      aoff[i] = (static_cast<uint32_t>(arow) * K + lkc * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int rt = (i * NW + wave) * kRPI + lane / kKC;
      int wrow;
      if (SWIGLU) wrow = (rt / HALF) * N + min(t.n0 + rt % HALF, N - 1);
      else wrow = min(t.n0 + rt, N - 1);
      boff[i] = (static_cast<uint32_t>(wrow) * K + lkc * 8) * 2u;
    }
    it_tile = j;
  };
  // part p (of kSUB) of a step's loads into buffer buf
  auto issue_part = [&](int p, int buf, uint32_t koff) {
    uint4* As = lds + buf * STAGE_U4;
    uint4* Bs = As + BM * kKC;
#pragma unroll
    for (int i = p * LA / kSUB; i < (p + 1) * LA / kSUB; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(Ab + (aoff[i] + koff)),
          (__attribute__((address_space(3))) void*)(As + (i * NW + wave) * 64), 16, 0, 0);
#pragma unroll
    for (int i = p * LB / kSUB; i < (p + 1) * LB / kSUB; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(iWb + (boff[i] + koff)),
          (__attribute__((address_space(3))) void*)(Bs + (i * NW + wave) * 64), 16, 0, 0);
  };
  // byte offset along K of step p's operands, switching the issue tile when p
  // starts a new one; steps past the end re-fetch the last step (valid
  // addresses, result unused)
  auto issue_koff = [&](int p) -> uint32_t {
    if (p >= S) p = S - 1;
    const int j = p / KT, kt = p - j * KT;
    if (j != it_tile) set_issue_tile(j);
    return static_cast<uint32_t>(kt) * kBK * 2u;
  };

  // LDS fragments of substep ks of the step held in buffer `buf`
  bf16x8_t fa[2][FM], fb[2][NQ];
  auto load_frags = [&](int buf, int ks, int slot) {
    const uint4* As = lds + buf * STAGE_U4;
    const uint4* Bs = As + BM * kKC;
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < (FM > NQ ? FM : NQ); ++i) {
      if (i < FM) {
        const int r = wm * (BM / 2) + i * 32 + (lane & 31);
        fa[slot][i] = __builtin_bit_cast(bf16x8_t, As[r * kKC + (ch ^ swz(r))]);
      }
      if (i < NQ) {
        // SwiGLU: blocks [0, NQ/2) are this wave's W1 rows, [NQ/2, NQ) the
        // matching W3 rows
        const int q = SWIGLU ? ((i / (NQ / 2)) * HALF + wn * (HALF / WN) + (i % (NQ / 2)) * 32 +
                                (lane & 31))
                             : (wn * (BNW / WN) + i * 32 + (lane & 31));
        fb[slot][i] = __builtin_bit_cast(bf16x8_t, Bs[q * kKC + (ch ^ swz(q))]);
      }
    }
  };
  // Step p becomes readable: this wave's loads of step p are done once at most
  // the (STAGES - 2) younger steps' loads are outstanding (loads complete in
  // order) and its own LDS reads of the step before are done; the barrier then
  // publishes every wave's step-p data and frees the buffer of step p - 1.
  // The loads of step p + STAGES - 1 go into that buffer in kSUB parts: part 0
  // right after the barrier, the others during the first substeps of step p
  // (pk / pb hold the pending step's K offset and buffer meanwhile).
  uint32_t pk = 0u;
  int pb = 0;
  auto sync_and_issue = [&](int p) {
    wait_vmcnt<(STAGES - 2) * LSTEP>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    pk = issue_koff(p + STAGES - 1);
    pb = (p + STAGES - 1) % STAGES;
    issue_part(0, pb, pk);
  };

  // instruction interleave of one substep: FM * NQ MFMAs with the FM + NQ LDS
  // reads of the next substep and about LSTEP / kSUB global loads between them
  constexpr int NMF = FM * NQ, NDS = FM + NQ, NVM = (LSTEP + kSUB - 1) / kSUB;
  constexpr uint32_t kStepBytes = kBK * 2;  // K bytes of one step in a row

  auto mfma_substep = [&](f32x16_t (&acc)[FM][NQ], int slot) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][q], acc[i][q], 0, 0, 0);
  };
  auto epilogue = [&](const Tile& ct, f32x16_t (&acc)[FM][NQ]) {
    const int valid = min(BM, ct.seg1 - ct.m0);
    // registers -> global; D[m][n] of a 32x32 MFMA tile is in lane
    // n + 32 * ((m / 4) % 2), register 4 * (m / 8) + m % 4.  Stores address C
    // with a uniform base and 32-bit byte offsets (C is below 4 GiB), which
    // keeps the epilogue's address registers few.
    char* Cb = reinterpret_cast<char*>(C);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (wm * (BM / 2) + i * 32 >= valid) continue;
      const int row0 = ct.m0 + wm * (BM / 2) + i * 32 + 4 * (lane >> 5);
#pragma unroll
      for (int q = 0; q < (SWIGLU ? NQ / 2 : NQ); ++q) {
        const int col = ct.n0 + (SWIGLU ? wn * (HALF / WN) : wn * (BNW / WN)) + q * 32 + (lane & 31);
        const uint32_t base = (static_cast<uint32_t>(row0) * static_cast<uint32_t>(N) +
                               static_cast<uint32_t>(col)) * 2u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dm = 8 * (r >> 2) + (r & 3);
          float v = acc[i][q][r];
          if constexpr (SWIGLU) {
            const float g = acc[i][q + NQ / 2][r];
            if constexpr (SAVE) {
              if (row0 + dm < ct.seg1 && col < N) {
                const uint32_t ab = (static_cast<uint32_t>(row0 + dm) * static_cast<uint32_t>(2 * N) +
                                     static_cast<uint32_t>(col)) * 2u;
                char* ABb = reinterpret_cast<char*>(AB);
                *reinterpret_cast<uint16_t*>(ABb + ab) = f32_to_bf16(v);
                *reinterpret_cast<uint16_t*>(ABb + ab + static_cast<uint32_t>(N) * 2u) = f32_to_bf16(g);
              }
            }
            v = silu_fast(v) * g;
          }
          if (row0 + dm < ct.seg1 && col < N)
            *reinterpret_cast<uint16_t*>(Cb + (base + static_cast<uint32_t>(dm * N) * 2u)) =
                f32_to_bf16(v);
        }
      }
    }
  };

  if (KT >= STAGES) {
    // Straight-line steps: the issue side changes tile only at tile
    // boundaries (the last STAGES steps of tile j fetch the first STAGES steps
    // of tile j + 1), so a step has no branch and the compiler sees every
    // outstanding LDS read when it places its waits.
    set_issue_tile(0);
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
#pragma unroll
      for (int q = 0; q < kSUB; ++q) issue_part(q, p, p * kStepBytes);
    wait_vmcnt<(STAGES - 2) * LSTEP>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    pk = (STAGES - 1) * kStepBytes;
    pb = STAGES - 1;
    issue_part(0, pb, pk);
    load_frags(0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);

    for (int j = 0; j < ntiles; ++j) {
      const Tile ct = decode_tile<BM, BN, CLASS>(vb + j * G, NT, prefix, segs, E_loc);
      f32x16_t acc[FM][NQ];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[i][q] = f32x16_t{};
      // The K loop of one tile.  ACT = false: this wave's rows of the tile
      // are all past the segment (a tile less than half full), so it only
      // helps with the loads and barriers and leaves its SIMD's MFMA pipe to
      // the other wave there.
      auto run_tile = [&](auto act) {
        constexpr bool ACT = decltype(act)::value;
        // one step: substep 0 fetches substep 1's fragments and the second
        // half of the pending step's loads between its MFMAs; substep 1
        // makes step s + 1 readable (barrier), sends the first half of step
        // s + STAGES's loads into this step's buffer and fetches step
        // s + 1's first fragments
        auto substep0 = [&](int s) {
          if constexpr (ACT) load_frags(s % STAGES, 1, 1);
          issue_part(1, pb, pk);
          if constexpr (ACT) {
            mfma_substep(acc, 0);
            interleave<0, NMF, NDS, NVM>();
          }
          __builtin_amdgcn_sched_barrier(0);
        };
        auto substep1 = [&](int s, uint32_t koff_next) {
          wait_vmcnt<(STAGES - 2) * LSTEP>();
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          pk = koff_next;
          pb = s % STAGES;  // (s + STAGES) % STAGES
          issue_part(0, pb, pk);
          load_frags((s + 1) % STAGES, 0, 0);
          if constexpr (ACT) {
            mfma_substep(acc, 1);
            interleave<0, NMF, NDS, NVM>();
          }
          __builtin_amdgcn_sched_barrier(0);
        };
        const int s0 = j * KT;
        for (int kt = 0; kt < KT - STAGES; ++kt) {
          substep0(s0 + kt);
          substep1(s0 + kt, (kt + STAGES) * kStepBytes);
        }
        // The last STAGES steps fetch the next tile's first steps (after the
        // last tile: re-fetch this tile's last step, valid and unused).  The
        // first of them still sends the second half of this tile's last
        // step, so the issue side switches tiles between its two substeps.
        const bool more = j + 1 < ntiles;
        substep0(s0 + KT - STAGES);
        if (more) set_issue_tile(j + 1);
        substep1(s0 + KT - STAGES, more ? 0u : (KT - 1) * kStepBytes);
        for (int kt = KT - STAGES + 1; kt < KT; ++kt) {
          substep0(s0 + kt);
          substep1(s0 + kt, more ? (kt + STAGES - KT) * kStepBytes : (KT - 1) * kStepBytes);
        }
      };
      if constexpr (NW == 8) {
        if (wm * (BM / 2) < ct.seg1 - ct.m0) run_tile(std::true_type{});
        else run_tile(std::false_type{});
      } else {
        run_tile(std::true_type{});
      }
      epilogue(ct, acc);
    }
  } else {
    // short K (fewer steps than stages): the issue side may run several
    // tiles ahead, so it switches tiles step by step
    for (int p = 0; p < STAGES - 1; ++p) {
      const uint32_t ko = issue_koff(p);
#pragma unroll
      for (int q = 0; q < kSUB; ++q) issue_part(q, p % STAGES, ko);
    }
    sync_and_issue(0);
    for (int j = 0; j < ntiles; ++j) {
      const Tile ct = decode_tile<BM, BN, CLASS>(vb + j * G, NT, prefix, segs, E_loc);
      f32x16_t acc[FM][NQ];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[i][q] = f32x16_t{};
      load_frags((j * KT) % STAGES, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      for (int kt = 0; kt < KT; ++kt) {
        const int s = j * KT + kt;
        const int buf = s % STAGES;
        load_frags(buf, 1, 1);
        issue_part(1, pb, pk);
        mfma_substep(acc, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < S) sync_and_issue(s + 1);
        mfma_substep(acc, 1);
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < S && kt + 1 < KT) load_frags((s + 1) % STAGES, 0, 0);
      }
      epilogue(ct, acc);
    }
  }
  wait_vmcnt<0>();  // redundant tail loads must land before the LDS is released
  __syncthreads();
}

}  // namespace moe
