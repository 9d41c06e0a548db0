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
// no staging registers) in K-steps of BK (32 or 64) through STAGES LDS
// buffers, so loads run STAGES - 1 steps ahead of the MFMAs.  A step's loads
// go out in two parts, right after the barrier that frees their buffer and
// during the first substep; MFMA operands are double buffered in registers
// (the next 16-deep substep's LDS reads overlap the current substep's MFMAs),
// and each step's barrier sits under the last substep's MFMAs.  The load
// stream runs across tile boundaries, so the next tile's operands are in
// flight during the current tile's epilogue.  A step's row is BK * 2 bytes in
// 16-byte chunks; chunk c of row r sits at chunk c ^ swz(r) (BK = 32: 4
// chunks, swz = (r >> 2) & 3; BK = 64: 8 chunks, swz = (r >> 1) & 7), so each
// 16-lane phase of a ds_read_b128 touches 16 distinct bank groups; the direct
// loads realise this by choosing which global chunk each lane fetches.  With
// BK = 64 one load instruction covers 8 rows x 128 bytes, whole 128-byte
// lines, where BK = 32 covers 16 rows x half a line: on gfx950 the whole-line
// pattern keeps the MFMA pipes measurably busier with the same bytes in
// flight, and halves the barriers per K.
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

constexpr int kBK = 32;          // K depth of one pipeline step (default; FP8 weights)
constexpr int kKC = kBK / 8;     // 16-byte chunks per 64-byte row
constexpr int kRPI = 64 / kKC;   // rows covered by one 64-lane 16-byte load (16)
constexpr int kSUB = kBK / 16;   // MFMA K-substeps per step (2)

// LDS row swizzle of a step with KC 16-byte chunks per row: chunk c of row r
// at c ^ swz(r), so 16 consecutive rows read at one chunk cover all 16
// 16-byte bank groups of a 256-byte bank row
template <int KC>
__device__ __forceinline__ int step_swz(int r) {
  static_assert(KC == 4 || KC == 8, "64- or 128-byte rows");
  return KC == 4 ? (r >> 2) & 3 : (r >> 1) & 7;
}

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

// dynamic LDS bytes of gemm_pipe_body<..., BM, BNW, STAGES, ..., BK> (FP8W:
// the weight rows of a step are 32 one-byte codes instead of 32 bf16 values)
// Output staging of the 8-wave 256-row bf16 tiles: one 32 x 32 bf16 block per
// wave, rows padded to 80 bytes (16-byte aligned reads, at most 2-way bank
// conflicts on the 8-byte writes)
constexpr int kOutRowBytes = 80;
constexpr size_t kOutStageBytes = static_cast<size_t>(8) * 32 * kOutRowBytes;

constexpr size_t pipe_lds_bytes(int BM, int BNW, int STAGES, bool fp8w = false, int BK = kBK) {
  return static_cast<size_t>(STAGES) * (BM + (fp8w ? BNW / 2 : BNW)) * BK * sizeof(uint16_t) +
         (BM == 256 && !fp8w ? kOutStageBytes : 0);
}

// One workgroup's share of the grouped GEMM: workgroup `bid` of `G` walks its
// tiles.  lds: pipe_lds_bytes(BM, BNW, STAGES); prefix, segs: E_loc + 1 ints
// of LDS each.  Every thread of the workgroup must call it (it has barriers).
// BNW weight rows per tile (256 or 128; SwiGLU: half W1, half W3).  NW waves
// (4 or 8: one or two per SIMD) split the tile 2 x NW/2.
// gather: if not null, activation row r is row gather[r] / gk of A (A rows
// read in place through the dispatch permutation instead of a permuted copy).
// wlist: if not null, expert e's packed weights (FP8W: codes) start at
// wlist[e] (a table of per-expert buffers) instead of W + e * (weight rows * K);
// slist (FP8W): if not null, expert e's block scales start at slist[e]
// instead of Ws + e * (rows / 128) * (K / 128).
// SAVE (SwiGLU only): the pre-activations are also stored, a = A W1 at
// AB[row][col] and g = A W3 at AB[row][N + col] (row pitch 2N), rounded to
// bf16, for the backward pass.
// FP8W: W holds E4M3 codes (one byte per weight, same packed layout) and Ws
// one fp32 power-of-two scale per 128 x 128 block ([E][rows / 128][K / 128])
// (NCCL EP page §2.1: FP8 expert compute with a scale tensor).  The codes go
// to LDS as they are (half the bytes of bf16 weights); each MFMA operand is
// converted from 8 codes to the 8 dequantised bf16 weights code x scale by
// the hardware's scaled conversion just before the MFMAs that use it (exact:
// an E4M3 value times a power of two is a bf16 value; a 32 x 32 tile's
// weight rows lie in one 128-row block, so each operand has one scale per
// 128-deep K block), so the MFMAs accumulate the dequantised weights'
// products in fp32 as the bf16 path does, with no rescaling of the
// accumulators.  K must be at least STAGES steps deep and a multiple of 128.  A weight row of a step is BK
// bytes of codes in 16-byte pieces fetched by BK / 16 neighbouring lanes (a
// 64-lane direct load covers 32 rows for BK = 32, 16 rows for BK = 64); in
// LDS piece c of row r sits at position c ^ fswz(r) of the row (BK = 32:
// (r >> 3) & 1; BK = 64: (r >> 2) & 3), so the 16 rows one 16-lane phase of a
// fragment read touches cover every bank once.
// BK: K depth of a pipeline step, 32 or 64 (64 needs K a multiple of 64).
// ready_out (producer): once all its tiles are stored, the workgroup releases
// them at agent scope (one release: a release per tile writes the L2 back
// every time and measured far slower) and adds each tile's rows x (output
// columns / 32) to ready_out[e], so expert e's counter reaches n_e * N / 32
// once every workgroup holding a tile of e, of any row class, is done.  ready_in (consumer, the next GEMM
// whose A is that output): before a wave issues the loads of a tile of
// expert e it waits until ready_in[e] reaches n_e * K / 32 and then
// acquires at agent scope (once per run of tiles of one expert); a wait that
// does not end within the spin limit sets MOE_ERR_HIP in err and goes on.
// Both need N and K multiples of 32.
template <bool SWIGLU, int BM, int BNW, int STAGES, int CLASS, int NW = 4, bool SAVE = false,
          bool FP8W = false, int BK = kBK>
__device__ __forceinline__ void gemm_pipe_body(const uint16_t* __restrict__ A,
                                               const int32_t* __restrict__ offsets, int E_loc,
                                               const uint16_t* __restrict__ W,
                                               uint16_t* __restrict__ C, int N, int K, int bid,
                                               int G, uint4* lds, int* prefix, int* segs,
                                               const int32_t* __restrict__ gather = nullptr,
                                               int gk = 1,
                                               const uint16_t* const* __restrict__ wlist = nullptr,
                                               uint16_t* __restrict__ AB = nullptr,
                                               const float* __restrict__ Ws = nullptr,
                                               uint32_t* ready_out = nullptr,
                                               const uint32_t* ready_in = nullptr,
                                               int* err = nullptr,
                                               const float* const* __restrict__ slist = nullptr) {
  static_assert(SWIGLU || !SAVE, "pre-activations exist only with SwiGLU");
  static_assert(!FP8W || !SAVE, "FP8 weights have no training forward");
  static_assert(BK == 32 || BK == 64, "step depth");
  constexpr int FPR = BK / 16;                // FP8W: 16-byte code pieces per weight row and step
  constexpr int KC = BK / 8;                  // 16-byte chunks per row per step
  constexpr int RPI = 64 / KC;                // rows covered by one 64-lane load
  constexpr int SUB = BK / 16;                // MFMA K-substeps per step
  constexpr int BN = SWIGLU ? BNW / 2 : BNW;  // output columns per tile
  constexpr int HALF = BNW / 2;               // SwiGLU: W1 rows (then as many W3 rows)
  constexpr int FM = BM / 64;                 // 32-row MFMA blocks per wave
  constexpr int WN = NW / 2;                  // waves along the weight rows (2 along M)
  constexpr int NQ = BNW / WN / 32;           // 32-column MFMA blocks per wave
  constexpr int LA = BM / RPI / NW;           // A loads per wave per step
  // B loads per wave per step (FP8W: 64 lanes x 16 codes cover 64 / FPR rows)
  constexpr int LB = FP8W ? BNW * FPR / 64 / NW : BNW / RPI / NW;
  constexpr int LSTEP = LA + LB;
  constexpr int BROW_U4 = FP8W ? FPR : KC;    // 16-byte chunks per weight row per step
  constexpr int STAGE_U4 = BM * KC + BNW * BROW_U4;
  // (SwiGLU: a wave's blocks are W1 blocks and the matching W3 blocks, so at
  // least two; 128 x 128 tiles with 8 waves give the other pass one)
  static_assert(FM >= 1 && NQ >= (SWIGLU ? 2 : 1) && LB >= 1 && (FP8W || LB % 2 == 0),
                "unsupported tile");
  static_assert((STAGES - 2) * LSTEP < 64, "outstanding loads exceed the vmcnt range");
  // 256-row bf16 tiles stage each 32 x 32 output block through LDS (the
  // bytes after the pipeline stages, pipe_lds_bytes) so that every store
  // writes whole 64-byte row segments
  constexpr bool STAGE_OUT = BM == 256 && !FP8W && !SAVE;
  static_assert(!(BM == 256 && !FP8W) || NW == 8, "the output staging holds 8 waves' blocks");
  static_assert(!FP8W || (BNW * FPR) % (64 * NW) == 0, "FP8 weight loads must tile the step");
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
  const int KT = K / BK;
  const int S = ntiles * KT;  // this workgroup's K-steps over all its tiles

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and everything derived from it, such
  // as the M0 bases of the direct loads) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const size_t wstride = static_cast<size_t>(SWIGLU ? 2 * N : N) * K;
  // LDS swizzle: chunk c of row r is stored at c ^ swz(r); swz spreads the 16
  // rows read by one 16-lane ds_read_b128 phase over all bank groups
  auto swz = [](int r) { return step_swz<KC>(r); };
  // FP8W: position swizzle of a code row's 16-byte pieces
  auto fswz = [](int r) { return FPR == 2 ? (r >> 3) & 1 : (r >> 2) & 3; };
  const char* Ab = reinterpret_cast<const char*>(A);

  // ---- issue side: the tile whose operands are being fetched
  int it_tile = -1;
  const char* iWb = nullptr;
  uint32_t aoff[LA], boff[LB];
  // ready_in: the expert whose rows were last seen complete and acquired; a
  // wave whose wait timed out waits no more (the error is already raised)
  int acq_e = -1;
  bool timed_out = false;
  auto set_issue_tile = [&](int j) {
    const Tile t = decode_tile<BM, BN, CLASS>(vb + j * G, NT, prefix, segs, E_loc);
    if (ready_in != nullptr && t.e != acq_e && !timed_out) {
      const uint32_t need =
          static_cast<uint32_t>(segs[t.e + 1] - segs[t.e]) * static_cast<uint32_t>(K / 32);
      int late = 0;
      if (lane == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(ready_in + t.e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               need) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins == (1u << 21)) {
            raise_error(err, MOE_ERR_HIP);
            late = 1;
            break;
          }
        }
      }
      timed_out = __builtin_amdgcn_readfirstlane(late) != 0;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      acq_e = t.e;
    }
    if constexpr (FP8W)  // one byte per code
      iWb = wlist != nullptr ? reinterpret_cast<const char*>(wlist[t.e])
                             : reinterpret_cast<const char*>(W) + t.e * wstride;
    else
      iWb = reinterpret_cast<const char*>(wlist != nullptr ? wlist[t.e] : W + t.e * wstride);
    // lane % KC is the LDS chunk position the lane writes; it fetches the
    // global chunk that belongs there
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int rt = (i * NW + wave) * RPI + lane / KC;  // row within the tile
      int arow = min(t.m0 + rt, t.seg1 - 1);
      if (gather != nullptr) arow = gather[arow] / gk;
      aoff[i] = (static_cast<uint32_t>(arow) * K + ((lane % KC) ^ swz(rt)) * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      if constexpr (FP8W) {
        // 16-byte slot (i * NW + wave) * 64 + lane: position p of tile row rt,
        // holding that row's piece c = p ^ fswz(rt)
        const int slot = (i * NW + wave) * 64 + lane;
        const int rt = slot / FPR, c = (slot % FPR) ^ fswz(rt);
        int wrow;
        if (SWIGLU) wrow = (rt / HALF) * N + min(t.n0 + rt % HALF, N - 1);
        else wrow = min(t.n0 + rt, N - 1);
        boff[i] = static_cast<uint32_t>(wrow) * K + c * 16u;
      } else {
        const int rt = (i * NW + wave) * RPI + lane / KC;
        int wrow;
        if (SWIGLU) wrow = (rt / HALF) * N + min(t.n0 + rt % HALF, N - 1);
        else wrow = min(t.n0 + rt, N - 1);
        boff[i] = (static_cast<uint32_t>(wrow) * K + ((lane % KC) ^ swz(rt)) * 8) * 2u;
      }
    }
    it_tile = j;
  };
  // part p (of 2) of a step's loads into buffer buf
  auto issue_part = [&](int p, int buf, uint32_t koff) {
    uint4* As = lds + buf * STAGE_U4;
    uint4* Bs = As + BM * KC;
#pragma unroll
    for (int i = p * LA / 2; i < (p + 1) * LA / 2; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(Ab + (aoff[i] + koff)),
          (__attribute__((address_space(3))) void*)(As + (i * NW + wave) * 64), 16, 0, 0);
    const uint32_t bkoff = FP8W ? koff / 2u : koff;  // codes: one byte per K
#pragma unroll
    for (int i = p * LB / 2; i < (p + 1) * LB / 2; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(iWb + (boff[i] + bkoff)),
          (__attribute__((address_space(3))) void*)(Bs + (i * NW + wave) * 64), 16, 0, 0);
  };
  // byte offset along K of step p's operands, switching the issue tile when p
  // starts a new one; steps past the end re-fetch the last step (valid
  // addresses, result unused)
  auto issue_koff = [&](int p) -> uint32_t {
    if (p >= S) p = S - 1;
    const int j = p / KT, kt = p - j * KT;
    if (j != it_tile) set_issue_tile(j);
    return static_cast<uint32_t>(kt) * BK * 2u;
  };

  // LDS fragments of substep ks of the step held in buffer `buf` (FP8W: the
  // weight fragments' 16 codes of both K halves as read, fbr, converted to fb
  // by cvt_frags before the MFMAs that use them)
  // (na: only the first NA of the wave's 32-row blocks, the ones holding rows
  // of the segment)
  bf16x8_t fa[2][FM], fb[2][NQ];
  uint4 fbr[2][FP8W ? NQ : 1];
  auto load_frags_n = [&](int buf, int ks, int slot, auto na) {
    constexpr int NA = decltype(na)::value;
    const uint4* As = lds + buf * STAGE_U4;
    const uint4* Bs = As + BM * KC;
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < (FM > NQ ? FM : NQ); ++i) {
      if (i < NA) {
        const int r = wm * (BM / 2) + i * 32 + (lane & 31);
        fa[slot][i] = __builtin_bit_cast(bf16x8_t, As[r * KC + (ch ^ swz(r))]);
      }
      if (i < NQ) {
        // SwiGLU: blocks [0, NQ/2) are this wave's W1 rows, [NQ/2, NQ) the
        // matching W3 rows
        const int q = SWIGLU ? ((i / (NQ / 2)) * HALF + wn * (HALF / WN) + (i % (NQ / 2)) * 32 +
                                (lane & 31))
                             : (wn * (BNW / WN) + i * 32 + (lane & 31));
        if constexpr (FP8W)
          fbr[slot][i] = Bs[q * FPR + (ks ^ fswz(q))];
        else
          fb[slot][i] = __builtin_bit_cast(bf16x8_t, Bs[q * KC + (ch ^ swz(q))]);
      }
    }
  };
  auto load_frags = [&](int buf, int ks, int slot) {
    load_frags_n(buf, ks, slot, std::integral_constant<int, FM>{});
  };
  // FP8W: the scale of this wave's MFMA tile q (its weight rows' 128-row
  // block) in K block kb
  constexpr int kScaleBlock = 128;
  const int RB = (SWIGLU ? 2 * N : N) / kScaleBlock, KB = K / kScaleBlock;
  // (se: the tile's expert's scales from slist, looked up once per tile; null
  // for the packed scales)
  auto frag_scale = [&](const float* se, const Tile& ct, int q, int kb) -> float {
    int wrow = SWIGLU ? (q / (NQ / 2)) * N + ct.n0 + wn * (HALF / WN) + (q % (NQ / 2)) * 32
                      : ct.n0 + wn * (BNW / WN) + q * 32;
    if (!SWIGLU) wrow = min(wrow, N - 1);  // columns past N are computed and dropped
    if (se != nullptr) return se[(wrow / kScaleBlock) * KB + kb];
    return Ws[(static_cast<size_t>(ct.e) * RB + wrow / kScaleBlock) * KB + kb];
  };
  // FP8W: codes of slot `slot` to dequantised bf16 operands, code x sq[q]
  // (the power-of-two scale of tile q's current K block); lanes 0..31 take
  // codes 0..7 of their 16, lanes 32..63 codes 8..15 (the K halves of the
  // 32 x 32 x 16 operand), two codes per conversion
  auto cvt_frags = [&](int slot, const float (&sq)[NQ]) {
    if constexpr (FP8W) {
      const bool hi = lane >= 32;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint4 v = fbr[slot][q];
        const int w0 = static_cast<int>(hi ? v.z : v.x), w1 = static_cast<int>(hi ? v.w : v.y);
        const float c = sq[q];
        fb[slot][q] = __builtin_bit_cast(bf16x8_t, make_uint4(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, c, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, c, true)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, c, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, c, true))));
      }
    }
  };
  // Step p becomes readable: this wave's loads of step p are done once at most
  // the (STAGES - 2) younger steps' loads are outstanding (loads complete in
  // order) and its own LDS reads of the step before are done; the barrier then
  // publishes every wave's step-p data and frees the buffer of step p - 1.
  // The loads of step p + STAGES - 1 go into that buffer in two parts: part 0
  // right after the barrier, part 1 during the first substep of step p (pk /
  // pb hold the pending step's K offset and buffer meanwhile).
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
  // reads of the next substep and (substeps that send a load part) about
  // LSTEP / 2 global loads between them
  constexpr int NMF = FM * NQ, NDS = FM + NQ, NVM = (LSTEP + 1) / 2;
  constexpr uint32_t kStepBytes = BK * 2;  // K bytes of one step in a row

  // (na: the MFMAs of the wave's first NA 32-row blocks only)
  auto mfma_substep_n = [&](f32x16_t (&acc)[FM][NQ], int slot, auto na) {
    constexpr int NA = decltype(na)::value;
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][q], fa[slot][i], acc[i][q], 0, 0, 0);
  };
  auto mfma_substep = [&](f32x16_t (&acc)[FM][NQ], int slot) {
    mfma_substep_n(acc, slot, std::integral_constant<int, FM>{});
  };
  // FP8W: after the last step of K block kb the conversions move on to block
  // kb + 1's scales.  sc holds the scales of blocks kb and kb + 1 of each
  // tile; those of block kb + 2 are loaded here, a whole block before they
  // are used.
  auto next_block_scales = [&](const float* se, const Tile& ct, int kb, float (&sc)[2][NQ]) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      sc[0][q] = sc[1][q];
      sc[1][q] = kb + 2 < KB ? frag_scale(se, ct, q, kb + 2) : 1.f;
    }
  };
  // (na: the wave's first NA 32-row blocks; the others hold no row of the
  // segment)
  auto epilogue_n = [&](const Tile& ct, f32x16_t (&acc)[FM][NQ], auto na) {
    constexpr int NA = decltype(na)::value;
    const int valid = min(BM, ct.seg1 - ct.m0);
    // registers -> global.  The MFMAs take the weight fragment as their
    // first operand, so a 32 x 32 tile holds D[n][m] (n: output column, m:
    // activation row): lane l has row m = l % 32 and, in registers 4g ..
    // 4g + 3, the four consecutive columns 8g + 4 (l / 32) .. + 3 (N is a
    // multiple of 64, so groups of four or eight columns lie on the same side
    // of N).  Stores address C with a uniform base and 32-bit byte offsets (C
    // is below 4 GiB), which keeps the epilogue's address registers few.
    char* Cb = reinterpret_cast<char*>(C);
    // fp32 -> bf16 by the hardware's packed conversion (round to nearest even)
    auto pack4 = [](const float (&v)[4]) {
      const bf16x2_t lo = __builtin_convertvector(f32x2_t{v[0], v[1]}, bf16x2_t);
      const bf16x2_t hi = __builtin_convertvector(f32x2_t{v[2], v[3]}, bf16x2_t);
      return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    };
    // the four output columns of register group g of block (i, q), SwiGLU applied
    auto block_vals = [&](int i, int q, int g, float (&v)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = acc[i][q][4 * g + c];
      if constexpr (SWIGLU) {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = silu_fast(v[c]) * acc[i][q + NQ / 2][4 * g + c];
      }
    };
    char* stg = reinterpret_cast<char*>(lds + STAGES * STAGE_U4) + wave * (32 * kOutRowBytes);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      if (wm * (BM / 2) + i * 32 >= valid) continue;
      const int rbase = ct.m0 + wm * (BM / 2) + i * 32;
#pragma unroll
      for (int q = 0; q < (SWIGLU ? NQ / 2 : NQ); ++q) {
        const int cbase = ct.n0 + (SWIGLU ? wn * (HALF / WN) : wn * (BNW / WN)) + q * 32;
        if constexpr (STAGE_OUT) {
          // the block into this wave's LDS rows (8 bytes per lane and group),
          // back as 16-byte pieces: lane l takes piece l % 4 of rows l / 4
          // and 16 + l / 4, so a store covers 16 rows x 64 bytes.  LDS
          // operations of one wave complete in order; the compiler barriers
          // keep the writes, reads and the next block's writes in that order.
          const int m = lane & 31;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
            block_vals(i, q, g, v);
            *reinterpret_cast<uint2*>(stg + m * kOutRowBytes + (8 * g + 4 * (lane >> 5)) * 2) =
                pack4(v);
          }
          asm volatile("" ::: "memory");
          const int pc = lane & 3, col = cbase + pc * 8;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = (lane >> 2) + 16 * t;
            const uint4 w = *reinterpret_cast<const uint4*>(stg + r * kOutRowBytes + pc * 16);
            if (rbase + r < ct.seg1 && col < N)
              *reinterpret_cast<uint4*>(Cb + (static_cast<uint32_t>(rbase + r) *
                                                   static_cast<uint32_t>(N) +
                                               static_cast<uint32_t>(col)) * 2u) = w;
          }
          asm volatile("" ::: "memory");
        } else {
          const int row = rbase + (lane & 31);
          if (row >= ct.seg1) continue;
          const int col0 = cbase + 4 * (lane >> 5);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = col0 + 8 * g;
            if (col >= N) continue;
            if constexpr (SAVE) {
              float a[4], gv[4];
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                a[c] = acc[i][q][4 * g + c];
                gv[c] = acc[i][q + NQ / 2][4 * g + c];
              }
              const uint32_t ab = (static_cast<uint32_t>(row) * static_cast<uint32_t>(2 * N) +
                                   static_cast<uint32_t>(col)) * 2u;
              char* ABb = reinterpret_cast<char*>(AB);
              *reinterpret_cast<uint2*>(ABb + ab) = pack4(a);
              *reinterpret_cast<uint2*>(ABb + ab + static_cast<uint32_t>(N) * 2u) = pack4(gv);
            }
            float v[4];
            block_vals(i, q, g, v);
            const uint32_t off = (static_cast<uint32_t>(row) * static_cast<uint32_t>(N) +
                                  static_cast<uint32_t>(col)) * 2u;
            *reinterpret_cast<uint2*>(Cb + off) = pack4(v);
          }
        }
      }
    }
  };
  auto epilogue = [&](const Tile& ct, f32x16_t (&acc)[FM][NQ]) {
    epilogue_n(ct, acc, std::integral_constant<int, FM>{});
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
      for (int q = 0; q < 2; ++q) issue_part(q, p, p * kStepBytes);
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
      // FP8W: the block scales of K blocks 0 and 1 of this tile's MFMA tiles
      float sc[2][NQ];
      const float* se = nullptr;
      if constexpr (FP8W) {
        if (slist != nullptr) se = slist[ct.e];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          sc[0][q] = frag_scale(se, ct, q, 0);
          sc[1][q] = KB > 1 ? frag_scale(se, ct, q, 1) : 1.f;
        }
      }
      // The K loop of one tile.  NA = the wave's 32-row blocks that hold rows
      // of the segment: the wave reads the fragments of and multiplies only
      // those (its other blocks' rows are not stored).  NA = 0: the wave's
      // rows are all past the segment (a tile less than half full), so it only
      // helps with the loads and barriers and issues no MFMAs (with 8 waves
      // it leaves its SIMD's MFMA pipe to the other wave there).  The next
      // step's first fragments are always read in full: they may belong to
      // the next tile.
      auto run_tile = [&](auto act) {
        constexpr int NA = decltype(act)::value;
        constexpr bool ACT = NA > 0;
        constexpr std::integral_constant<int, NA> na{};
        constexpr int NMFA = NA * NQ;
        // one step: substep 0 fetches substep 1's fragments and sends the
        // second half of the pending step's loads between its MFMAs (BK =
        // 64: substeps 1 and 2 fetch the fragments of the substep after
        // them); the last substep makes step s + 1 readable (barrier), sends
        // the first half of step s + STAGES's loads into this step's buffer
        // and fetches step s + 1's first fragments
        auto substep0 = [&](int s) {
          if constexpr (ACT) load_frags_n(s % STAGES, 1, 1, na);
          issue_part(1, pb, pk);
          if constexpr (ACT) {
            cvt_frags(0, sc[0]);
            mfma_substep_n(acc, 0, na);
            interleave<0, NMFA, NA + NQ, NVM>();
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (SUB == 4) {
            if constexpr (ACT) {
              load_frags_n(s % STAGES, 2, 0, na);
              cvt_frags(1, sc[0]);
              mfma_substep_n(acc, 1, na);
              interleave<0, NMFA, NA + NQ, 0>();
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ACT) {
              load_frags_n(s % STAGES, 3, 1, na);
              cvt_frags(0, sc[0]);
              mfma_substep_n(acc, 0, na);
              interleave<0, NMFA, NA + NQ, 0>();
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        auto substep1 = [&](int s, uint32_t koff_next) {
          wait_vmcnt<(STAGES - 2) * LSTEP>();
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          pk = koff_next;
          pb = s % STAGES;  // (s + STAGES) % STAGES
          issue_part(0, pb, pk);
          load_frags((s + 1) % STAGES, 0, 0);
          if constexpr (ACT) {
            cvt_frags(1, sc[0]);
            mfma_substep_n(acc, 1, na);
            interleave<0, NMFA, NDS, NVM>();
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (ACT && FP8W) {
            const int kt = s % KT;
            if ((kt + 1) % (kScaleBlock / BK) == 0)
              next_block_scales(se, ct, kt / (kScaleBlock / BK), sc);
          }
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
        epilogue_n(ct, acc, na);
      };
      // the wave's rows in the segment: none, at most one 32-row block (the
      // last tile of an expert with a few rows past a multiple of 256), or
      // more (every block; the other partial counts measured no faster)
      const int wrows = ct.seg1 - ct.m0 - wm * (BM / 2);
      if (wrows > 32) {
        run_tile(std::integral_constant<int, FM>{});
      } else if (wrows <= 0) {
        run_tile(std::integral_constant<int, 0>{});
      } else {
        run_tile(std::integral_constant<int, 1>{});
      }
    }
  } else if constexpr (!FP8W) {
    // short K (fewer steps than stages): the issue side may run several
    // tiles ahead, so it switches tiles step by step
    // (FP8W: never reached, the launcher requires K >= STAGES steps)
    for (int p = 0; p < STAGES - 1; ++p) {
      const uint32_t ko = issue_koff(p);
#pragma unroll
      for (int q = 0; q < 2; ++q) issue_part(q, p % STAGES, ko);
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
        if constexpr (SUB == 4) {
          load_frags(buf, 2, 0);
          mfma_substep(acc, 1);
          __builtin_amdgcn_sched_barrier(0);
          load_frags(buf, 3, 1);
          mfma_substep(acc, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
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
  // ready_out: every tile of this workgroup is stored (the barrier above);
  // one release at agent scope publishes them all, then each tile's rows x
  // columns / 32 are counted for its expert
  if (ready_out != nullptr) {
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      for (int j = 0; j < ntiles; ++j) {
        const Tile t = decode_tile<BM, BN, CLASS>(vb + j * G, NT, prefix, segs, E_loc);
        const int rows = min(BM, t.seg1 - t.m0), cols = min(BN, N - t.n0);
        __hip_atomic_fetch_add(ready_out + t.e, static_cast<uint32_t>(rows * (cols / 32)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // prefix / segs may be rewritten by the caller's next phase
  }
}

}  // namespace moe
