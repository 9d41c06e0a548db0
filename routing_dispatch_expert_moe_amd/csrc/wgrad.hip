// Expert weight gradients: for every local expert e, C_e = P_e^T Q_e summed
// over the expert's rows (the reduction runs over tokens, not features):
//   dW13_e [2f][d] = dab_e^T x_perm_e     (packed like w13: W1^T rows, W3^T rows)
//   dW2_e  [d][f]  = do_e^T  h_e          (packed like w2: W2^T rows)
// NCCL EP page, §3.2 (training adaptation): the expert backward that runs
// between the gradient dispatch and combine.
//
// bf16: the MFMA operands must run along the reduction, which here is the
// row (token) dimension, so both operands are first transposed into
// K-contiguous form, one block per expert: expert e's block of PT is
// [M][Kpad_e] (its rows, zero-padded to Kpad_e, a multiple of 32) at element
// M * kseg[e], with kseg the prefix of the Kpad (QT likewise with N), so the
// 256 operand rows a tile reads are one contiguous run of memory whatever the
// number of experts.  The GEMM then runs 256 x 256 output
// tiles (8 waves, 32x32x16 bf16 MFMA, direct-to-LDS loads through a 4-stage
// pipeline, the same LDS layout and swizzle as the forward's grouped GEMM),
// one tile per workgroup, K = the expert's padded rows, fp32 results.
// fp32: a VALU kernel reads the row-major operands directly (its LDS tiles
// are row-major in the reduction dimension anyway).
#include "gemm_pipe.h"
#include "launch.h"

namespace moe {

constexpr int kSegAlign = 32;  // column padding of each expert's block

// kseg[e] = sum over e' < e of roundup(rows of e', 32); kseg[E_loc] = total.
__global__ __launch_bounds__(64) void kseg_kernel(const int32_t* __restrict__ offsets, int E_loc,
                                                  int32_t* __restrict__ kseg) {
  const int lane = threadIdx.x;
  const int per = (E_loc + kWave - 1) / kWave;
  const int lo = lane * per;
  auto padded = [&](int e) {
    const int n = offsets[e + 1] - offsets[e];
    return (n + kSegAlign - 1) / kSegAlign * kSegAlign;
  };
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < E_loc) local += padded(lo + i);
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  int run = incl - local;
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E_loc) {
      kseg[e] = run;
      run += padded(e);
    }
  }
  if (lane == kWave - 1) kseg[E_loc] = incl;
}

// For a column kk of the padded space (expert e: kseg[e] <= kk < kseg[e+1],
// local column j = kk - kseg[e]) the element (m, kk) of the transposed operand
// lives at M * kseg[e] + m * Kpad_e + j and holds row r = offsets[e] + j of P
// (row pitch M) at column m, or 0 in the padding (j >= rows of e).  A 64 x 64
// tile of (kk, m) per workgroup through LDS; a 16-byte run of 8 columns never
// crosses an expert (every Kpad is a multiple of 32).  Columns past kseg[E_loc]
// do not exist.
__global__ __launch_bounds__(256) void transpose_seg_kernel(const uint16_t* __restrict__ P,
                                                            int M, const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ kseg,
                                                            int E_loc, uint16_t* __restrict__ PT) {
  __shared__ uint16_t tile[64][64 + 8];
  __shared__ int src_row[64];
  __shared__ int64_t dst_base[64];   // M * kseg[e] + j for column kk0 + i
  __shared__ int dst_pitch[64];      // Kpad_e
  const int kk0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const int total = kseg[E_loc];
  if (kk0 >= total) return;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int kk = kk0 + tid;
    int r = -1;
    if (kk < total) {
      int lo = 0, hi = E_loc - 1;  // largest e with kseg[e] <= kk
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (kseg[mid] <= kk) lo = mid; else hi = mid - 1;
      }
      const int local = kk - kseg[lo];
      if (local < offsets[lo + 1] - offsets[lo]) r = offsets[lo] + local;
      dst_base[tid] = static_cast<int64_t>(M) * kseg[lo] + local;
      dst_pitch[tid] = kseg[lo + 1] - kseg[lo];
    }
    src_row[tid] = r;
  }
  __syncthreads();
  // load: 64 source rows x 8 chunks of 8 columns
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + u * 256;
    const int kr = i >> 3, ch = i & 7;
    const int r = src_row[kr];
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r >= 0 && m0 + ch * 8 < M) v = *reinterpret_cast<const uint4*>(P + (size_t)r * M + m0 + ch * 8);
    const uint32_t pw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[kr][ch * 8 + 2 * q] = static_cast<uint16_t>(pw[q]);
      tile[kr][ch * 8 + 2 * q + 1] = static_cast<uint16_t>(pw[q] >> 16);
    }
  }
  __syncthreads();
  // store: 64 output rows (m) x 8 chunks of 8 columns (kk)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + u * 256;
    const int mr = i >> 3, ch = i & 7;
    if (m0 + mr >= M || kk0 + ch * 8 >= total) continue;
    uint32_t pw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      pw[q] = static_cast<uint32_t>(tile[ch * 8 + 2 * q][mr]) |
              (static_cast<uint32_t>(tile[ch * 8 + 2 * q + 1][mr]) << 16);
    const int c0 = ch * 8;
    *reinterpret_cast<uint4*>(PT + dst_base[c0] + static_cast<int64_t>(m0 + mr) * dst_pitch[c0]) =
        make_uint4(pw[0], pw[1], pw[2], pw[3]);
  }
}

namespace wgt {

// the K step, 16-byte chunks per row and rows per 64-lane load are the
// forward GEMM's (pipe::kBK = 32, kKC = 4, kRPI = 16)
constexpr int BM = 256, BN = 256, NW = 8, WN = 4;
constexpr int FM = BM / 64;              // 32-row MFMA blocks per wave (4)
constexpr int NQ = BN / WN / 32;         // 32-column MFMA blocks per wave (2)
constexpr int LA = BM / kRPI / NW;       // A loads per wave per step (2)
constexpr int LB = BN / kRPI / NW;       // B loads per wave per step (2)
constexpr int LSTEP = LA + LB;
constexpr int STAGES = 4;
constexpr int STAGE_U4 = (BM + BN) * kKC;

}  // namespace wgt

// epilogue staging: half the tile's rows, fp32, rows padded to 264 floats
// (the two row groups one store instruction covers land 32 banks apart)
constexpr int kOutPitch = wgt::BN + 8;
constexpr size_t wgrad_lds_bytes() {
  const size_t pipe = static_cast<size_t>(wgt::STAGES) * wgt::STAGE_U4 * sizeof(uint4);
  const size_t out = static_cast<size_t>(wgt::BM / 2) * kOutPitch * sizeof(float);
  return pipe > out ? pipe : out;
}

// Tiles: 256 x 256 blocks of C_e (fp32, row pitch N), numbered expert-major,
// then M-tiles, then N-tiles (neighbouring ids share a PT tile).  A tile of
// expert e costs about KT_e + kTileOverhead pipeline steps, so the tile
// sequence is cut into 8 ranges of equal cost, one per XCD (workgroup ids are
// dealt round-robin over the XCDs), and the XCD's workgroups take its tiles
// in turn: neighbouring tiles run together and share operands in that XCD's
// L2, and a few hot experts cannot pile up on one XCD.
constexpr int kTileOverhead = 4;

// First tile of the split point `part` of `parts`: the smallest tile index
// whose preceding tiles cost at least part / parts of the total.  Run by one
// whole wave; every lane returns the same value.
__device__ int cost_split(const int32_t* __restrict__ kseg, int E_loc, int per_e, int part,
                          int parts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (E_loc + kWave - 1) / kWave;
  const int lo = lane * per;
  auto cost = [&](int e) {  // per-tile cost of expert e
    return static_cast<int64_t>((kseg[e + 1] - kseg[e]) / kBK + kTileOverhead);
  };
  int64_t local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < E_loc) local += cost(lo + i);
  int64_t incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t v = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += v;
  }
  const int64_t total = __shfl(incl, kWave - 1, kWave);
  // target in (per-tile cost) x (tiles) units
  const int64_t tau = total * per_e * part / parts;
  int64_t run = (incl - local) * per_e;
  int found = part >= parts ? E_loc * per_e : -1;
  if (found < 0) {
    for (int i = 0; i < per; ++i) {
      const int e = lo + i;
      if (e >= E_loc) break;
      const int64_t c = cost(e);
      if (tau < run + c * per_e) {
        const int64_t t = tau <= run ? 0 : (tau - run + c - 1) / c;
        found = (run <= tau || lane == 0) ? e * per_e + static_cast<int>(t) : -1;
        break;
      }
      run += c * per_e;
    }
  }
  // exactly one lane's run holds the target (every expert costs at least
  // kTileOverhead); an empty result means the target is the end
  const uint64_t has = __ballot(found >= 0 && !(lo >= E_loc));
  if (has == 0) return E_loc * per_e;
  return __shfl(found, __builtin_ctzll(has), kWave);
}

// Persistent: one workgroup per CU walks its XCD's tile range.
__global__ __launch_bounds__(512, 1) void wgrad_bf16_kernel(const uint16_t* __restrict__ PT,
                                                            const uint16_t* __restrict__ QT,
                                                            const int32_t* __restrict__ kseg,
                                                            int E_loc, int M, int N, int tiles_m,
                                                            int tiles_n, float* __restrict__ C) {
  using namespace wgt;
  extern __shared__ uint4 lds[];
  __shared__ int range[2];
  const int G = gridDim.x, bid = blockIdx.x;
  const int per_e = tiles_m * tiles_n;
  const bool by_xcd = (G & 7) == 0;
  const int xcd = by_xcd ? (bid & 7) : 0, parts = by_xcd ? 8 : 1;
  const int local = by_xcd ? (bid >> 3) : bid, stride = by_xcd ? (G >> 3) : G;
  if (threadIdx.x < kWave) {
    const int a = cost_split(kseg, E_loc, per_e, xcd, parts);
    const int b = cost_split(kseg, E_loc, per_e, xcd + 1, parts);
    if (threadIdx.x == 0) {
      range[0] = a;
      range[1] = b;
    }
  }
  __syncthreads();
  const int t_lo = range[0], t_hi = range[1];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  auto swz = [](int r) { return (r >> 2) & 3; };
  const int lkc = (lane % kKC) ^ swz(lane / kKC);

  for (int vb = t_lo + local; vb < t_hi; vb += stride) {
  const int e = vb / per_e;
  const int rem = vb - e * per_e;
  const int m0 = (rem / tiles_n) * BM, n0 = (rem % tiles_n) * BN;
  const int k0 = kseg[e];
  const int kpad = kseg[e + 1] - k0;  // the expert's padded rows: the K of its tiles
  const int KT = kpad / kBK;

  f32x16_t acc[FM][NQ];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[i][q] = f32x16_t{};

  if (KT > 0) {
    const char* pa[LA];
    const char* pb[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int rt = (i * NW + wave) * kRPI + lane / kKC;
      pa[i] = reinterpret_cast<const char*>(PT + static_cast<size_t>(M) * k0 +
                                            (size_t)min(m0 + rt, M - 1) * kpad + lkc * 8);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int rt = (i * NW + wave) * kRPI + lane / kKC;
      pb[i] = reinterpret_cast<const char*>(QT + static_cast<size_t>(N) * k0 +
                                            (size_t)min(n0 + rt, N - 1) * kpad + lkc * 8);
    }
    // step p's loads into buffer p % STAGES (steps past the end re-fetch the
    // last one: valid addresses, result unused)
    auto issue = [&](int p) {
      const int ps = min(p, KT - 1);
      const uint32_t koff = static_cast<uint32_t>(ps) * kBK * 2u;
      uint4* As = lds + (p % STAGES) * STAGE_U4;
      uint4* Bs = As + BM * kKC;
#pragma unroll
      for (int i = 0; i < LA; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(pa[i] + koff),
            (__attribute__((address_space(3))) void*)(As + (i * NW + wave) * 64), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < LB; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(pb[i] + koff),
            (__attribute__((address_space(3))) void*)(Bs + (i * NW + wave) * 64), 16, 0, 0);
    };
    bf16x8_t fa[2][FM], fb[2][NQ];
    auto frags = [&](int buf, int ks, int slot) {
      const uint4* As = lds + buf * STAGE_U4;
      const uint4* Bs = As + BM * kKC;
      const int ch = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * (BM / 2) + i * 32 + (lane & 31);
        fa[slot][i] = __builtin_bit_cast(bf16x8_t, As[r * kKC + (ch ^ swz(r))]);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int r = wn * (BN / WN) + q * 32 + (lane & 31);
        fb[slot][q] = __builtin_bit_cast(bf16x8_t, Bs[r * kKC + (ch ^ swz(r))]);
      }
    };
    auto mfma = [&](int slot) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          acc[i][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][q], acc[i][q], 0, 0, 0);
    };
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue(p);
    // step p becomes readable once at most the STAGES - 2 younger steps'
    // loads are outstanding (loads complete in order) and the barrier has
    // published every wave's share
    wait_vmcnt<(STAGES - 2) * LSTEP>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(STAGES - 1);
    frags(0, 0, 0);
    for (int s = 0; s < KT; ++s) {
      const int buf = s % STAGES;
      // substep 0: the second half's fragments load under the first half's MFMAs
      frags(buf, 1, 1);
      mfma(0);
      // step s + 1 becomes readable; this wave's reads of step s are done, so
      // after the barrier step s's buffer takes step s + STAGES; the next
      // step's first fragments load under the second half's MFMAs
      wait_vmcnt<(STAGES - 2) * LSTEP>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      issue(s + STAGES);
      frags((s + 1) % STAGES, 0, 0);
      mfma(1);
    }
    wait_vmcnt<0>();
  }
  // Epilogue through LDS, half the rows at a time: the waves owning those rows
  // place their accumulators (D[m][n] of a 32x32 MFMA tile sits in lane
  // n + 32 * ((m / 4) % 2), register 4 * (m / 8) + m % 4), then every wave
  // writes whole 1 KB row runs with 16-byte streaming stores (the gradients
  // are not read again here).
  __syncthreads();  // every wave is done with the pipeline's buffers
  float* Ls = reinterpret_cast<float*>(lds);
  float* Ce = C + (size_t)e * M * N;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + 8 * (r >> 2) + (r & 3) + 4 * (lane >> 5);
            const int col = wn * (BN / WN) + q * 32 + (lane & 31);
            Ls[row * kOutPitch + col] = acc[i][q][r];
          }
    }
    __syncthreads();
    const int c = n0 + lane * 4;
    for (int rr = wave; rr < BM / 2; rr += NW) {
      const int m = m0 + half * (BM / 2) + rr;
      if (m < M && c < N)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(Ls + rr * kOutPitch + lane * 4),
                                    reinterpret_cast<f32x4_t*>(Ce + (size_t)m * N + c));
    }
    __syncthreads();
  }
  }
}

// fp32: C_e[m][n] = sum over the expert's rows r of P[r][m] Q[r][n]; 64 x 64
// tiles of 4 x 4 per thread, rows in steps of 16 through LDS.
__global__ __launch_bounds__(256) void wgrad_f32_kernel(const float* __restrict__ P,
                                                        const float* __restrict__ Q,
                                                        const int32_t* __restrict__ offsets,
                                                        int M, int N, int tiles_m, int tiles_n,
                                                        float* __restrict__ C) {
  __shared__ float Ps[16][64 + 4];
  __shared__ float Qs[16][64 + 4];
  const int per_e = tiles_m * tiles_n;
  const int e = blockIdx.x / per_e;
  const int rem = blockIdx.x - e * per_e;
  const int m0 = (rem / tiles_n) * 64, n0 = (rem % tiles_n) * 64;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = r0; k0 < r1; k0 += 16) {
    {
      const int kr = tid >> 4, c4 = (tid & 15) * 4;
      const int r = k0 + kr;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (r < r1 && m0 + c4 < M) a = *reinterpret_cast<const float4*>(P + (size_t)r * M + m0 + c4);
      if (r < r1 && n0 + c4 < N) b = *reinterpret_cast<const float4*>(Q + (size_t)r * N + n0 + c4);
      Ps[kr][c4] = a.x; Ps[kr][c4 + 1] = a.y; Ps[kr][c4 + 2] = a.z; Ps[kr][c4 + 3] = a.w;
      Qs[kr][c4] = b.x; Qs[kr][c4 + 1] = b.y; Qs[kr][c4 + 2] = b.z; Qs[kr][c4 + 3] = b.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = Ps[kk][ty * 4 + i];
        b[i] = Qs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Ce = C + (size_t)e * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) Ce[(size_t)m * N + n] = acc[i][j];
    }
  }
}

size_t wgrad_ldk(int64_t max_rows, int E_loc) {
  const int64_t k = max_rows + static_cast<int64_t>(E_loc) * (kSegAlign - 1);
  return static_cast<size_t>((k + 63) / 64 * 64);
}

size_t wgrad_ws_bytes(int64_t max_rows, int E_loc, int d, int f, int bf16) {
  const size_t head = (static_cast<size_t>(E_loc + 1) * 4 + 255) & ~static_cast<size_t>(255);
  if (!bf16) return head;
  // the larger pass (dW13) holds 2f x ldk elements of PT and d x ldk of QT
  return head + static_cast<size_t>(2 * f + d) * wgrad_ldk(max_rows, E_loc) * 2;
}

namespace {

int run_bf16(const uint16_t* P, int M, const uint16_t* Q, int N, const int32_t* offsets,
             int E_loc, const int32_t* kseg, size_t ldk, uint16_t* PT, uint16_t* QT, float* C,
             hipStream_t s) {
  const dim3 tp(static_cast<unsigned>(ldk / 64), static_cast<unsigned>((M + 63) / 64));
  hipLaunchKernelGGL(transpose_seg_kernel, tp, dim3(256), 0, s, P, M, offsets, kseg, E_loc, PT);
  const dim3 tq(static_cast<unsigned>(ldk / 64), static_cast<unsigned>((N + 63) / 64));
  hipLaunchKernelGGL(transpose_seg_kernel, tq, dim3(256), 0, s, Q, N, offsets, kseg, E_loc, QT);
  static LdsAttr attr;
  if (int rc = set_dynamic_lds_once(reinterpret_cast<const void*>(wgrad_bf16_kernel),
                                    wgrad_lds_bytes(), attr))
    return rc;
  const int tiles_m = (M + wgt::BM - 1) / wgt::BM, tiles_n = (N + wgt::BN - 1) / wgt::BN;
  hipLaunchKernelGGL(wgrad_bf16_kernel, dim3(static_cast<unsigned>(device_cu_count())), dim3(512),
                     wgrad_lds_bytes(), s, PT, QT, kseg, E_loc, M, N, tiles_m, tiles_n, C);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_ffn_wgrad(const void* x_perm, const void* h, const void* do_perm, const void* dab,
                     const int32_t* offsets, int E_loc, int64_t max_rows, int d, int f, int bf16,
                     float* dw13, float* dw2, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!bf16) {
    const int tm13 = (2 * f + 63) / 64, tn13 = (d + 63) / 64;
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(static_cast<unsigned>(E_loc * tm13 * tn13)),
                       dim3(256), 0, s, static_cast<const float*>(dab),
                       static_cast<const float*>(x_perm), offsets, 2 * f, d, tm13, tn13, dw13);
    const int tm2 = (d + 63) / 64, tn2 = (f + 63) / 64;
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(static_cast<unsigned>(E_loc * tm2 * tn2)), dim3(256),
                       0, s, static_cast<const float*>(do_perm), static_cast<const float*>(h),
                       offsets, d, f, tm2, tn2, dw2);
    return static_cast<int>(hipGetLastError());
  }
  char* w = static_cast<char*>(ws);
  int32_t* kseg = reinterpret_cast<int32_t*>(w);
  const size_t head = (static_cast<size_t>(E_loc + 1) * 4 + 255) & ~static_cast<size_t>(255);
  const size_t ldk = wgrad_ldk(max_rows, E_loc);
  uint16_t* PT = reinterpret_cast<uint16_t*>(w + head);
  hipLaunchKernelGGL(kseg_kernel, dim3(1), dim3(64), 0, s, offsets, E_loc, kseg);
  // dW2 = do^T h: PT from do (M = d), QT from h (N = f)
  int e = run_bf16(static_cast<const uint16_t*>(do_perm), d, static_cast<const uint16_t*>(h), f,
                   offsets, E_loc, kseg, ldk, PT, PT + static_cast<size_t>(d) * ldk, dw2, s);
  if (e != 0) return e;
  // dW13 = dab^T x_perm: PT from dab (M = 2f), QT from x_perm (N = d)
  return run_bf16(static_cast<const uint16_t*>(dab), 2 * f, static_cast<const uint16_t*>(x_perm),
                  d, offsets, E_loc, kseg, ldk, PT, PT + static_cast<size_t>(2 * f) * ldk, dw13, s);
}

}  // namespace moe
