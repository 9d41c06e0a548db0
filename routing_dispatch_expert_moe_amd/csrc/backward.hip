// Backward pass of the MoE layer: the elementwise, combine-side, router and
// weight-gradient kernels.  (The two input-gradient GEMMs are the forward's
// grouped GEMMs over the transposed weights; see api.cpp.)
//
// NCCL EP page, §3.2 (training adaptation): the backward step reuses the
// forward's routing handle: the output gradient goes to the experts through
// it, the experts run their backward, and the input gradients come back
// through the same handle.  Here the handle is the dispatch plan (pair_pos,
// offsets); what is computed is the derivative of the forward layer with the
// routing decisions held fixed.
#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// Combine backward: for each token t and choice j with a local row r,
// do_perm[r] = w[t][j] * dy[t] (one rounding) and dgate[t][j] = dy[t] . y_perm[r]
// (fp32, lane partials in chunk order, then a fixed butterfly); pairs without
// a local row get dgate 0.  One wave per token; every row is touched once.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint4* __restrict__ dy, const uint4* __restrict__ y_perm,
    const int32_t* __restrict__ pair_pos, const float* __restrict__ topk_w, int T, int k,
    int chunks, uint4* __restrict__ do_perm, float* __restrict__ dgate) {
  constexpr int EPC = BF16 ? 8 : 4;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int rows[MOE_MAX_K];
  float w[MOE_MAX_K], dot[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    rows[j] = j < k ? pair_pos[(size_t)t * k + j] : -1;
    w[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
    dot[j] = 0.f;
  }
  auto unpack = [](const uint4& v, float* f) {
    if constexpr (BF16) {
      unpack8(v, f);
    } else {
      f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
  };
  for (int c = lane; c < chunks; c += kWave) {
    const uint4 g = dy[(size_t)t * chunks + c];
    uint4 v[MOE_MAX_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j)
      if (rows[j] >= 0) v[j] = y_perm[(size_t)rows[j] * chunks + c];
    float fg[EPC];
    unpack(g, fg);
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (rows[j] < 0) continue;
      float fy[EPC], o[EPC];
      unpack(v[j], fy);
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        dot[j] = fmaf(fg[i], fy[i], dot[j]);
        o[i] = w[j] * fg[i];
      }
      uint4 out;
      if constexpr (BF16) {
        out = pack8(o);
      } else {
        out = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                         __float_as_uint(o[3]));
      }
      do_perm[(size_t)rows[j] * chunks + c] = out;
    }
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    if (j >= k) break;
    const float s = wave_sum_f32(dot[j]);
    if (lane == 0) dgate[(size_t)t * k + j] = rows[j] >= 0 ? s : 0.f;
  }
}

int launch_combine_backward(const void* dy, const void* y_perm, const int32_t* pair_pos,
                            const float* topk_w, int T, int k, int d, int bf16, void* do_perm,
                            float* dgate, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return 0;
  const int chunks = bf16 ? d / 8 : d / 4;
  dim3 grid((T + 3) / 4), block(256);
  if (bf16)
    hipLaunchKernelGGL(combine_backward_kernel<true>, grid, block, 0, s,
                       static_cast<const uint4*>(dy), static_cast<const uint4*>(y_perm), pair_pos,
                       topk_w, T, k, chunks, static_cast<uint4*>(do_perm), dgate);
  else
    hipLaunchKernelGGL(combine_backward_kernel<false>, grid, block, 0, s,
                       static_cast<const uint4*>(dy), static_cast<const uint4*>(y_perm), pair_pos,
                       topk_w, T, k, chunks, static_cast<uint4*>(do_perm), dgate);
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Gate backward: dlogits[t][e] from dgate[t][j] through the gate function of
// the k chosen logits (recomputed from the logits), 0 for the other experts.
//   softmax over the chosen: dl_j = w_j (dg_j - sum_i w_i dg_i)
//   sigmoid normalised:      dl_j = s_j (1 - s_j) (dg_j - sum_i w_i dg_i) / S
// One wave per token; lane j < k holds choice j; the row is written whole.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_backward_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dgate, int T, int E, int k, int gate, float* __restrict__ dlogits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const bool on = lane < k;
  const int e = on ? topk_idx[(size_t)t * k + lane] : 0;
  const float l = on ? logits[(size_t)t * E + e] + 0.f : 0.f;
  const float dg = on ? dgate[(size_t)t * k + lane] : 0.f;
  const float x0 = __shfl(l, 0, kWave);
  float v, sg = 0.f;
  if (gate == MOE_GATE_SOFTMAX_TOPK_RENORM) {
    v = on ? expf(l - x0) : 0.f;
  } else {
    sg = on ? 1.f / (1.f + expf(-l)) : 0.f;
    v = sg;
  }
  const float tot = wave_sum_f32(v);
  const float w = v / tot;
  const float centred = dg - wave_sum_f32(w * dg);
  const float dl = gate == MOE_GATE_SOFTMAX_TOPK_RENORM ? w * centred
                                                         : sg * (1.f - sg) * centred / tot;
  for (int c = lane; c < E; c += kWave) {
    float out = 0.f;
    for (int j = 0; j < k; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      const float vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dl), j));
      if (c == ej) out = vj;
    }
    dlogits[(size_t)t * E + c] = out;
  }
}

int launch_gate_backward(const float* logits, const int32_t* topk_idx, const float* dgate, int T,
                         int E, int k, int gate, float* dlogits, void* stream) {
  if (T == 0) return 0;
  hipLaunchKernelGGL(gate_backward_kernel, dim3((T + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), logits, topk_idx, dgate, T, E, k, gate,
                     dlogits);
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// SwiGLU backward: h = silu(a) * g with a, g the saved pre-activations (ab
// rows: a then g, f each).  da = dh * g * s * (1 + a (1 - s)), dg = dh * a * s,
// s = sigmoid(a), written as dab rows (da then dg).  Rows [0, offsets[E_loc]);
// one 16-byte chunk of columns per thread.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void swiglu_backward_kernel(
    const uint4* __restrict__ dh, const uint4* __restrict__ ab,
    const int32_t* __restrict__ offsets, int E_loc, int fc, uint4* __restrict__ dab) {
  constexpr int EPC = BF16 ? 8 : 4;
  const int64_t n = offsets[E_loc];
  const int64_t total = n * fc;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / fc;
    const int c = static_cast<int>(i - r * fc);
    const uint4 vh = dh[r * fc + c];
    const uint4 va = ab[r * 2 * fc + c];
    const uint4 vg = ab[r * 2 * fc + fc + c];
    float fh[EPC], fa[EPC], fg[EPC], da[EPC], dg[EPC];
    if constexpr (BF16) {
      unpack8(vh, fh); unpack8(va, fa); unpack8(vg, fg);
    } else {
      const uint32_t* ph = &vh.x; const uint32_t* pa = &va.x; const uint32_t* pg = &vg.x;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        fh[q] = __uint_as_float(ph[q]); fa[q] = __uint_as_float(pa[q]); fg[q] = __uint_as_float(pg[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < EPC; ++q) {
      const float s = 1.f / (1.f + expf(-fa[q]));
      da[q] = fh[q] * fg[q] * s * (1.f + fa[q] * (1.f - s));
      dg[q] = fh[q] * fa[q] * s;
    }
    uint4 oa, og;
    if constexpr (BF16) {
      oa = pack8(da); og = pack8(dg);
    } else {
      oa = make_uint4(__float_as_uint(da[0]), __float_as_uint(da[1]), __float_as_uint(da[2]), __float_as_uint(da[3]));
      og = make_uint4(__float_as_uint(dg[0]), __float_as_uint(dg[1]), __float_as_uint(dg[2]), __float_as_uint(dg[3]));
    }
    dab[r * 2 * fc + c] = oa;
    dab[r * 2 * fc + fc + c] = og;
  }
}

int launch_swiglu_backward(const void* dh, const void* ab, const int32_t* offsets, int E_loc,
                           int64_t max_rows, int f, int bf16, void* dab, void* stream) {
  if (max_rows == 0) return 0;
  const int fc = bf16 ? f / 8 : f / 4;
  int64_t blocks = (max_rows * fc + 255) / 256;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    hipLaunchKernelGGL(swiglu_backward_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, s, static_cast<const uint4*>(dh), static_cast<const uint4*>(ab), offsets,
                       E_loc, fc, static_cast<uint4*>(dab));
  else
    hipLaunchKernelGGL(swiglu_backward_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, static_cast<const uint4*>(dh),
                       static_cast<const uint4*>(ab), offsets, E_loc, fc,
                       static_cast<uint4*>(dab));
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Router backward (logits = x . W_g, W_g [d][E] fp32):
//   dx[t][c] += sum_e dlogits[t][e] W_g[c][e]   (fp32 sum, one more rounding)
//   dW_g[c][e] = sum_t x[t][c] dlogits[t][e]    (fp32, fixed order)
// dx: a workgroup owns 8 tokens and 2048 columns (8 per thread); W_g rows are
// read once per workgroup in blocks of 8 experts.  dW_g: workgroups own
// 64-token slices and 2048 columns, write partial sums per slice, and a second
// kernel adds the slices in order (no atomics).
// ---------------------------------------------------------------------------
constexpr int kRbTok = 8;        // tokens per dx workgroup
constexpr int kRbSlice = 64;     // tokens per dW_g slice

template <bool BF16>
__global__ __launch_bounds__(256) void router_backward_dx_kernel(
    const float* __restrict__ dlogits, const float* __restrict__ wg, int T, int d, int E,
    void* __restrict__ dx) {
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  const int t0 = blockIdx.x * kRbTok;
  if (c0 >= d) return;
  float acc[kRbTok][8];
#pragma unroll
  for (int i = 0; i < kRbTok; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
  for (int e0 = 0; e0 < E; e0 += 8) {
    float w[8][8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) w[q][j] = e0 + j < E ? wg[(size_t)(c0 + q) * E + e0 + j] : 0.f;
#pragma unroll
    for (int i = 0; i < kRbTok; ++i) {
      if (t0 + i >= T) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float g = e0 + j < E ? dlogits[(size_t)(t0 + i) * E + e0 + j] : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] = fmaf(g, w[q][j], acc[i][q]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRbTok; ++i) {
    if (t0 + i >= T) break;
    if constexpr (BF16) {
      uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(dx) + (size_t)(t0 + i) * d + c0);
      float f[8];
      unpack8(*p, f);
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] += acc[i][q];
      *p = pack8(f);
    } else {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(dx) + (size_t)(t0 + i) * d + c0);
      float4 a = p[0], b = p[1];
      a.x += acc[i][0]; a.y += acc[i][1]; a.z += acc[i][2]; a.w += acc[i][3];
      b.x += acc[i][4]; b.y += acc[i][5]; b.z += acc[i][6]; b.w += acc[i][7];
      p[0] = a;
      p[1] = b;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void router_backward_dwg_kernel(
    const void* __restrict__ x, const float* __restrict__ dlogits, int T, int d, int E,
    float* __restrict__ part) {
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  const int t0 = blockIdx.x * kRbSlice;
  if (c0 >= d) return;
  const int t1 = min(T, t0 + kRbSlice);
  for (int e0 = 0; e0 < E; e0 += 8) {
    float acc[8][8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[q][j] = 0.f;
    for (int t = t0; t < t1; ++t) {
      float xv[8];
      if constexpr (BF16) {
        unpack8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * d + c0), xv);
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * d + c0);
        const float4 a = p[0], b = p[1];
        xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
        xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float g = e0 + j < E ? dlogits[(size_t)t * E + e0 + j] : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q][j] = fmaf(xv[q], g, acc[q][j]);
      }
    }
    float* out = part + (size_t)blockIdx.x * d * E;
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (e0 + j < E) out[(size_t)(c0 + q) * E + e0 + j] = acc[q][j];
  }
}

__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int S,
                                                         int64_t n, float* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < S; ++k) s += part[(size_t)k * n + i];
  out[i] = s;
}

size_t router_backward_ws_bytes(int T, int d, int E) {
  const size_t S = (static_cast<size_t>(T) + kRbSlice - 1) / kRbSlice;
  return S * static_cast<size_t>(d) * E * sizeof(float);
}

int launch_router_backward(const void* x, const float* wg, const float* dlogits, int T, int d,
                           int E, int bf16, void* dx, float* dwg, float* part, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cb = (d / 8 + 255) / 256;
  if (T == 0) {
    hipLaunchKernelGGL(sum_slices_kernel, dim3((d * E + 255) / 256), dim3(256), 0, s, part, 0,
                       static_cast<int64_t>(d) * E, dwg);
    return static_cast<int>(hipGetLastError());
  }
  const dim3 gdx((T + kRbTok - 1) / kRbTok, cb);
  const int S = (T + kRbSlice - 1) / kRbSlice;
  const dim3 gdw(S, cb);
  if (bf16) {
    hipLaunchKernelGGL(router_backward_dx_kernel<true>, gdx, dim3(256), 0, s, dlogits, wg, T, d, E, dx);
    hipLaunchKernelGGL(router_backward_dwg_kernel<true>, gdw, dim3(256), 0, s, x, dlogits, T, d, E, part);
  } else {
    hipLaunchKernelGGL(router_backward_dx_kernel<false>, gdx, dim3(256), 0, s, dlogits, wg, T, d, E, dx);
    hipLaunchKernelGGL(router_backward_dwg_kernel<false>, gdw, dim3(256), 0, s, x, dlogits, T, d, E, part);
  }
  const int64_t n = static_cast<int64_t>(d) * E;
  hipLaunchKernelGGL(sum_slices_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, part, S, n, dwg);
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
