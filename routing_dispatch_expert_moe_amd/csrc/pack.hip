// One-time weight re-layout into the K-contiguous packed form (MoE
// sparse-activation page §4.2 layer 2: each expert's weights contiguous,
// re-ordered once at load; DWDP page: W3 and W1 as one first-layer operand).
//   w13[e][n][c]     = w1[e][c][n]   (n < f)
//   w13[e][f + n][c] = w3[e][c][n]
//   w2p[e][c][n]     = w2[e][n][c]
// 64 x 64 tiles transposed through LDS (padded rows avoid bank conflicts).
#include "common.h"
#include "launch.h"

namespace moe {

// dst[z][j][i] = src[z][i][j] for a batch of R x S matrices, dst rows strided by dst_zstride
template <typename Tel>
__global__ __launch_bounds__(256) void transpose_kernel(const Tel* __restrict__ src, int R, int S,
                                                        Tel* __restrict__ dst, size_t dst_zstride) {
  __shared__ Tel tile[64][65];
  const int z = blockIdx.z;
  const Tel* s = src + (size_t)z * R * S;
  Tel* o = dst + (size_t)z * dst_zstride;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int i = i0 + r, j = j0 + tx;
    if (i < R && j < S) tile[r][tx] = s[(size_t)i * S + j];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int j = j0 + r, i = i0 + tx;
    if (j < S && i < R) o[(size_t)j * R + i] = tile[tx][r];
  }
}

template <typename Tel>
static void transpose(const void* src, int E, int R, int S, void* dst, size_t dst_zstride,
                      hipStream_t st) {
  dim3 grid((S + 63) / 64, (R + 63) / 64, E);
  hipLaunchKernelGGL(transpose_kernel<Tel>, grid, dim3(256), 0, st, static_cast<const Tel*>(src),
                     R, S, static_cast<Tel*>(dst), dst_zstride);
}

int launch_pack(const void* w1, const void* w3, const void* w2, int E_loc, int d, int f,
                int elem_bytes, void* w13, void* w2p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t zs13 = static_cast<size_t>(2) * f * d;  // elements per packed W13 expert
  const size_t zs2 = static_cast<size_t>(d) * f;
  char* w13b = static_cast<char*>(w13);
  if (elem_bytes == 2) {
    transpose<uint16_t>(w1, E_loc, d, f, w13b, zs13, s);
    transpose<uint16_t>(w3, E_loc, d, f, w13b + static_cast<size_t>(f) * d * 2, zs13, s);
    transpose<uint16_t>(w2, E_loc, f, d, w2p, zs2, s);
  } else {
    transpose<float>(w1, E_loc, d, f, w13b, zs13, s);
    transpose<float>(w3, E_loc, d, f, w13b + static_cast<size_t>(f) * d * 4, zs13, s);
    transpose<float>(w2, E_loc, f, d, w2p, zs2, s);
  }
  return static_cast<int>(hipGetLastError());
}

// The first FFN half's backward operand: w13_t[e][c] = W1[e][c][:] ‖ W3[e][c][:]
// (rows of 2f, K-contiguous for the input-gradient GEMM), 16-byte chunks.
__global__ __launch_bounds__(256) void concat_rows_kernel(const uint4* __restrict__ a,
                                                          const uint4* __restrict__ b,
                                                          int64_t rows, int chunks,
                                                          uint4* __restrict__ out) {
  const int64_t total = rows * 2 * chunks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / (2 * chunks);
    const int c = static_cast<int>(i - r * 2 * chunks);
    out[i] = c < chunks ? a[r * chunks + c] : b[r * chunks + c - chunks];
  }
}

int launch_pack_backward(const void* w1, const void* w3, int E_loc, int d, int f, int elem_bytes,
                         void* w13_t, void* stream) {
  const int chunks = f * elem_bytes / 16;
  const int64_t rows = static_cast<int64_t>(E_loc) * d;
  int64_t blocks = (rows * 2 * chunks + 255) / 256;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(concat_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(w1),
                     static_cast<const uint4*>(w3), rows, chunks, static_cast<uint4*>(w13_t));
  return static_cast<int>(hipGetLastError());
}

}  // namespace moe
