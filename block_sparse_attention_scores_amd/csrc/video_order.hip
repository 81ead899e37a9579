// Video-aware block organisation (the Top-p sparse-attention abstract, mlsift
// listing, tag "sequence parallelism": tokens are organised into blocks in a
// video-aware way).  Tokens of a (T, Hl, Wl) latent are put in 3-D tile order:
// tiles in raster order over the tile grid, raster order inside a tile, edge
// tiles clipped.
//
//   order_kernel  : one thread per token; its position in closed form (all
//                   tokens of earlier t-slabs, earlier tile rows of its slab,
//                   earlier tiles of its row, then its rank inside the tile)
//   qorder_kernel : one workgroup; a running prefix over positions counts the
//                   query-share tokens before each one
//   permute_kernel: grid-stride row gather, 16- or 4-byte chunks
#include <algorithm>

#include "sa_common.h"

namespace sa {
namespace {

__global__ __launch_bounds__(256) void order_kernel(int T, int Hl, int Wl, int tt, int th, int tw,
                                                    int32_t* __restrict__ order,
                                                    int32_t* __restrict__ inverse) {
  const int64_t n = (int64_t)T * Hl * Wl;
  for (int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; r < n;
       r += (int64_t)gridDim.x * blockDim.x) {
    const int x = (int)(r % Wl), y = (int)((r / Wl) % Hl), t = (int)(r / ((int64_t)Wl * Hl));
    const int a = t / tt, b = y / th, c = x / tw;
    const int ta = min(tt, T - a * tt);   // extents of this token's (clipped) tile
    const int yb = min(th, Hl - b * th);
    const int xc = min(tw, Wl - c * tw);
    const int64_t pos = (int64_t)a * tt * Hl * Wl + (int64_t)ta * b * th * Wl +
                        (int64_t)ta * yb * c * tw +
                        ((int64_t)(t - a * tt) * yb + (y - b * th)) * xc + (x - c * tw);
    inverse[r] = (int32_t)pos;
    order[pos] = (int32_t)r;
  }
}

constexpr int kQThreads = 1024;

__global__ __launch_bounds__(kQThreads) void qorder_kernel(const int32_t* __restrict__ order,
                                                           int64_t n, int64_t q_start,
                                                           int64_t q_valid,
                                                           int32_t* __restrict__ q_order,
                                                           int32_t* __restrict__ q_inverse) {
  __shared__ int scratch[kQThreads / kWave + 1];
  int64_t base = 0;   // query tokens in positions before this chunk
  for (int64_t p0 = 0; p0 < n; p0 += kQThreads) {
    const int64_t p = p0 + threadIdx.x;
    int64_t r = -1;
    if (p < n) {
      const int64_t o = order[p] - q_start;
      if (o >= 0 && o < q_valid) r = o;
    }
    int total;
    const int incl = block_inclusive_scan((int)(r >= 0), scratch, &total);
    if (r >= 0) {
      const int64_t qp = base + incl - 1;
      q_order[qp] = (int32_t)r;
      q_inverse[r] = (int32_t)qp;
    }
    base += total;
    __syncthreads();   // scratch is reused by the next chunk
  }
}

template <typename C>
__global__ __launch_bounds__(256) void permute_kernel(int heads, int64_t rows, int cpr,
                                                      const int32_t* __restrict__ idx,
                                                      const C* __restrict__ src, int64_t src_rows,
                                                      C* __restrict__ dst, int64_t dst_rows) {
  // one chunk per thread and step; chunk c of row r of head h
  const int64_t total = (int64_t)heads * dst_rows * cpr;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(u % cpr);
    const int64_t hr = u / cpr;
    const int64_t r = hr % dst_rows, h = hr / dst_rows;
    C val{};
    if (r < rows) {
      const int64_t s = idx[r];
      if (s >= 0 && s < src_rows) val = src[(h * src_rows + s) * cpr + c];
    }
    dst[hr * cpr + c] = val;
  }
}

}  // namespace

hipError_t launch_video_order(int T, int Hl, int Wl, int tt, int th, int tw, int64_t q_start,
                              int64_t q_valid, int32_t* order, int32_t* inverse, int32_t* q_order,
                              int32_t* q_inverse, hipStream_t s) {
  const int64_t n = (int64_t)T * Hl * Wl;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(order_kernel, dim3(grid), dim3(256), 0, s, T, Hl, Wl, tt, th, tw, order,
                     inverse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qorder_kernel, dim3(1), dim3(kQThreads), 0, s, order, n, q_start, q_valid,
                     q_order, q_inverse);
  return hipGetLastError();
}

hipError_t launch_permute_rows(int heads, int64_t rows, int row_bytes, const int32_t* idx,
                               const void* src, int64_t src_rows, void* dst, int64_t dst_rows,
                               bool wide, hipStream_t s) {
  const int64_t chunks = (int64_t)heads * dst_rows * (row_bytes / (wide ? 16 : 4));
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((chunks + 255) / 256, 8192));
  if (wide) {
    hipLaunchKernelGGL(permute_kernel<uint4>, dim3(grid), dim3(256), 0, s, heads, rows,
                       row_bytes / 16, idx, (const uint4*)src, src_rows, (uint4*)dst, dst_rows);
  } else {
    hipLaunchKernelGGL(permute_kernel<uint32_t>, dim3(grid), dim3(256), 0, s, heads, rows,
                       row_bytes / 4, idx, (const uint32_t*)src, src_rows, (uint32_t*)dst,
                       dst_rows);
  }
  return hipGetLastError();
}

}  // namespace sa
