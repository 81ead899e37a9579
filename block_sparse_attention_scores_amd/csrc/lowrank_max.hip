// Token-level low-rank predictor with max aggregation ("Dynamic Sparsity in
// Large-Scale Video DiT Training", section "The idea": query-key scores are
// predicted token by token through two rank-16 matrices and the critical
// pairs are kept).  The block pair's score is its largest predicted
// token-pair score (q_a W_q) . (k_b W_k).
//
//   project_kernel  X~[h, row, :] = X[h, src, :] W[h], fp64 sums stored as
//                   fp32.  src = row for valid rows, else the first row of
//                   the row's block: a duplicate token cannot change a max,
//                   so the block maxima need no masking.
//   blockmax_kernel one workgroup per (head, query block, run of key blocks);
//                   each wave scores its 32 query tokens against the 128 keys
//                   of a key block on v_mfma_f32_32x32x2_f32 (the inner index
//                   8g + s of lane group g at step s, the same on both
//                   operands), keeps the max of the 32 x 128 outputs, and the
//                   four wave maxima combine in LDS.
#include <float.h>

#include <algorithm>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kTokRank = 16;
constexpr int kRunKB = 32;   // key blocks per workgroup

__device__ __forceinline__ double elem(const uint16_t* x, int e) {
  return (double)__uint_as_float((uint32_t)x[e] << 16);
}
__device__ __forceinline__ double elem(const float* x, int e) { return (double)x[e]; }

template <typename T>
__global__ __launch_bounds__(256) void project_kernel(const T* __restrict__ x,
                                                      const float* __restrict__ w, int H,
                                                      int64_t rows, int64_t valid, int D, int B,
                                                      float* __restrict__ xt) {
  const int64_t total = (int64_t)H * rows * kTokRank;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(u % kTokRank);
    const int64_t hr = u / kTokRank;
    const int64_t row = hr % rows, h = hr / rows;
    const int64_t src = row < valid ? row : (row / B) * B;
    const T* xr = x + (h * rows + src) * D;
    const float* wh = w + h * D * kTokRank;
    double s = 0.0;
    for (int e = 0; e < D; ++e) s += elem(xr, e) * (double)wh[e * kTokRank + c];
    xt[u] = (float)s;
  }
}

__global__ __launch_bounds__(256) void blockmax_kernel(const float* __restrict__ qt,
                                                       const float* __restrict__ kt, int nqb,
                                                       int nkb, int B, int64_t q_rows,
                                                       int64_t kv_rows, double* __restrict__ S) {
  __shared__ float wmax[4][kRunKB];
  const int h = blockIdx.z, i = blockIdx.y, j0 = blockIdx.x * kRunKB;
  const int wave = threadIdx.x / kWave, lane = lane_id(), g = lane >> 5, lr = lane & 31;
  const int jn = min(kRunKB, nkb - j0);
  const int qtiles = B / 32;   // 32-token query tiles per block (2 or 4)
  const int ktiles = B / 32;
  for (int jj = 0; jj < jn; ++jj) wmax[wave][jj] = -FLT_MAX;
  // waves beyond the block's query tiles (B = 64) keep -FLT_MAX
  if (wave < qtiles) {
    const float4* qa = reinterpret_cast<const float4*>(
        qt + ((int64_t)h * q_rows + (int64_t)i * B + 32 * wave + lr) * kTokRank + 8 * g);
    const float4 a0 = qa[0], a1 = qa[1];
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    for (int jj = 0; jj < jn; ++jj) {
      const int64_t kb = (int64_t)h * kv_rows + (int64_t)(j0 + jj) * B;
      float mx = -FLT_MAX;
      for (int t = 0; t < ktiles; ++t) {
        const float4* kp = reinterpret_cast<const float4*>(kt + (kb + 32 * t + lr) * kTokRank + 8 * g);
        const float4 b0 = kp[0], b1 = kp[1];
        const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
      }
      mx = wave_reduce(mx, [](float x, float y) { return fmaxf(x, y); });
      if (lane == 0) wmax[wave][jj] = mx;
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < jn; t += blockDim.x) {
    const float m = fmaxf(fmaxf(wmax[0][t], wmax[1][t]), fmaxf(wmax[2][t], wmax[3][t]));
    S[((int64_t)h * nqb + i) * nkb + j0 + t] = (double)m;
  }
}

template <typename T>
hipError_t project(const T* x, const float* w, int H, int64_t rows, int64_t valid, int D, int B,
                   float* xt, hipStream_t s) {
  const int64_t total = (int64_t)H * rows * kTokRank;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 16384);
  hipLaunchKernelGGL(project_kernel<T>, dim3(grid), dim3(256), 0, s, x, w, H, rows, valid, D, B,
                     xt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_projection(const Dims& g, const void* q, const void* k, const float* wq,
                                   const float* wk, float* qtok, float* ktok, hipStream_t s) {
  hipError_t e;
  if (g.dtype == SA_BF16) {
    e = project((const uint16_t*)q, wq, g.H, g.q_rows, g.q_valid, g.d, g.B, qtok, s);
    if (e == hipSuccess) e = project((const uint16_t*)k, wk, g.H, g.kv_rows, g.kv_valid, g.d, g.B, ktok, s);
  } else {
    e = project((const float*)q, wq, g.H, g.q_rows, g.q_valid, g.d, g.B, qtok, s);
    if (e == hipSuccess) e = project((const float*)k, wk, g.H, g.kv_rows, g.kv_valid, g.d, g.B, ktok, s);
  }
  return e;
}

hipError_t launch_lowrank_max(const Dims& g, const void* q, const void* k, const float* wq,
                              const float* wk, float* qtok, float* ktok, double* scores,
                              hipStream_t s) {
  const hipError_t e = launch_token_projection(g, q, k, wq, wk, qtok, ktok, s);
  if (e != hipSuccess) return e;
  const dim3 grid((g.nkb + kRunKB - 1) / kRunKB, g.nqb, g.H);
  hipLaunchKernelGGL(blockmax_kernel, grid, dim3(256), 0, s, qtok, ktok, g.nqb, g.nkb, g.B,
                     g.q_rows, g.kv_rows, scores);
  return hipGetLastError();
}

}  // namespace sa
