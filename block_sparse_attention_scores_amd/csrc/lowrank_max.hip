// Token-level low-rank predictor with max aggregation ("Dynamic Sparsity in
// Large-Scale Video DiT Training", section "The idea": query-key scores are
// predicted token by token through two rank-16 matrices and the critical
// pairs are kept).  The block pair's score is its largest predicted
// token-pair score (q_a W_q) . (k_b W_k).
//
//   project_kernel  X~[h, row, :] = X[h, src, :] W[h], fp64 sums (in input
//                   order) rounded to fp32 and stored split into bf16 hi and
//                   lo (token_mma.h); one thread per row with W[h] in LDS.
//                   src = row for valid rows, else the first row of the
//                   row's block: a duplicate token cannot change a max, so
//                   the block maxima need no masking.
//   blockmax_kernel one workgroup per (head, query block, run of key blocks);
//                   each wave scores its 32 query tokens against the 128 keys
//                   of a key block (split-bf16 matrix-core products, see
//                   token_mma.h) and keeps the max of the 32 x 128 outputs;
//                   the four wave maxima combine in LDS.
#include <float.h>

#include <algorithm>

#include "token_mma.h"

namespace sa {
namespace {

constexpr int kTokRank = 16;
constexpr int kTokWords = 2 * kTokRank;   // bf16 hi and lo per token
constexpr int kRunKB = 32;   // key blocks per workgroup


__device__ __forceinline__ void load8(const uint16_t* p, double* x) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = (double)__uint_as_float(w[k] << 16);
    x[2 * k + 1] = (double)__uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, double* x) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

constexpr int kProjRows = 256;   // rows (threads) per workgroup

template <typename T>
__global__ __launch_bounds__(kProjRows) void project_kernel(const T* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            int64_t rows, int64_t valid, int D,
                                                            int B, uint16_t* __restrict__ xt) {
  __shared__ double wl[128 * kTokRank];   // W[h] as fp64, [e][c]
  const int h = blockIdx.y;
  for (int u = threadIdx.x; u < D * kTokRank; u += kProjRows)
    wl[u] = (double)w[(int64_t)h * D * kTokRank + u];
  __syncthreads();
  const int64_t row = (int64_t)blockIdx.x * kProjRows + threadIdx.x;
  if (row >= rows) return;   // no barrier below
  const int64_t src = row < valid ? row : (row / B) * B;
  const T* xr = x + ((int64_t)h * rows + src) * D;
  double acc[kTokRank];
#pragma unroll
  for (int c = 0; c < kTokRank; ++c) acc[c] = 0.0;
  for (int e0 = 0; e0 < D; e0 += 8) {
    double xe[8];
    load8(xr + e0, xe);
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int c = 0; c < kTokRank; ++c) acc[c] = fma(xe[k], wl[(e0 + k) * kTokRank + c], acc[c]);
  }
  float xf[kTokRank];
#pragma unroll
  for (int c = 0; c < kTokRank; ++c) xf[c] = (float)acc[c];
  token::split_store(xf, xt + ((int64_t)h * rows + row) * kTokWords);
}

__global__ __launch_bounds__(256, 2) void blockmax_kernel(const uint16_t* __restrict__ qt,
                                                       const uint16_t* __restrict__ kt, int nqb,
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
    const token::Split a =
        token::split_load(qt + ((int64_t)h * q_rows + (int64_t)i * B + 32 * wave + lr) * kTokWords, g);
    for (int jj = 0; jj < jn; ++jj) {
      const int64_t kb = (int64_t)h * kv_rows + (int64_t)(j0 + jj) * B;
      float mx = -FLT_MAX;
      for (int t = 0; t < ktiles; ++t) {
        const token::Split b = token::split_load(kt + (kb + 32 * t + lr) * kTokWords, g);
        const f32x16 acc = token::scores(a, b);
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
                   uint16_t* xt, hipStream_t s) {
  const dim3 grid((unsigned)((rows + kProjRows - 1) / kProjRows), H);
  hipLaunchKernelGGL(project_kernel<T>, grid, dim3(kProjRows), 0, s, x, w, rows, valid, D, B, xt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_projection(const Dims& g, const void* q, const void* k, const float* wq,
                                   const float* wk, uint16_t* qtok, uint16_t* ktok, hipStream_t s) {
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
                              const float* wk, uint16_t* qtok, uint16_t* ktok, double* scores,
                              hipStream_t s) {
  const hipError_t e = launch_token_projection(g, q, k, wq, wk, qtok, ktok, s);
  if (e != hipSuccess) return e;
  const dim3 grid((g.nkb + kRunKB - 1) / kRunKB, g.nqb, g.H);
  hipLaunchKernelGGL(blockmax_kernel, grid, dim3(256), 0, s, qtok, ktok, g.nqb, g.nkb, g.B,
                     g.q_rows, g.kv_rows, scores);
  return hipGetLastError();
}

}  // namespace sa
