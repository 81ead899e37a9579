// Token-level low-rank predictor with max aggregation ("Dynamic Sparsity in
// Large-Scale Video DiT Training", section "The idea": query-key scores are
// predicted token by token through two rank-16 matrices and the critical
// pairs are kept).  The block pair's score is its largest predicted
// token-pair score (q_a W_q) . (k_b W_k).
//
//   project_kernel   X~[h, row, :] = X[h, src, :] W[h], fp64 sums in input
//                    order, stored as 16 fp64 (128 bytes per token); one
//                    thread per row with W[h] in LDS.  src = row for valid
//                    rows, else the first row of the row's block: a
//                    duplicate token cannot change a max, so the block
//                    maxima need no masking (the mass estimator masks).
//   blockmax_kernel  one workgroup per (head, query block, run of key
//                    blocks); each key block's projections are staged in LDS
//                    (double-buffered) and each wave scores its query tokens
//                    against the block's keys on the fp64 matrix cores
//                    (token_f64.h), keeping the max; the wave maxima combine
//                    in LDS.  Scores are fp64 dot products of fp64
//                    projections, so the block maxima are exact to fp64
//                    rounding.
#include <float.h>

#include <algorithm>

#include "token_f64.h"

namespace sa {
namespace {

using token::kRank;
using token::kRow;
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
                                                            int B, double* __restrict__ xt) {
  __shared__ double wl[128 * kRank];   // W[h] as fp64, [e][c]
  const int h = blockIdx.y;
  for (int u = threadIdx.x; u < D * kRank; u += kProjRows)
    wl[u] = (double)w[(int64_t)h * D * kRank + u];
  __syncthreads();
  const int64_t row = (int64_t)blockIdx.x * kProjRows + threadIdx.x;
  if (row >= rows) return;   // no barrier below
  const int64_t src = row < valid ? row : (row / B) * B;
  const T* xr = x + ((int64_t)h * rows + src) * D;
  double acc[kRank];
#pragma unroll
  for (int c = 0; c < kRank; ++c) acc[c] = 0.0;
  for (int e0 = 0; e0 < D; e0 += 8) {
    double xe[8];
    load8(xr + e0, xe);
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int c = 0; c < kRank; ++c) acc[c] = fma(xe[k], wl[(e0 + k) * kRank + c], acc[c]);
  }
  double2* o = reinterpret_cast<double2*>(xt + ((int64_t)h * rows + row) * kRank);
#pragma unroll
  for (int c = 0; c < kRank / 2; ++c) o[c] = make_double2(acc[2 * c], acc[2 * c + 1]);
}

// B = 128: each wave owns two 16-token query tiles; B = 64: one.
template <int B>
__global__ __launch_bounds__(256, 2) void blockmax_kernel(const double* __restrict__ qt,
                                                       const double* __restrict__ kt, int nqb,
                                                       int nkb, int64_t q_rows, int64_t kv_rows,
                                                       double* __restrict__ S) {
  constexpr int QT = B / 64, KT = B / 16;
  __shared__ double ks[2][B * kRow];
  __shared__ double wmax[4][kRunKB];
  const int h = blockIdx.z, i = blockIdx.y, j0 = blockIdx.x * kRunKB;
  const int wave = threadIdx.x / kWave, lane = lane_id(), g = lane >> 4, r = lane & 15;
  const int jn = min(kRunKB, nkb - j0);
  double a[QT][4];
#pragma unroll
  for (int t = 0; t < QT; ++t)
    token::operand_global(qt + ((int64_t)h * q_rows + (int64_t)i * B + 16 * (QT * wave + t) + r) * kRank,
                          g, a[t]);
  const double* kh = kt + (int64_t)h * kv_rows * kRank;
  token::stage(kh + (int64_t)j0 * B * kRank, ks[0], B);
  __syncthreads();
  for (int jj = 0; jj < jn; ++jj) {
    // the other buffer was last read before the previous barrier
    if (jj + 1 < jn) token::stage(kh + (int64_t)(j0 + jj + 1) * B * kRank, ks[(jj + 1) & 1], B);
    const double* kb = ks[jj & 1];
    double mx = -DBL_MAX;
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      double b[4];
      token::operand_lds(kb, 16 * u + r, g, b);
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const token::f64x4 d = token::tile(a[t], b);
        mx = fmax(mx, fmax(fmax(d[0], d[1]), fmax(d[2], d[3])));
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmax(mx, token::shfl_xor_f64(mx, m));
    if (lane == 0) wmax[wave][jj] = mx;
    __syncthreads();
  }
  for (int t = threadIdx.x; t < jn; t += blockDim.x)
    S[((int64_t)h * nqb + i) * nkb + j0 + t] =
        fmax(fmax(wmax[0][t], wmax[1][t]), fmax(wmax[2][t], wmax[3][t]));
}

template <typename T>
hipError_t project(const T* x, const float* w, int H, int64_t rows, int64_t valid, int D, int B,
                   double* xt, hipStream_t s) {
  const dim3 grid((unsigned)((rows + kProjRows - 1) / kProjRows), H);
  hipLaunchKernelGGL(project_kernel<T>, grid, dim3(kProjRows), 0, s, x, w, rows, valid, D, B, xt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_projection(const Dims& g, const void* q, const void* k, const float* wq,
                                   const float* wk, double* qtok, double* ktok, hipStream_t s) {
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
                              const float* wk, double* qtok, double* ktok, double* scores,
                              hipStream_t s) {
  const hipError_t e = launch_token_projection(g, q, k, wq, wk, qtok, ktok, s);
  if (e != hipSuccess) return e;
  const dim3 grid((g.nkb + kRunKB - 1) / kRunKB, g.nqb, g.H);
  if (g.B == 128)
    hipLaunchKernelGGL(blockmax_kernel<128>, grid, dim3(256), 0, s, qtok, ktok, g.nqb, g.nkb,
                       g.q_rows, g.kv_rows, scores);
  else
    hipLaunchKernelGGL(blockmax_kernel<64>, grid, dim3(256), 0, s, qtok, ktok, g.nqb, g.nkb,
                       g.q_rows, g.kv_rows, scores);
  return hipGetLastError();
}

}  // namespace sa
