// Token-level low-rank predictor aggregated by predicted softmax mass
// ("Dynamic Sparsity in Large-Scale Video DiT Training", section "The idea":
// query-key scores are predicted token by token through two rank-16 matrices
// in place of the full scores).  The predicted scores, scaled by the
// selection temperature tau, are read as attention logits:
//
//   z_ab    = tau * (q_a W_q) . (k_b W_k)            valid keys b only
//   L[a, j] = ln sum_{b in key block j} exp(z_ab)     (per query token, per key block)
//   LSE_a   = ln sum_j exp(L[a, j])
//   M[i, j] = (1 / n_i) sum_{valid a in query block i} exp(L[a, j] - LSE_a)
//   S[i, j] = ln M[i, j]
//
// so that a softmax over a row of S gives back the masses (each row of M sums
// to one) and top-k keeps the largest masses.
//
//   (projections: launch_token_projection, fp64)
//   block_lse_kernel   one workgroup per (head, query block, run of key
//                      blocks); each key block's projections are staged in LDS
//                      (double-buffered); each wave forms the fp64 scores of
//                      its query tokens against the block's keys on the fp64
//                      matrix cores (keys as rows, so a lane holds 4 keys of
//                      one query per 16-key tile), masks keys past kv_valid
//                      and writes L[a, j] in fp64 (layout [H, nKB, q_rows]).
//                      Each exponential is 2^n * exp2(f) with n an integer and
//                      f in [-1, 0] formed exactly in fp64, f rounded to fp32
//                      (2^-25 absolute) and exp2 in fp32; the sums are fp64.
//                      So L is within about 2^-23 of the exact value.
//   block_mass_kernel  one workgroup per (head, query block): LSE_a over j by
//                      one thread per query (online max and sum, fp64), then
//                      one thread per key block sums exp(L - LSE) over the
//                      valid queries in query order (fp64) and writes S.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "token_f64.h"

namespace sa {
namespace {

using token::kRank;
using token::kRow;
constexpr int kRunKB = 16;      // key blocks per workgroup in block_lse_kernel
constexpr double kLog2e = 1.4426950408889634074;

// exp(x) for x <= 0 to about 2^-23 relative: x log2 e = n + f with n an
// integer and f in [-1, 0] (exact up to the fp64 product), exp2(f) in fp32.
__device__ __forceinline__ double exp_nonpos(double x) {
  const double y = x * kLog2e;
  if (y < -1000.0) return 0.0;
  const double n = ceil(y);
  const float f = (float)(y - n);
  return ldexp((double)__builtin_amdgcn_exp2f(f), (int)n);
}

// B = 128: each wave owns two 16-token query tiles; B = 64: one.
template <int B>
__global__ __launch_bounds__(256, 2) void block_lse_kernel(const double* __restrict__ qt,
                                                        const double* __restrict__ kt, int nkb,
                                                        int64_t q_rows, int64_t kv_rows,
                                                        int64_t kv_valid, double tau,
                                                        double* __restrict__ L) {
  constexpr int QT = B / 64, KT = B / 16;
  __shared__ double ks[2][B * kRow];
  const int h = blockIdx.z, i = blockIdx.y, j0 = blockIdx.x * kRunKB;
  const int wave = threadIdx.x / kWave, lane = lane_id(), g = lane >> 4, r = lane & 15;
  const int jn = min(kRunKB, nkb - j0);
  // B operands: this lane supplies query token 16 (QT wave + t) + r of the block
  double bq[QT][4];
#pragma unroll
  for (int t = 0; t < QT; ++t)
    token::operand_global(qt + ((int64_t)h * q_rows + (int64_t)i * B + 16 * (QT * wave + t) + r) * kRank,
                          g, bq[t]);
  const double* kh = kt + (int64_t)h * kv_rows * kRank;
  token::stage(kh + (int64_t)j0 * B * kRank, ks[0], B);
  __syncthreads();
  for (int jj = 0; jj < jn; ++jj) {
    const int j = j0 + jj;
    if (jj + 1 < jn) token::stage(kh + (int64_t)(j + 1) * B * kRank, ks[(jj + 1) & 1], B);
    const double* kb = ks[jj & 1];
    // valid keys of this block (uniform); only the last block is ragged
    const int lim = (int)min<int64_t>(B, kv_valid - (int64_t)j * B);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      // tile u, element q: key 16u + 4q + g of the block, query r of tile t
      token::f64x4 z[KT];
#pragma unroll
      for (int u = 0; u < KT; ++u) {
        double a[4];
        token::operand_lds(kb, 16 * u + r, g, a);
        z[u] = token::tile(a, bq[t]);
      }
      double mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < KT; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (16 * u + 4 * q + g < lim) mx = fmax(mx, z[u][q]);
      mx = fmax(mx, token::shfl_xor_f64(mx, 16));
      mx = fmax(mx, token::shfl_xor_f64(mx, 32));
      double sum = 0.0;
#pragma unroll
      for (int u = 0; u < KT; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (16 * u + 4 * q + g < lim) sum += exp_nonpos(tau * (z[u][q] - mx));
      sum += token::shfl_xor_f64(sum, 16);
      sum += token::shfl_xor_f64(sum, 32);
      // every block holds a valid key, so mx is finite and sum >= 1
      if (g == 0)
        L[((int64_t)h * nkb + j) * q_rows + (int64_t)i * B + 16 * (QT * wave + t) + r] =
            tau * mx + log(sum);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void block_mass_kernel(const double* __restrict__ L, int nqb,
                                                         int nkb, int B, int64_t q_rows,
                                                         int64_t q_valid,
                                                         double* __restrict__ S) {
  __shared__ double lse[128];
  const int h = blockIdx.y, i = blockIdx.x, t = threadIdx.x;
  const int64_t q0 = (int64_t)i * B;
  const int n_valid = (int)min<int64_t>(B, q_valid - q0);
  const double* Lh = L + (int64_t)h * nkb * q_rows + q0;
  if (t < B) {
    double m = -INFINITY, s = 0.0;
    if (t < n_valid) {
      for (int j = 0; j < nkb; ++j) {
        const double v = Lh[(int64_t)j * q_rows + t];
        if (v > m) {
          s = s * exp(m - v) + 1.0;
          m = v;
        } else {
          s += exp(v - m);
        }
      }
    }
    lse[t] = t < n_valid ? m + log(s) : INFINITY;   // +inf: the query adds nothing
  }
  __syncthreads();
  for (int j = t; j < nkb; j += blockDim.x) {
    const double2* row = reinterpret_cast<const double2*>(Lh + (int64_t)j * q_rows);
    double acc = 0.0;
    for (int c = 0; c < B / 2; ++c) {
      const double2 v = row[c];
      acc += exp(v.x - lse[2 * c]);
      acc += exp(v.y - lse[2 * c + 1]);
    }
    const double m = acc / n_valid;
    S[((int64_t)h * nqb + i) * nkb + j] = m > 0.0 ? log(m) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_lowrank_mass(const Dims& g, const void* q, const void* k, const float* wq,
                               const float* wk, double tau, double* qtok, double* ktok,
                               double* lbuf, double* scores, hipStream_t s) {
  hipError_t e = launch_token_projection(g, q, k, wq, wk, qtok, ktok, s);
  if (e != hipSuccess) return e;
  const dim3 grid((g.nkb + kRunKB - 1) / kRunKB, g.nqb, g.H);
  if (g.B == 128)
    hipLaunchKernelGGL(block_lse_kernel<128>, grid, dim3(256), 0, s, qtok, ktok, g.nkb, g.q_rows,
                       g.kv_rows, g.kv_valid, tau, lbuf);
  else
    hipLaunchKernelGGL(block_lse_kernel<64>, grid, dim3(256), 0, s, qtok, ktok, g.nkb, g.q_rows,
                       g.kv_rows, g.kv_valid, tau, lbuf);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_mass_kernel, dim3(g.nqb, g.H), dim3(256), 0, s, lbuf, g.nqb, g.nkb, g.B,
                     g.q_rows, g.q_valid, scores);
  return hipGetLastError();
}

}  // namespace sa
