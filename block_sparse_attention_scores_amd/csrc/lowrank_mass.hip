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
//   (projections: launch_token_projection, fp64 sums rounded to fp32 and
//    stored as bf16 hi + lo)
//   block_lse_kernel   one workgroup per (head, query block, run of key
//                      blocks); each wave forms S^T = K~ Q~^T for its 32 query
//                      tokens against a key block (split-bf16 matrix-core
//                      products, token_mma.h; keys as rows, so each lane
//                      holds one query's scores),
//                      masks keys past kv_valid, and writes L[a, j] (fp32,
//                      layout [H, nKB, q_rows]: 32 consecutive queries per
//                      store).
//   block_mass_kernel  one workgroup per (head, query block): LSE_a over j by
//                      one thread per query (online max and sum), then one
//                      thread per key block sums exp(L - LSE) over the valid
//                      queries in query order and writes S as fp64.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "token_mma.h"

namespace sa {
namespace {

constexpr int kTokWords = 32;   // bf16 hi and lo of the 16 components per token
constexpr int kRunKB = 16;      // key blocks per workgroup in block_lse_kernel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;

template <int B>
__global__ __launch_bounds__(256, 2) void block_lse_kernel(const uint16_t* __restrict__ qt,
                                                        const uint16_t* __restrict__ kt, int nkb,
                                                        int64_t q_rows, int64_t kv_rows,
                                                        int64_t kv_valid, float tau,
                                                        float* __restrict__ L) {
  constexpr int kTiles = B / 32;   // 32-key tiles per block
  const int h = blockIdx.z, i = blockIdx.y, j0 = blockIdx.x * kRunKB;
  const int wave = threadIdx.x / kWave, lane = lane_id(), g = lane >> 5, lr = lane & 31;
  if (wave >= kTiles) return;   // B = 64: two waves hold the block's queries
  const int jn = min(kRunKB, nkb - j0);
  const int64_t qrow = (int64_t)i * B + 32 * wave + lr;
  // B operand: this lane's query, rank components 8g .. 8g+7
  const token::Split bq = token::split_load(qt + ((int64_t)h * q_rows + qrow) * kTokWords, g);
  const float tl = tau * kLog2e;   // logits in log2 units: z * log2(e) = tl * score
  for (int jj = 0; jj < jn; ++jj) {
    const int j = j0 + jj;
    const int64_t key0 = (int64_t)j * B;
    // valid keys of this block (uniform); only the last block is ragged
    const int lim = (int)min<int64_t>(B, kv_valid - key0);
    f32x16 acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const token::Split ak =
          token::split_load(kt + ((int64_t)h * kv_rows + key0 + 32 * t + lr) * kTokWords, g);
      acc[t] = token::scores(ak, bq);
    }
    // reg r of tile t: key 32t + 8(r/4) + 4g + r%4 of the block, this lane's query
    if (__builtin_expect(lim < B, 0)) {
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + 8 * (r >> 2) + 4 * g + (r & 3) >= lim) acc[t][r] = -INFINITY;
    }
    // max of the raw scores (tl > 0), then exp2(tl * s - tl * max) as one FMA
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float off = -mx * tl;
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[t][r], tl, off));
    sum += __shfl_xor(sum, 32, kWave);
    // every block holds a valid key, so mx is finite and sum >= 1
    if (g == 0) L[((int64_t)h * nkb + j) * q_rows + qrow] = (mx * tl + __log2f(sum)) * kLn2;
  }
}

__global__ __launch_bounds__(256) void block_mass_kernel(const float* __restrict__ L, int nqb,
                                                         int nkb, int B, int64_t q_rows,
                                                         int64_t q_valid,
                                                         double* __restrict__ S) {
  __shared__ float lse[128];
  const int h = blockIdx.y, i = blockIdx.x, t = threadIdx.x;
  const int64_t q0 = (int64_t)i * B;
  const int n_valid = (int)min<int64_t>(B, q_valid - q0);
  const float* Lh = L + (int64_t)h * nkb * q_rows + q0;
  if (t < B) {
    float m = -INFINITY, s = 0.f;
    if (t < n_valid) {
      for (int j = 0; j < nkb; ++j) {
        const float v = Lh[(int64_t)j * q_rows + t];
        if (v > m) {
          s = s * __expf(m - v) + 1.f;
          m = v;
        } else {
          s += __expf(v - m);
        }
      }
    }
    lse[t] = t < n_valid ? m + __logf(s) : INFINITY;   // +inf: the query adds nothing
  }
  __syncthreads();
  for (int j = t; j < nkb; j += blockDim.x) {
    const float4* row = reinterpret_cast<const float4*>(Lh + (int64_t)j * q_rows);
    float acc = 0.f;
    for (int c = 0; c < B / 4; ++c) {
      const float4 v = row[c];
      acc += __expf(v.x - lse[4 * c]);
      acc += __expf(v.y - lse[4 * c + 1]);
      acc += __expf(v.z - lse[4 * c + 2]);
      acc += __expf(v.w - lse[4 * c + 3]);
    }
    const double m = (double)acc / n_valid;
    S[((int64_t)h * nqb + i) * nkb + j] = m > 0.0 ? log(m) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_lowrank_mass(const Dims& g, const void* q, const void* k, const float* wq,
                               const float* wk, float tau, uint16_t* qtok, uint16_t* ktok,
                               float* lbuf, double* scores, hipStream_t s) {
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
