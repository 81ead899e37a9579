// Rank-16 token-pair scores of the token-level estimators on the fp64 matrix
// cores (v_mfma_f64_16x16x4_f64).  A token's projection x~ = x W is 16 fp64
// components (128 bytes, rows of [H, rows, 16]).  One 16 x 16 tile of scores
// is four MFMA steps; at step s, lane group g = lane / 16 supplies component
// 4s + g of the token in row lane % 16 of each operand.  Products and sums are
// fp64, so a score is the fp64 dot product up to the order of its 16 terms.
#ifndef SA_TOKEN_F64_H
#define SA_TOKEN_F64_H

#include "sa_common.h"

namespace sa {
namespace token {

constexpr int kRank = 16;
constexpr int kRow = 18;   // LDS row of one token's projection: 16 doubles + 2 of padding

typedef __attribute__((ext_vector_type(4))) double f64x4;

// Projections of n consecutive tokens (src: n rows of 16 doubles, 16-byte
// aligned) into LDS rows of kRow doubles, by all threads of the workgroup.
__device__ __forceinline__ void stage(const double* __restrict__ src, double* lds, int n) {
  const double2* s2 = reinterpret_cast<const double2*>(src);
  for (int p = threadIdx.x; p < n * (kRank / 2); p += blockDim.x) {
    const int r = p / (kRank / 2), c = 2 * (p % (kRank / 2));
    const double2 v = s2[p];
    lds[r * kRow + c] = v.x;
    lds[r * kRow + c + 1] = v.y;
  }
}

// This lane's four operand values (steps 0..3) of the token in LDS row `row`.
__device__ __forceinline__ void operand_lds(const double* lds, int row, int g, double (&o)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) o[s] = lds[row * kRow + 4 * s + g];
}

// ... of a token row in global memory (16 doubles).
__device__ __forceinline__ void operand_global(const double* __restrict__ tok, int g,
                                               double (&o)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) o[s] = tok[4 * s + g];
}

// 16 x 16 scores D[m][n] = <a_m, b_n>: a from the lane with lane % 16 = m, b
// from the lane with lane % 16 = n.  Lane l holds D[4q + l/16][l % 16] in
// element q.
__device__ __forceinline__ f64x4 tile(const double (&a)[4], const double (&b)[4]) {
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const int2 w = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(__shfl_xor(w.x, m, kWave), __shfl_xor(w.y, m, kWave)));
}

}  // namespace token
}  // namespace sa

#endif
