// Rank-16 token-pair scores on the bf16 matrix cores for the token-level
// estimators.  Each fp32 projection component x is stored split into bf16
// hi = RNE(x) and lo = RNE(x - hi); a lane holds 8 consecutive components of
// one token (the k = 8g .. 8g+7 slice of v_mfma_f32_32x32x16_bf16 for lane
// group g), and hi.hi + hi.lo + lo.hi is accumulated in fp32 (smallest terms
// first).  The products are exact in
// fp32; the split represents x to 2^-18 relative and the dropped lo.lo term
// is below 2^-18 |q_c k_c|, so with fp32 accumulation a 16-term score is
// within about 2^-16 sum_c |q_c k_c| of the exact one.
#ifndef SA_TOKEN_MMA_H
#define SA_TOKEN_MMA_H

#include "sa_common.h"

namespace sa {
namespace token {

typedef __attribute__((ext_vector_type(8))) float f32v8;

struct Split {
  bf16x8 hi, lo;
};

// A token as stored by the projection: 16 bf16 hi components, then the 16 bf16
// lo components (64 bytes, 16-byte aligned).  Lane group g takes components
// 8g .. 8g+7 of each.
__device__ __forceinline__ Split split_load(const uint16_t* tok, int g) {
  const uint4 hi = reinterpret_cast<const uint4*>(tok)[g];
  const uint4 lo = reinterpret_cast<const uint4*>(tok)[2 + g];
  return {__builtin_bit_cast(bf16x8, hi), __builtin_bit_cast(bf16x8, lo)};
}

// fp32 x -> bf16 hi = RNE(x), lo = RNE(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void split_store(const float* x, uint16_t* tok) {
  f32v8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = x[k];
    b[k] = x[8 + k];
  }
  const bf16x8 ha = __builtin_convertvector(a, bf16x8), hb = __builtin_convertvector(b, bf16x8);
  const bf16x8 la = __builtin_convertvector(a - __builtin_convertvector(ha, f32v8), bf16x8);
  const bf16x8 lb = __builtin_convertvector(b - __builtin_convertvector(hb, f32v8), bf16x8);
  uint4* o = reinterpret_cast<uint4*>(tok);
  o[0] = __builtin_bit_cast(uint4, ha);
  o[1] = __builtin_bit_cast(uint4, hb);
  o[2] = __builtin_bit_cast(uint4, la);
  o[3] = __builtin_bit_cast(uint4, lb);
}

// 32 x 32 tile: rows from a (m = lane % 32), columns from b (n = lane % 32);
// lane l holds column l % 32, rows 8(r/4) + 4(l/32) + r%4 in register r
__device__ __forceinline__ f32x16 scores(const Split& a, const Split& b) {
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.lo, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b.lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b.hi, acc, 0, 0, 0);
  return acc;
}

}  // namespace token
}  // namespace sa

#endif
