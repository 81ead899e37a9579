// Device-side helpers shared by the HIP kernels of the sparse attention path
// (gfx950, wave64).  Host launchers of every translation unit are declared at
// the end and called from api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// bf16 <-> fp32 on raw 16-bit patterns (bf16 is the top half of an fp32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Block-wide reductions and scans over blockDim.x threads (a multiple of 64).
// `scratch` holds at least blockDim.x/64 elements of T.  Every thread gets the
// result.  The order of combination is fixed, so results are deterministic.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = op(v, __shfl_xor(v, off, kWave));
  return v;
}

template <typename T, typename Op>
__device__ T block_reduce(T v, T* scratch, Op op) {
  v = wave_reduce(v, op);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (lane_id() == 0) scratch[w] = v;
  __syncthreads();
  T r = scratch[0];
  for (int i = 1; i < nw; ++i) r = op(r, scratch[i]);
  return r;
}

// Inclusive scan within a wave (Hillis-Steele over shuffles).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    T o = __shfl_up(v, off, kWave);
    if (l >= off) v = v + o;
  }
  return v;
}

// Inclusive block scan; `scratch` >= blockDim.x/64 + 1 elements.  Returns the
// inclusive prefix for this thread and writes the block total to *total.
template <typename T>
__device__ T block_inclusive_scan(T v, T* scratch, T* total) {
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  T inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane_id() == kWave - 1) scratch[w] = inc;
  __syncthreads();
  T base = T(0), all = T(0);
  for (int i = 0; i < nw; ++i) {
    if (i < w) base = base + scratch[i];
    all = all + scratch[i];
  }
  *total = all;
  return base + inc;
}

}  // namespace sa

// ---- host launchers (one per translation unit), used by api.hip ----------
namespace sa {
struct Dims {
  int H, d, B, nqb, nkb, W, rank;   // rank: of the projected block means (0: none)
  int score_mode;
  int64_t q_rows, q_valid, kv_rows, kv_valid;
  int dtype;
};

hipError_t launch_pool(const Dims& g, const void* q, const void* k, const float* wq,
                       const float* wk, double* qbar, double* kbar, double* qt, double* kt,
                       hipStream_t s);
hipError_t launch_scores(const Dims& g, const double* qx, const double* kx, int inner,
                         double scale, double* scores, hipStream_t s);
hipError_t launch_select(const Dims& g, const double* scores, int mode, double top_p,
                         int top_k, uint32_t* bits, int32_t* counts, hipStream_t s);
hipError_t launch_count_bits(const Dims& g, const uint32_t* bits, int32_t* counts,
                             hipStream_t s);
hipError_t launch_csr(const Dims& g, const uint32_t* bits, const int32_t* counts,
                      int32_t* row_ptr, int32_t* col_idx, hipStream_t s);
int mark_groups(const Dims& g);
hipError_t launch_demand(const Dims& g, const int32_t* row_ptr, const int32_t* col_idx,
                         uint32_t* part, int32_t* slot_of, int32_t* demand_ptr,
                         int32_t* demand_idx, int64_t cap, int32_t* dev_status, hipStream_t s);
hipError_t launch_pack(const Dims& g, const int32_t* demand_ptr, const int32_t* demand_idx,
                       const void* k, const void* v, void* kp, void* vp, int64_t cap,
                       const int32_t* row_ptr, const int32_t* col_idx, const int32_t* slot_of,
                       int32_t* col_slot, hipStream_t s);
// Work queue (longest first, per-XCD ranges) and attention in one call; ws
// holds attn_ws_bytes(g) bytes sized on the current device.
size_t attn_ws_bytes(const Dims& g);
// The work queue alone (whole items, never halves): what launch_attn needs
// when given exactly this many workspace bytes.
size_t attn_queue_ws_bytes(const Dims& g);
int attn_workgroups(const Dims& g, int schedule);
hipError_t launch_attn(const Dims& g, const void* q, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* col_slot, const void* k,
                       const void* v, void* out, float* lse, void* ws, size_t ws_bytes,
                       float sm_scale, int schedule, uint64_t* wg_clock, hipStream_t s);
// Fused estimation, selection (mode SA_TOP_P with a top_k floor, or SA_TOP_K)
// and attention (fused.hip): qx [H*nQB, dim] and kx [H*nKB, dim] fp64 (block
// means or their projections), S = scale * qx.kx.
hipError_t launch_fused(const Dims& g, const double* qx, const double* kx, int dim, double scale,
                        int mode, double top_p, int top_k, const void* q, const void* k,
                        const void* v, void* out, float* lse, uint32_t* mask_bits, float sm_scale,
                        int32_t* ctr, hipStream_t s);
hipError_t launch_video_order(int T, int Hl, int Wl, int tt, int th, int tw, int64_t q_start,
                              int64_t q_valid, int32_t* order, int32_t* inverse, int32_t* q_order,
                              int32_t* q_inverse, hipStream_t s);
hipError_t launch_permute_rows(int heads, int64_t rows, int row_bytes, const int32_t* idx,
                               const void* src, int64_t src_rows, void* dst, int64_t dst_rows,
                               bool wide, hipStream_t s);
hipError_t launch_backward(const Dims& g, const void* q, const void* k, const void* v,
                           const void* out, const void* dout, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, void* dq, void* dk,
                           void* dv, float* delta, uint32_t* bits, int32_t* counts,
                           int32_t* col_ptr, int32_t* row_idx, int32_t* order, float sm_scale,
                           hipStream_t s);
// Token projections for the token-level estimators: per token the 16 fp64
// components of x W (128 bytes).
hipError_t launch_token_projection(const Dims& g, const void* q, const void* k, const float* wq,
                                   const float* wk, double* qtok, double* ktok, hipStream_t s);
hipError_t launch_lowrank_mass(const Dims& g, const void* q, const void* k, const float* wq,
                               const float* wk, double tau, double* qtok, double* ktok,
                               double* lbuf, double* scores, hipStream_t s);
hipError_t launch_lowrank_max(const Dims& g, const void* q, const void* k, const float* wq,
                              const float* wk, double* qtok, double* ktok, double* scores,
                              hipStream_t s);
}  // namespace sa
