// Backward of the block-sparse attention (the training workload: the DSV
// explainer's speedups, "What it costs", are training numbers).  For the
// forward's P = softmax(z), z = sm_scale <q_a, k_b> over the selected blocks:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = sm_scale dS K,  dK = sm_scale dS^T Q.
// P is recomputed from the forward's LSE, never stored.
//
//   delta_kernel    D per query row (fp32), one wave per row
//   row_bits_kernel the block mask rebuilt from the CSR (one wave per row)
//   csc_*_kernel    the transpose of the block lists (per key block, the query
//                   blocks that selected it, ascending): count, scan, fill
//   lpt_order_kernel the dK/dV launch order: head by head, longest lists first
//   bwd_dq_kernel   one workgroup per (head, query block): over its CSR row,
//                   dP^T = V dO^T, then S^T = K Q^T, dS^T, dQ^T += K^T dS^T;
//                   the next V loads during the K phase and the next K during
//                   the next V phase
//   bwd_dkdv_kernel one workgroup per (head, key block), in that order: over its CSC column,
//                   S = Q K^T, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS;
//                   two LDS buffers, the next query block loads during compute;
//                   one wave per SIMD, so each wave runs its own software
//                   pipeline: the exponentials of tile t between the score
//                   MFMAs of tile t + 1
// In both, operand fragments are read from LDS a few MFMAs ahead of their use
// and scheduling fences hold the reads there.
// All GEMMs are v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are
// rounded to bf16 as MFMA operands.  Blocks arrive in LDS through direct loads
// with the K swizzle (logical 16-byte chunk c of row r at c ^ (r & 15)); the
// same rows are read either as MFMA A rows (ds_read_b128) or transposed
// (ds_read_b64_tr_b16).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "mfma_bf16.h"

namespace sa {
namespace {

using namespace bf16mma;

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    int64_t rows_total, int64_t q_rows,
                                                    int64_t q_valid, float* __restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows_total) return;   // whole wave
  float s = 0.f;
  if (row % q_rows < q_valid) {
    const uint32_t o2 = reinterpret_cast<const uint32_t*>(out + row * kD)[lane];
    const uint32_t d2 = reinterpret_cast<const uint32_t*>(dout + row * kD)[lane];
    s = fmaf(bf16_lo(o2), bf16_lo(d2), bf16_hi(o2) * bf16_hi(d2));
  }
  s = wave_reduce(s, [](float a, float b) { return a + b; });
  if (lane == 0) delta[row] = s;
}

// The block mask rebuilt from the CSR: one wave per row ORs its column ids
// into LDS words (ids outside [0, nkb) are ignored), then writes the row.
constexpr int kBitsWaves = 4;
constexpr int kMaxWords = 4096 / 32;
__global__ __launch_bounds__(kBitsWaves * kWave) void row_bits_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int rows, int nkb,
    int W, uint32_t* __restrict__ bits) {
  __shared__ uint32_t words[kBitsWaves][kMaxWords];
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r = blockIdx.x * kBitsWaves + wv;
  if (r >= rows) return;   // whole wave; no workgroup barrier below
  for (int w = lane; w < W; w += kWave) words[wv][w] = 0u;
  __builtin_amdgcn_wave_barrier();
  const int e1 = row_ptr[r + 1];
  for (int e = row_ptr[r] + lane; e < e1; e += kWave) {
    const int j = col_idx[e];
    if ((unsigned)j < (unsigned)nkb) atomicOr(&words[wv][j >> 5], 1u << (j & 31));
  }
  __builtin_amdgcn_wave_barrier();
  for (int w = lane; w < W; w += kWave) bits[(int64_t)r * W + w] = words[wv][w];
}

// per key block (h, j): the query blocks i whose mask row has bit j, ascending;
// count only (fill == false) or write them at col_ptr (fill == true)
template <bool kFill>
__global__ __launch_bounds__(256) void csc_kernel(const uint32_t* __restrict__ bits, int H,
                                                  int nqb, int nkb, int W,
                                                  const int32_t* __restrict__ col_ptr,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ row_idx) {
  for (int u = blockIdx.x * blockDim.x + threadIdx.x; u < H * nkb; u += gridDim.x * blockDim.x) {
    const int h = u / nkb, j = u % nkb;
    const uint32_t* b = bits + (int64_t)h * nqb * W + (j >> 5);
    const uint32_t m = 1u << (j & 31);
    int c = 0, o = kFill ? col_ptr[u] : 0;
#pragma unroll 8
    for (int i = 0; i < nqb; ++i) {
      const bool hit = (b[(int64_t)i * W] & m) != 0;
      if (kFill && hit) row_idx[o + c] = i;
      c += hit ? 1 : 0;
    }
    if (!kFill) counts[u] = c;
  }
}

constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void csc_scan_kernel(const int32_t* __restrict__ counts,
                                                                int n, int32_t* __restrict__ col_ptr) {
  __shared__ int scratch[kScanThreads / kWave + 1];
  int base = 0;
  for (int p0 = 0; p0 < n; p0 += kScanThreads) {
    const int p = p0 + threadIdx.x;
    const int c = p < n ? counts[p] : 0;
    int total;
    const int incl = block_inclusive_scan(c, scratch, &total);
    if (p < n) col_ptr[p] = base + incl - c;
    base += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) col_ptr[n] = base;
}

// Launch order of the dK/dV workgroups: head by head, and within a head the
// key blocks by descending column length (longest first, so that the long
// columns do not finish last, while the workgroups in flight still share one
// head's Q and dO in the caches).  One workgroup per head counts lengths
// 0..nqb into LDS bins; units of equal length land in the order their atomic
// increments happen, which changes nothing but the schedule: every unit
// writes only its own dK and dV.  Without room for the bins, the natural order.
constexpr int kOrderThreads = 1024, kOrderBins = 4096;
__global__ __launch_bounds__(kOrderThreads) void lpt_order_kernel(const int32_t* __restrict__ counts,
                                                                   int nkb, int nqb,
                                                                   int32_t* __restrict__ order) {
  __shared__ int bins[kOrderBins];
  __shared__ int scratch[kOrderThreads / kWave + 1];
  const int t = threadIdx.x, nb = nqb + 1;
  const int64_t u0 = (int64_t)blockIdx.x * nkb;   // this head's first unit
  if (nb > kOrderBins) {
    for (int j = t; j < nkb; j += kOrderThreads) order[u0 + j] = (int32_t)(u0 + j);
    return;
  }
  for (int b = t; b < nb; b += kOrderThreads) bins[b] = 0;
  __syncthreads();
  for (int j = t; j < nkb; j += kOrderThreads) atomicAdd(&bins[nb - 1 - counts[u0 + j]], 1);
  __syncthreads();
  // exclusive scan of the bins (index nb - 1 - length: longest first), in chunks
  int base = 0;
  for (int b0 = 0; b0 < nb; b0 += kOrderThreads) {
    const int b = b0 + t;
    const int c = b < nb ? bins[b] : 0;
    int total;
    const int incl = block_inclusive_scan(c, scratch, &total);
    __syncthreads();
    if (b < nb) bins[b] = base + incl - c;
    base += total;
    __syncthreads();
  }
  for (int j = t; j < nkb; j += kOrderThreads)
    order[u0 + atomicAdd(&bins[nb - 1 - counts[u0 + j]], 1)] = (int32_t)(u0 + j);
}

// ---------------------------------------------------------------------------
// lane-constant LDS offsets of one wave (K swizzle throughout)
struct Offsets {
  int dma[4];    // direct loads: row 4i + L/16, physical chunk L%16
  int rowa[8];   // A rows: row lq (+32t via immediate), logical chunk 2s + g
  int tr[4][2];  // transposed A: rows 4 kgb + e (kgb & 3 = g, g+2), columns 32u + 16(a&1) + 4q
};

__device__ __forceinline__ void make_offsets(Offsets& o, int lane) {
  const int lq = lane & 31, g = lane >> 5;
  const int rr = lane >> 4, pc = lane & 15;
#pragma unroll
  for (int p = 0; p < 4; ++p) o.dma[p] = rr * 256 + ((pc ^ (4 * p + rr)) << 4);
#pragma unroll
  for (int s = 0; s < 8; ++s) o.rowa[s] = lq * 256 + (((2 * s + g) ^ (lq & 15)) << 4);
  const int a = lane >> 4, jj = lane & 15, e = jj >> 2, qq = jj & 3;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kg = g + 2 * hh;              // low two bits of the row group
      const int c16 = 4 * u + 2 * (a & 1) + (qq >> 1);
      o.tr[u][hh] = 1024 * kg + 256 * e + ((c16 ^ (4 * kg + e)) << 4) + 8 * (qq & 1);
    }
}

// A operand rows 32t + lq of a swizzled tile, k-step s
__device__ __forceinline__ bf16x8 rows_a(const uint16_t* tile, const Offsets& o, int t, int s) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + o.rowa[s] +
                                          t * 8192);
}
// transposed A operand, columns 32u.. of the tile, rows of k-step (t, h2)
__device__ __forceinline__ bf16x8 cols_a(const uint16_t* tile, const Offsets& o, int u, int t,
                                         int h2) {
  const int rows = 1024 * (8 * t + 4 * h2);
  const u32x2 lo = lds_read_tr(tile, o.tr[u][0] + rows);
  const u32x2 hi = lds_read_tr(tile, o.tr[u][1] + rows);
  const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, w);
}

// fragments of row `row` (0..127) of one 128-row block of a [rows, 128] bf16
// tensor as the B operand: k-step s holds columns 16s + 8g .. +8 (the
// descriptor spans the block only, so its offsets stay small at any length)
__device__ __forceinline__ void load_b(bf16x8 (&f)[8], const uint16_t* block, int row, int g) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(block, kTileBytes);
#pragma unroll
  for (int s = 0; s < 8; ++s)
    f[s] = __builtin_bit_cast(bf16x8, buf_load16(r, row * 256 + 16 * g, 32 * s));
}

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    uint16_t* __restrict__ dq, int nqb, int nkb, int64_t q_rows, int64_t q_valid,
    int64_t kv_rows, int64_t kv_valid, float scale_log2, float sm_scale) {
  __shared__ __attribute__((aligned(1024))) uint16_t kl[kB * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t vl[kB * kD];
  const int item = blockIdx.x;
  const int h = item / nqb, i = item % nqb;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, g = lane >> 5;
  Offsets off;
  make_offsets(off, lane);
  const int64_t qrow = (int64_t)i * kB + 32 * wave + lq;   // this lane's query
  const int64_t qbase = (int64_t)h * q_rows;

  bf16x8 qf[8], df[8];
  load_b(qf, q + (qbase + (int64_t)i * kB) * kD, 32 * wave + lq, g);
  load_b(df, dout + (qbase + (int64_t)i * kB) * kD, 32 * wave + lq, g);
  const float l = lse[qbase + qrow];
  const bool live = qrow < q_valid && l > -INFINITY;
  const float lse2 = live ? l * kLog2e : INFINITY;   // +inf: P = 0
  const float dlt = delta[qbase + qrow];

  f32x16 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;

  // Per block j (V_j landed, K_j in flight at the top):
  //   dP^T = V dO^T (V rows); wait for K_j, barrier; load V_{j+1};
  //   S^T = K Q^T, dS^T, dQ^T += K^T dS^T (K rows, K transposed);
  //   wait for V_{j+1}, barrier; load K_{j+1}.
  const int e0 = __builtin_amdgcn_readfirstlane(row_ptr[item]);
  const int e1 = __builtin_amdgcn_readfirstlane(row_ptr[item + 1]);
  auto src_of = [&](int e) -> int64_t {   // block offset of entry e, -1 if outside the row
    const int j = __builtin_amdgcn_readfirstlane(col_idx[e]);
    return (unsigned)j < (unsigned)nkb ? ((int64_t)h * kv_rows + (int64_t)j * kB) * kD : -1;
  };
  int e = e0;
  int64_t src = -1;
  while (e < e1 && (src = src_of(e)) < 0) ++e;
  if (e < e1) {
    dma_block(v + src, vl, wave, off.dma);
    dma_block(k + src, kl, wave, off.dma);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  while (e < e1) {
    const int j = __builtin_amdgcn_readfirstlane(col_idx[e]);
    int en = e + 1;
    int64_t sn = -1;
    while (en < e1 && (sn = src_of(en)) < 0) ++en;
    f32x16 dpacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) dpacc[t][r] = 0.f;
    // V rows read two fragments ahead of their MFMA; the scheduling fences
    // keep them there (left alone, the compiler waits on each read right
    // before its MFMA)
    {
      bf16x8 fv[32];
#pragma unroll
      for (int i = 0; i < 2; ++i) fv[i] = rows_a(vl, off, i >> 3, i & 7);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i + 2 < 32) fv[i + 2] = rows_a(vl, off, (i + 2) >> 3, (i + 2) & 7);
        __builtin_amdgcn_sched_barrier(0);
        dpacc[i >> 3] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[i], df[i & 7], dpacc[i >> 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's K_j loads
    __syncthreads();
    if (en < e1) dma_block(v + sn, vl, wave, off.dma);
    const int lim = __builtin_amdgcn_readfirstlane((int)min((int64_t)kB, kv_valid - (int64_t)j * kB));
    // raised wave priority over the phase that mixes exponentials and MFMAs
    // (the other workgroup's wave on the SIMD fills in from its dP MFMAs)
    __builtin_amdgcn_s_setprio(1);
    // K rows (fk, k-step i) and transposed K (fc, half j / 4, d-tile j % 4) read
    // two fragments ahead of their MFMA, fenced
    bf16x8 fk[8], fc[8];
    fk[0] = rows_a(kl, off, 0, 0);
    fk[1] = rows_a(kl, off, 0, 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + 2 < 8) fk[i + 2] = rows_a(kl, off, t, i + 2);
        else fc[i - 6] = cols_a(kl, off, (i - 6) & 3, t, (i - 6) >> 2);
        __builtin_amdgcn_sched_barrier(0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[i], qf[i], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // reg r: key 32t + 8(r/4) + 4g + r%4 of this lane's query
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        const float p = key < lim ? __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -lse2)) : 0.f;
        ds[r] = p * (dpacc[t][r] - dlt);
      }
      const bf16x8 dsf[2] = {to_bf16x8(ds, 0), to_bf16x8(ds, 8)};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j + 2 < 8) fc[j + 2] = cols_a(kl, off, (j + 2) & 3, t, (j + 2) >> 2);
        else if (t + 1 < 4) fk[j - 6] = rows_a(kl, off, t + 1, j - 6);
        __builtin_amdgcn_sched_barrier(0);
        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc[j], dsf[j >> 2], acc[j & 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's V_{j+1} loads
    __syncthreads();
    if (en < e1) dma_block(k + sn, kl, wave, off.dma);
    e = en;
  }
  // dQ[query][d], reg r of tile u -> d = 32u + 8(r/4) + 4g + r%4
  uint16_t* op = dq + (qbase + qrow) * kD;
  const float sc = qrow < q_valid ? sm_scale : 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 o4;
#pragma unroll
      for (int x = 0; x < 4; ++x) o4[x] = acc[u][4 * r4 + x] * sc;
      *reinterpret_cast<bf16x4*>(op + 32 * u + 8 * r4 + 4 * g) = __builtin_convertvector(o4, bf16x4);
    }
}

// Element n of one query block's MFMA sequence in the dK/dV kernel: kind 0 =
// A (score / dP, fragment idx of tile t), 1 = C (dV / dK, fragment idx of tile t).
struct SeqElem {
  int kind, t, idx;
};
__host__ __device__ constexpr SeqElem seq_elem(int n) {
  if (n < 16) return {0, 0, n};
  const int m = n - 16;
  if (m >= 96) return {1, 3, m - 96};
  const int b = m / 32, pos = m % 32;
  return pos < 16 ? SeqElem{0, b + 1, pos} : SeqElem{1, b, pos - 16};
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
    const int32_t* __restrict__ order, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int nqb, int nkb, int64_t q_rows, int64_t q_valid, int64_t kv_rows, int64_t kv_valid,
    float scale_log2, float sm_scale) {
  // two buffers: the next query block loads while this one is computed
  __shared__ __attribute__((aligned(1024))) uint16_t qbuf[2][kB * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t dbuf[2][kB * kD];
  __shared__ __attribute__((aligned(16))) float lse_b[2][kB];
  __shared__ __attribute__((aligned(16))) float dlt_b[2][kB];
  const int unit = __builtin_amdgcn_readfirstlane(order[blockIdx.x]);
  const int h = unit / nkb, j = unit % nkb;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, g = lane >> 5;
  Offsets off;
  make_offsets(off, lane);
  const int64_t krow = (int64_t)j * kB + 32 * wave + lq;   // this lane's key
  const int64_t kbase = (int64_t)h * kv_rows;
  const bool key_ok = krow < kv_valid;

  bf16x8 kf[8], vf[8];
  load_b(kf, k + (kbase + (int64_t)j * kB) * kD, 32 * wave + lq, g);
  load_b(vf, v + (kbase + (int64_t)j * kB) * kD, 32 * wave + lq, g);

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dka[u][r] = 0.f; dva[u][r] = 0.f; }

  const int c0 = __builtin_amdgcn_readfirstlane(col_ptr[unit]);
  const int c1 = __builtin_amdgcn_readfirstlane(col_ptr[unit + 1]);
  // query block i of column entry c into buffer b (Q, dO by direct loads;
  // LSE in log2 units, +inf for rows without attention so P = 0; D)
  auto stage = [&](int c, int b) {
    const int i = __builtin_amdgcn_readfirstlane(row_idx[c]);
    const int64_t qb = (int64_t)h * q_rows + (int64_t)i * kB;
    dma_block(q + qb * kD, qbuf[b], wave, off.dma);
    dma_block(dout + qb * kD, dbuf[b], wave, off.dma);
    if (tid < kB) {
      const int64_t row = (int64_t)i * kB + tid;
      const float l = lse[qb + tid];
      lse_b[b][tid] = (row < q_valid && l > -INFINITY) ? l * kLog2e : INFINITY;
      dlt_b[b][tid] = delta[qb + tid];
    }
  };
  if (c0 < c1) stage(c0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c = c0, b = 0; c < c1; ++c, b ^= 1) {
    if (c + 1 < c1) stage(c + 1, b ^ 1);   // that buffer was last read before the barrier
    const uint16_t* ql = qbuf[b];
    const uint16_t* dl = dbuf[b];
    const float* lse_s = lse_b[b];
    const float* dlt_s = dlt_b[b];
    // One wave per SIMD, so the wave must overlap its own work.  The MFMAs of
    // one query block run as one sequence: A(0), then per tile t the score
    // and dP MFMAs of tile t + 1 (A) with the exponentials of tile t between
    // them, then tile t's dV/dK MFMAs (C); tile 3's exponentials sit between
    // the C MFMAs of tile 2.  Each operand fragment is read
    // kAhead MFMAs before its use, into a ring of registers, and scheduling
    // fences keep every MFMA in its place.  Per tile t:
    //   A fragment i: rows of Q (i even) or dO (i odd), k-step i / 2;
    //   C fragment j: transposed dO (j even) or Q (j odd), half j / 8, d-tile (j / 2) % 4.
    // Every accumulator sees its terms in the plain loop's order.
    constexpr int kAhead = 6, kRing = 8, kSeq = 128;
    auto read = [&](auto nc) -> bf16x8 {
      constexpr SeqElem e = seq_elem(decltype(nc)::value);
      if constexpr (e.kind == 0) return rows_a((e.idx & 1) ? dl : ql, off, e.t, e.idx >> 1);
      else return cols_a((e.idx & 1) ? ql : dl, off, (e.idx >> 1) & 3, e.t, e.idx >> 3);
    };
    bf16x8 ring[kRing];
    f32x16 sacc[2], dpacc[2], p, ds;
    f32x4 l4[2][4], d4[2][4];   // LSE and D of tiles t and t + 1 (slot t & 1)
    bf16x8 pf[2], dsf[2];
    // P and dS of tile t, entry r (query 32t + 8(r/4) + 4g + r%4, this lane's key)
    auto softmax_r = [&](int t, int r) {
      const float pv = key_ok ? __builtin_amdgcn_exp2f(fmaf(sacc[t & 1][r], scale_log2,
                                                            -l4[t & 1][r >> 2][r & 3]))
                              : 0.f;
      p[r] = pv;
      ds[r] = pv * (dpacc[t & 1][r] - d4[t & 1][r >> 2][r & 3]);
    };
    auto load_stats = [&](int t) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int q0 = 32 * t + 8 * r4 + 4 * g;
        l4[t & 1][r4] = *reinterpret_cast<const f32x4*>(lse_s + q0);
        d4[t & 1][r4] = *reinterpret_cast<const f32x4*>(dlt_s + q0);
      }
    };
    static_for<0, kAhead>([&](auto nc) { ring[decltype(nc)::value % kRing] = read(nc); });
    static_for<0, kSeq>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      constexpr SeqElem e = seq_elem(n);
      if constexpr (n + kAhead < kSeq)
        ring[(n + kAhead) % kRing] = read(std::integral_constant<int, n + kAhead>{});
      if constexpr (e.kind == 0) {
        if constexpr (e.idx == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) { sacc[e.t & 1][r] = 0.f; dpacc[e.t & 1][r] = 0.f; }
        }
        if constexpr (e.t >= 1) softmax_r(e.t - 1, e.idx);
      } else {
        if constexpr (e.idx == 0) {
          pf[0] = to_bf16x8(p, 0);
          pf[1] = to_bf16x8(p, 8);
          dsf[0] = to_bf16x8(ds, 0);
          dsf[1] = to_bf16x8(ds, 8);
        }
        // tile 3 has no score MFMAs after it: its P and dS are formed between
        // the dV/dK MFMAs of tile 2 (p and ds are free once tile 2 is packed)
        if constexpr (e.t == 2) softmax_r(3, e.idx);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 f = ring[n % kRing];
      if constexpr (e.kind == 0) {
        if constexpr (e.idx & 1)
          dpacc[e.t & 1] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, vf[e.idx >> 1], dpacc[e.t & 1], 0, 0, 0);
        else
          sacc[e.t & 1] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, kf[e.idx >> 1], sacc[e.t & 1], 0, 0, 0);
      } else {
        constexpr int u = (e.idx >> 1) & 3, h2 = e.idx >> 3;
        if constexpr (e.idx & 1)
          dka[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, dsf[h2], dka[u], 0, 0, 0);
        else
          dva[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[h2], dva[u], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the LSE and D of tile t are loaded as its score MFMAs start: they are
      // used a tile later
      if constexpr (e.kind == 0 && e.idx == 0) load_stats(e.t);
    });
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next block
    __syncthreads();
  }
  // dK, dV [key][d], reg r of tile u -> d = 32u + 8(r/4) + 4g + r%4
  uint16_t* kp = dk + (kbase + krow) * kD;
  uint16_t* vp = dv + (kbase + krow) * kD;
  const float sk = key_ok ? sm_scale : 0.f, sv = key_ok ? 1.f : 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 k4, v4;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        k4[x] = dka[u][4 * r4 + x] * sk;
        v4[x] = dva[u][4 * r4 + x] * sv;
      }
      *reinterpret_cast<bf16x4*>(kp + 32 * u + 8 * r4 + 4 * g) = __builtin_convertvector(k4, bf16x4);
      *reinterpret_cast<bf16x4*>(vp + 32 * u + 8 * r4 + 4 * g) = __builtin_convertvector(v4, bf16x4);
    }
}

}  // namespace

hipError_t launch_backward(const Dims& g, const void* q, const void* k, const void* v,
                           const void* out, const void* dout, const float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, void* dq, void* dk,
                           void* dv, float* delta, uint32_t* bits, int32_t* counts,
                           int32_t* col_ptr, int32_t* row_idx, int32_t* order, float sm_scale,
                           hipStream_t s) {
  const int64_t qrows_total = (int64_t)g.H * g.q_rows;
  hipLaunchKernelGGL(delta_kernel, dim3((unsigned)((qrows_total + 3) / 4)), dim3(256), 0, s,
                     (const uint16_t*)out, (const uint16_t*)dout, qrows_total, g.q_rows,
                     g.q_valid, delta);
  const int cols = g.H * g.nkb;
  const int rows = g.H * g.nqb;
  hipLaunchKernelGGL(row_bits_kernel, dim3((rows + kBitsWaves - 1) / kBitsWaves),
                     dim3(kBitsWaves * kWave), 0, s, row_ptr, col_idx, rows, g.nkb, g.W, bits);
  const int grid = std::min((cols + 255) / 256, 1024);
  hipLaunchKernelGGL(csc_kernel<false>, dim3(grid), dim3(256), 0, s, bits, g.H, g.nqb, g.nkb,
                     g.W, (const int32_t*)nullptr, counts, (int32_t*)nullptr);
  hipLaunchKernelGGL(csc_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, cols, col_ptr);
  hipLaunchKernelGGL(csc_kernel<true>, dim3(grid), dim3(256), 0, s, bits, g.H, g.nqb, g.nkb,
                     g.W, col_ptr, (int32_t*)nullptr, row_idx);
  hipLaunchKernelGGL(lpt_order_kernel, dim3(g.H), dim3(kOrderThreads), 0, s, counts, g.nkb,
                     g.nqb, order);
  const float scale_log2 = sm_scale * kLog2e;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(g.H * g.nqb), dim3(256), 0, s, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, delta,
                     row_ptr, col_idx, (uint16_t*)dq, g.nqb, g.nkb, g.q_rows, g.q_valid,
                     g.kv_rows, g.kv_valid, scale_log2, sm_scale);
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(cols), dim3(256), 0, s, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, lse, delta,
                     col_ptr, row_idx, order, (uint16_t*)dk, (uint16_t*)dv, g.nqb, g.nkb, g.q_rows,
                     g.q_valid, g.kv_rows, g.kv_valid, scale_log2, sm_scale);
  return hipGetLastError();
}

}  // namespace sa
