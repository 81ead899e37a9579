// The bf16 attention of one query block (128 queries, d = 128) over a list
// of key/value blocks, shared by the forward kernels: the three-call path's
// attn_bf16_kernel reads its list from the CSR in global memory, the fused
// estimation + attention kernel from a list it selected into LDS.
//
// Workgroup of four waves; wave w owns queries 32w..32w+31.  Per key block:
//   S phase      S^T = K Q^T on MFMA (K from LDS, Q in registers)
//   barrier      (all waves done with K; this wave's V loads have landed)
//   K loads      the next block's K goes into LDS
//   softmax, PV  O^T += V^T P^T (V from LDS through transposing reads)
//   barrier      (all waves done with V; the next K has landed)
//   V loads      the next block's V goes into LDS
// Online softmax in the exp2 domain (the standard running-max / rescale /
// running-sum identity of flash-style attention).
#pragma once

#include <math.h>

#include "mfma_bf16.h"

namespace sa {
namespace bf16mma {

// Unnormalised state of one wave's 32 queries: O^T accumulators (reg r of
// d-tile u -> d = 32u + 8(r/4) + 4g + r%4 of query lane%32), running max (log2
// units) and this lane's half of the running sum.
struct AttnState {
  f32x16 oacc[4];
  float m_run, l_run;
};

// Key block list read from a CSR in global memory: entry e is block
// col_idx[e] of head h, read from the packed slot col_slot[e] when col_slot
// is given (-1: skipped), else from the full K/V.
struct CsrBlockList {
  const int32_t* __restrict__ col_idx;
  const int32_t* __restrict__ col_slot;
  int h, nkb;
  __device__ __forceinline__ int col(int e) const {
    return __builtin_amdgcn_readfirstlane(col_idx[e]);
  }
  __device__ __forceinline__ int64_t src(int e) const {
    const int j = col(e);
    if ((unsigned)j >= (unsigned)nkb) return -1;
    return col_slot ? (int64_t)__builtin_amdgcn_readfirstlane(col_slot[e]) : (int64_t)h * nkb + j;
  }
  // entry e's values, loaded now and resolved after a later wait
  struct Raw {
    int j, slot;
  };
  __device__ __forceinline__ Raw fetch(int e) const { return {col_idx[e], col_slot ? col_slot[e] : 0}; }
  __device__ __forceinline__ int64_t src_of(const Raw& r, int& j) const {
    j = __builtin_amdgcn_readfirstlane(r.j);
    if ((unsigned)j >= (unsigned)nkb) return -1;
    return col_slot ? (int64_t)__builtin_amdgcn_readfirstlane(r.slot) : (int64_t)h * nkb + j;
  }
};

// Key block list held in LDS (16-bit block ids of head h, full K/V).
struct LdsBlockList {
  const uint16_t* ids;
  int h, nkb;
  __device__ __forceinline__ int col(int e) const { return __builtin_amdgcn_readfirstlane(ids[e]); }
  __device__ __forceinline__ int64_t src(int e) const {
    const int j = col(e);
    return (unsigned)j < (unsigned)nkb ? (int64_t)h * nkb + j : -1;
  }
  struct Raw {
    int j, slot;
  };
  __device__ __forceinline__ Raw fetch(int e) const { return {ids[e], 0}; }
  __device__ __forceinline__ int64_t src_of(const Raw& r, int& j) const {
    j = __builtin_amdgcn_readfirstlane(r.j);
    return (unsigned)j < (unsigned)nkb ? (int64_t)h * nkb + j : -1;
  }
};

// Attention of query block i of head h over entries [e0, e1) of `list`.
// kl, vl: 32 KiB LDS tiles each (1 KiB aligned).  Leaves the unnormalised
// state in `st`; every wave of the workgroup must call it with the same
// arguments (it holds barriers).
template <class List>
__device__ __forceinline__ void attend_blocks(AttnState& st, const List& list, int e0, int e1,
                                              uint16_t* kl, uint16_t* vl,
                                              const uint16_t* __restrict__ q,
                                              const uint16_t* __restrict__ k,
                                              const uint16_t* __restrict__ v, int h, int i,
                                              int64_t q_rows, int64_t kv_valid, float scale_log2) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, g = lane >> 5;
  const int qloc = 32 * wave + lq;                                // query row within the block

  // lane offsets of the block loads (see dma_block): row 4i + L/16, chunk L%16
  int kvo[4], vvo[4];
  {
    const int rr = lane >> 4, pc = lane & 15;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      kvo[p] = rr * 256 + ((pc ^ (4 * p + rr)) << 4);
      vvo[p] = rr * 256 + ((pc ^ (4 * rr)) << 4);
    }
  }
  // K operand reads: row 32t + lq, logical chunk 2s + g -> chunk (2s + g) ^ (lq & 15)
  int ka[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) ka[s] = lq * 256 + (((2 * s + g) ^ (lq & 15)) << 4);
  // V operand reads (transposing): lane j of 16-lane group a reads row
  // 4 kga + e, columns 32u + 16 (a & 1) + 4 q .. +3, with e = j / 4, q = j % 4
  int va[4];
  {
    const int a = lane >> 4, j = lane & 15, e = j >> 2, qq = j & 3;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      va[u] = 1024 * g + 256 * e + 64 * (u ^ e) + 32 * (a & 1) + 8 * qq;
  }

  // Q fragments (B operand of S^T = K Q^T): d = 16s + 8g .. +8
  bf16x8 qf[8];
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(q + ((int64_t)h * q_rows + (int64_t)i * kB) * kD, kTileBytes);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, qloc * 256 + 16 * g, 32 * s));
  }

#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[u][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // The list entry after the current block is loaded one block ahead and
  // resolved after that block's closing wait, so that no block starts by
  // waiting on a global load.
  int e = e0;
  int64_t blk = -1;
  while (e < e1 && (blk = list.src(e)) < 0) ++e;
  int j = e < e1 ? list.col(e) : 0;
  typename List::Raw rn{0, 0};
  if (e < e1) {
    dma_block(k + blk * (kB * kD), kl, wave, kvo);
    dma_block(v + blk * (kB * kD), vl, wave, vvo);
    if (e + 1 < e1) rn = list.fetch(e + 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  while (e < e1) {
    // the next block: entry e + 1 (already loaded), or a later one if it is skipped
    int en = e + 1, jn = 0;
    int64_t bn = -1;
    if (en < e1) {
      bn = list.src_of(rn, jn);
      if (bn < 0) {
        ++en;
        while (en < e1 && (bn = list.src(en)) < 0) ++en;
        if (en < e1) jn = list.col(en);
      }
    }
    if (en + 1 < e1) rn = list.fetch(en + 1);

    // S^T tile t: keys 32t.., this lane's query; reg r -> key 32t + 8(r/4) + 4g + r%4
    f32x16 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
    // K fragments of step s + 1 are read while the MFMAs of step s run.  The
    // scheduling fences keep them there: left alone, the compiler folds the
    // two fragment sets into one and waits on each read right before its MFMA.
    bf16x8 kf[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      kf[0][t] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kl) + ka[0] +
                                                  t * 8192);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          kf[(s + 1) & 1][t] = *reinterpret_cast<const bf16x8*>(
              reinterpret_cast<const char*>(kl) + ka[s + 1] + t * 8192);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s & 1][t], qf[s], sacc[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    __builtin_amdgcn_s_waitcnt(0);   // this wave's V loads
    __syncthreads();
    if (en < e1) dma_block(k + bn * (kB * kD), kl, wave, kvo);

    // valid keys of this block (uniform); only the sequence's last block is ragged
    const int lim = __builtin_amdgcn_readfirstlane((int)min((int64_t)kB, kv_valid - (int64_t)j * kB));
    float mx = -INFINITY;
    if (__builtin_expect(lim < kB, 0)) {
      const int lim_g = lim - 4 * g;   // key 32t + 8(r/4) + 4g + r%4 >= lim
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + 8 * (r >> 2) + (r & 3) >= lim_g) sacc[t][r] = -INFINITY;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
    {
      // the two 32-lane halves hold the two key halves of each query: swapping
      // them across registers (v_permlane32_swap) leaves each lane one copy
      // of its own half's max and one of the other's
      const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
      mx = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1])) * scale_log2;
    }
    // The running max only moves when some query's block max exceeds it by
    // more than 8 (log2 units): until then P = exp2(S*scale - m) stays below
    // 2^8, and softmax does not depend on which reference max is used.  Most
    // rescales of O are skipped (wave-uniform branch).
    if (__ballot(mx > m_run + 8.f)) {
      const float mn = fmaxf(m_run, mx);
      // v_exp_f32 directly: masses below 2^-126 flush to 0, which softmax tolerates
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[u][r] *= alpha;
      l_run *= alpha;
      m_run = mn;
    }
    const float mn = m_run;
    // Raised wave priority for the softmax and P V phase, where exponentials
    // and MFMAs alternate: the other workgroup's wave on this SIMD, when it is
    // in its score MFMAs, fills the slots this one leaves (measured 0.5-1%
    // faster than raising the score phase instead).
    __builtin_amdgcn_s_setprio(1);

    // per key tile t: P = exp2(S*scale - m), then O^T += V^T P^T over k-steps
    // (t, h2) covering keys 32t + 16h2 .. +16: slots 0-3 are keys 4*kga .. +3 and
    // slots 4-7 keys 4*(kga+2) .. +3, kga = 8t + 4h2 + g (the transposing reads
    // at rows 4 kga + e and 4 (kga + 2) + e).
    // The 32 P V MFMAs run as one sequence (n: k-step n / 4 = 2t + h2, d-tile
    // n % 4, so consecutive MFMAs feed different accumulators), each V
    // fragment read kAhead MFMAs ahead into a ring of registers, and the
    // exponentials of tile t + 1 spread over the MFMAs of tile t (two per
    // MFMA); scheduling fences keep every MFMA in its place.  The row sum and
    // every accumulator see their terms in the plain loop's order.
    constexpr int kAhead = 4, kRing = 6;
    auto vread = [&](auto nc) -> u32x4 {
      constexpr int n = decltype(nc)::value, ks = n / 4, u = n % 4;
      const int rows = 1024 * (8 * (ks >> 1) + 4 * (ks & 1));
      const u32x2 lo = lds_read_tr(vl, va[u] + rows);
      const u32x2 hi = lds_read_tr(vl, va[u] + rows + 2048);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    u32x4 ring[kRing];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[0][r], scale_log2, -mn));
      sacc[0][r] = p;
      ps += p;
    }
    static_for<0, kAhead>([&](auto nc) { ring[decltype(nc)::value % kRing] = vread(nc); });
    bf16x8 pf;
    static_for<0, 32>([&](auto nc) {
      constexpr int n = decltype(nc)::value, ks = n / 4, t = ks / 2, h2 = ks % 2, u = n % 4;
      if constexpr (n + kAhead < 32)
        ring[(n + kAhead) % kRing] = vread(std::integral_constant<int, n + kAhead>{});
      if constexpr (t + 1 < 4) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int r = 2 * (n % 8) + x;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t + 1][r], scale_log2, -mn));
          sacc[t + 1][r] = p;
          ps += p;
        }
      }
      if constexpr (u == 0) pf = to_bf16x8(sacc[t], 8 * h2);
      __builtin_amdgcn_sched_barrier(0);
      st.oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, ring[n % kRing]), pf, st.oacc[u], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    l_run += ps;
    __builtin_amdgcn_s_setprio(0);

    __builtin_amdgcn_s_waitcnt(0);   // this wave's K loads of the next block
    __syncthreads();
    if (en < e1) dma_block(v + bn * (kB * kD), vl, wave, vvo);
    e = en;
    j = jn;
  }
  st.m_run = m_run;
  st.l_run = l_run;
}

// Normalise and store one wave's 32 queries of query block i of head h:
// out [H, q_rows, d] bf16; lse (NULL or [H, q_rows]) in natural-log units.
// Query rows at or beyond q_valid, and rows that attended to nothing, get
// out = 0 and lse = -inf.
__device__ __forceinline__ void store_rows(const AttnState& st, uint16_t* __restrict__ out,
                                           float* __restrict__ lse, int h, int i, int64_t q_rows,
                                           int64_t q_valid) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lq = lane & 31, g = lane >> 5;
  const int64_t qrow = (int64_t)i * kB + 32 * wave + lq;
  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
  const bool live = qrow < q_valid && l_tot > 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
  uint16_t* op = out + ((int64_t)h * q_rows + qrow) * kD;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 o4;
#pragma unroll
      for (int x = 0; x < 4; ++x) o4[x] = st.oacc[u][4 * r4 + x] * inv;
      *reinterpret_cast<bf16x4*>(op + 32 * u + 8 * r4 + 4 * g) = __builtin_convertvector(o4, bf16x4);
    }
  if (lse && g == 0)
    lse[(int64_t)h * q_rows + qrow] =
        live ? (st.m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace bf16mma
}  // namespace sa
