// Attention over the selected key blocks only ("Dynamic Sparsity in
// Large-Scale Video DiT Training", section "The idea": sparse attention
// kernels that never build the full score matrix; neighbouring queries, one
// query block, share one selected key/value set) with the work balanced over
// the device so uneven per-head sparsity does not leave CUs idle (same page
// and section, the paragraph on uneven work; the Top-p sparse-attention
// abstract, mlsift listing: rank-level stragglers).
//
// queue_kernel : one workgroup orders the work units (items, or halves of
//                their block lists) into per-XCD ranges, in (range, head
//                group, half, item) order; see "work queue" below.
// attn_f32     : fp32 path (one thread per query, 32-key LDS sub-tiles,
//                online softmax in fp32), one workgroup per item.
// attn_bf16    : bf16 MFMA path, d = 128, block = 128, persistent: each
//                workgroup of four waves takes units from its XCD's queue;
//                wave w owns queries 32w..32w+31.  Per key block: K and V go
//                into LDS by direct loads (XOR-swizzled rows); S^T = K Q^T
//                with v_mfma_f32_32x32x16_bf16 so that each lane holds one
//                query's scores (row max = local max + one cross-half
//                exchange); online softmax in the exp2 domain; P^T goes
//                straight from the accumulator registers into the B operand
//                of O^T = V^T P^T, with V read through transposing LDS reads.
//                Halves of an item combine their partial states in a fixed
//                order (attend_item).
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "attend_bf16.h"

namespace sa {
namespace {

using namespace bf16mma;

// ---------------------------------------------------------------------------
// work queue
// ---------------------------------------------------------------------------
// A work unit is a (head, query block) item, or one half of its selected-block
// list when items are split (see split_items below); unit id = 2*item + half.
// The selected entries of all items, in item order, are cut into kXcd equal
// shares of work, one range per XCD: a unit belongs to the range of the middle
// of its entries.  Concurrent workgroups of an XCD then attend to the same
// head's key/value blocks, which stay resident in that XCD's L2.  Inside a
// range, units go head by head, first halves before second halves, and in
// query-block order within those: neighbouring query blocks select similar
// key blocks, so the workgroups of an XCD share more of them in L2 (heads are
// grouped by 2^hshift when there are thousands of them).  xq[x] .. xq[x+1] is
// range x; ctr[x] (zeroed here) is its cursor; done[item] (zeroed here when
// split) counts the published halves of an item.
//
// The order is a sort on (group, item) with group = 2 (range + head group) +
// half.  Along the item order both the range and the head are non-decreasing
// (for either half), so every group is a contiguous run of items: a unit's
// position is its group's start plus the number of the group's units before
// it, which for first halves is its item offset from the group's first item
// and for second halves the number of split items in between.  No atomic
// decides any position, so the order is deterministic.
constexpr int kXcd = 8;
constexpr int kQueueThreads = 1024;
constexpr int kQueueMaxGroups = 4096;

struct QueueShape {
  int nqb, hshift;
};

// Selected-block range [lo, hi) of half `part` of item r (the whole list when
// the item is not split; halves only for lists of two or more entries).
struct Range {
  int lo, hi;
  bool halved;
};
__device__ __forceinline__ Range unit_range(const int32_t* row_ptr, int r, int part, int split) {
  const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
  if (!split || e1 - e0 < 2) return {e0, e1, false};
  const int mid = e0 + (e1 - e0 + 1) / 2;
  return part ? Range{mid, e1, true} : Range{e0, mid, true};
}

__device__ __forceinline__ int unit_xcd(Range u, int64_t total) {
  const int64_t mid = (int64_t)u.lo + (u.hi - u.lo) / 2;
  return total > 0 ? (int)min<int64_t>(kXcd - 1, mid * kXcd / total) : 0;
}

__device__ __forceinline__ int unit_group(Range u, int r, int part, const QueueShape& qs,
                                          int64_t total) {
  return 2 * (unit_xcd(u, total) + ((r / qs.nqb) >> qs.hshift)) + part;
}

__global__ __launch_bounds__(kQueueThreads) void queue_kernel(const int32_t* __restrict__ row_ptr,
                                                              int rows, QueueShape qs, int split,
                                                              int32_t* __restrict__ units,
                                                              int32_t* __restrict__ xq,
                                                              int32_t* __restrict__ ctr,
                                                              int32_t* __restrict__ done) {
  __shared__ int gstart[kQueueMaxGroups];   // group sizes, then their starts
  __shared__ int gfirst[kQueueMaxGroups];   // first item of each group
  __shared__ int gsplit[kQueueMaxGroups];   // split items before a second-half group's first
  __shared__ int xcnt[kXcd];
  __shared__ int red[kQueueThreads / kWave + 1];
  const int t = threadIdx.x;
  const int heads = rows / qs.nqb;
  const int ng = 2 * (kXcd + ((heads - 1) >> qs.hshift) + 1);
  const int64_t total = row_ptr[rows];
  if (!split) {
    // Whole items only: along the item order both the range and the head are
    // non-decreasing, so the sort is the identity, and range x starts at the
    // first item whose range is x or more (one pass, no scans).
    for (int r = t; r < rows; r += kQueueThreads) {
      units[r] = 2 * r;
      const int xr = unit_xcd(unit_range(row_ptr, r, 0, 0), total);
      const int xp = r > 0 ? unit_xcd(unit_range(row_ptr, r - 1, 0, 0), total) : -1;
      for (int x = xp + 1; x <= xr; ++x) xq[x] = r;
      if (r == rows - 1)
        for (int x = xr + 1; x <= kXcd; ++x) xq[x] = rows;
    }
    if (t < kXcd) ctr[t] = 0;
    if (rows == 0 && t <= kXcd) xq[t] = 0;
    return;
  }
  for (int b = t; b < ng; b += kQueueThreads) {
    gstart[b] = 0;
    gfirst[b] = INT_MAX;
  }
  if (t < kXcd) xcnt[t] = 0;
  if (split)
    for (int r = t; r < rows; r += kQueueThreads) done[r] = 0;
  __syncthreads();
  // group sizes and first items (order-independent, so deterministic)
  for (int r = t; r < rows; r += kQueueThreads) {
    const Range u0 = unit_range(row_ptr, r, 0, split);
    const int g0 = unit_group(u0, r, 0, qs, total);
    atomicAdd(&gstart[g0], 1);
    atomicMin(&gfirst[g0], r);
    atomicAdd(&xcnt[unit_xcd(u0, total)], 1);
    if (u0.halved) {
      const Range u1 = unit_range(row_ptr, r, 1, split);
      const int g1 = unit_group(u1, r, 1, qs, total);
      atomicAdd(&gstart[g1], 1);
      atomicMin(&gfirst[g1], r);
      atomicAdd(&xcnt[unit_xcd(u1, total)], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the group sizes, contiguous chunk per thread
  const int per = (ng + kQueueThreads - 1) / kQueueThreads;
  const int lo = min(ng, t * per), hi = min(ng, lo + per);
  int local = 0;
  for (int b = lo; b < hi; ++b) local += gstart[b];
  int all;
  int run = block_inclusive_scan(local, red, &all) - local;
  __syncthreads();
  for (int b = lo; b < hi; ++b) {
    const int c = gstart[b];
    gstart[b] = run;
    run += c;
  }
  if (t == 0) {
    int acc = 0;
    for (int x = 0; x < kXcd; ++x) {
      xq[x] = acc;
      ctr[x] = 0;
      acc += xcnt[x];
    }
    xq[kXcd] = acc;
  }
  __syncthreads();
  // positions, chunk by chunk in item order with a running count of split items
  int carry = 0;
  for (int base = 0; base < rows; base += kQueueThreads) {
    const int r = base + t;
    Range u0{0, 0, false}, u1{0, 0, false};
    int g0 = 0, g1 = 0;
    if (r < rows) {
      u0 = unit_range(row_ptr, r, 0, split);
      g0 = unit_group(u0, r, 0, qs, total);
      if (u0.halved) {
        u1 = unit_range(row_ptr, r, 1, split);
        g1 = unit_group(u1, r, 1, qs, total);
      }
    }
    const int flag = u0.halved ? 1 : 0;
    int chunk;
    const int before = carry + block_inclusive_scan(flag, red, &chunk) - flag;
    if (flag && gfirst[g1] == r) gsplit[g1] = before;
    __syncthreads();
    if (r < rows) {
      units[gstart[g0] + (r - gfirst[g0])] = 2 * r;
      if (flag) units[gstart[g1] + (before - gsplit[g1])] = 2 * r + 1;
    }
    carry += chunk;
    __syncthreads();
  }
}

// Next unit for a persistent workgroup: its own XCD's range first, then the
// others' (stealing).  -1 when every range is exhausted.
__device__ __forceinline__ int pop_item(const int32_t* __restrict__ items,
                                        const int32_t* __restrict__ xq, int32_t* ctr, int home) {
  for (int k = 0; k < kXcd; ++k) {
    const int x = (home + k) & (kXcd - 1);
    const int n = xq[x + 1] - xq[x];
    if (n <= 0) continue;
    if (__hip_atomic_load(&ctr[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
    const int idx = atomicAdd(&ctr[x], 1);
    if (idx < n) return items[xq[x] + idx];
  }
  return -1;
}

__device__ __forceinline__ int xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & (kXcd - 1);
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(BLK) void attn_f32_kernel(
    const float* __restrict__ q, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ col_slot,
    const float* __restrict__ k, const float* __restrict__ v, float* __restrict__ out,
    float* __restrict__ lse, const int32_t* __restrict__ items, int nqb, int nkb,
    int64_t q_rows, int64_t q_valid, int64_t kv_rows, int64_t kv_valid, float sm_scale) {
  constexpr int SUB = 32;
  __shared__ float4 ks[SUB * D / 4];
  __shared__ float4 vs[SUB * D / 4];
  const int item = items[blockIdx.x] >> 1;   // never split on this path
  const int h = item / nqb, i = item % nqb;
  const int t = threadIdx.x;
  const int64_t a = (int64_t)i * BLK + t;
  const float* qrow = q + ((int64_t)h * q_rows + a) * D;
  float qr[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = qrow[c];
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int e0 = row_ptr[item], e1 = row_ptr[item + 1];
  for (int e = e0; e < e1; ++e) {
    const int j = col_idx[e];
    int64_t blk;
    if (col_slot) {
      blk = col_slot[e];
      if (blk < 0) continue;
    } else {
      if ((unsigned)j >= (unsigned)nkb) continue;
      blk = (int64_t)h * nkb + j;
    }
    const float4* kb = reinterpret_cast<const float4*>(k + blk * BLK * D);
    const float4* vb = reinterpret_cast<const float4*>(v + blk * BLK * D);
    for (int sub = 0; sub < BLK / SUB; ++sub) {
      const int64_t key0 = (int64_t)j * BLK + sub * SUB;
      if (key0 >= kv_valid) break;
      __syncthreads();
      for (int x = t; x < SUB * D / 4; x += BLK) {
        ks[x] = kb[sub * SUB * D / 4 + x];
        vs[x] = vb[sub * SUB * D / 4 + x];
      }
      __syncthreads();
      float s[SUB];
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < SUB; ++kk) {
        const float* kr = reinterpret_cast<const float*>(ks) + kk * D;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc = fmaf(qr[c], kr[c], acc);
        s[kk] = (key0 + kk < kv_valid) ? acc * sm_scale : -INFINITY;
        mx = fmaxf(mx, s[kk]);
      }
      const float mn = fmaxf(m, mx);
      const float alpha = expf(m - mn);
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
      for (int kk = 0; kk < SUB; ++kk) {
        const float p = expf(s[kk] - mn);
        l += p;
        const float* vr = reinterpret_cast<const float*>(vs) + kk * D;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = fmaf(p, vr[c], o[c]);
      }
      m = mn;
    }
  }
  float* orow = out + ((int64_t)h * q_rows + a) * D;
  const bool live = a < q_valid && l > 0.f;
  const float inv = live ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) orow[c] = o[c] * inv;
  if (lse) lse[(int64_t)h * q_rows + a] = live ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------------------
// bf16 MFMA path, d = 128, block = 128
// ---------------------------------------------------------------------------
// One (head, query block) item, or one half of its block list, by one
// workgroup of four waves (attend_blocks in attend_bf16.h).  A halved item
// ends by publishing its unnormalised partial state, or, when the other half
// is already published, by combining the two and writing the output.
constexpr int kPartO = 16 * 256 * 4;              // fp32 O of the 256 lanes
constexpr int kSlotFloats = kPartO + 2 * 256;     // + running max and sum per lane

__device__ __forceinline__ void attend_item(
    int unit, int split, float* __restrict__ partial, int32_t* __restrict__ done, int* flag,
    uint16_t* kl, uint16_t* vl, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ col_slot, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    int nqb, int nkb, int64_t q_rows, int64_t q_valid, int64_t kv_valid, float scale_log2) {
  const int item = unit >> 1, part = unit & 1;
  const int tid = threadIdx.x;
  const int h = item / nqb, i = item % nqb;
  // every value below is uniform across the workgroup; readfirstlane keeps it
  // in scalar registers (buffer descriptors need them)
  const Range range = unit_range(row_ptr, item, part, split);
  const int e0 = __builtin_amdgcn_readfirstlane(range.lo);
  const int e1 = __builtin_amdgcn_readfirstlane(range.hi);
  AttnState st;
  attend_blocks(st, CsrBlockList{col_idx, col_slot, h, nkb}, e0, e1, kl, vl, q, k, v, h, i,
                q_rows, kv_valid, scale_log2);

  if (range.halved) {
    // Partial state of this half: value x of O chunk c = 4u + r4 of lane tid
    // at float (4c + x)*256 + tid, so that each single-word store or load
    // instruction of a wave covers 256 contiguous bytes (whole lines, which
    // matters for stores that write through the L2).
    float* mine = partial + ((size_t)item * 2 + part) * kSlotFloats;
    const float* other = partial + ((size_t)item * 2 + (part ^ 1)) * kSlotFloats;
    if (tid == 0) *flag = __hip_atomic_load(&done[item], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int merge = *flag;
    __syncthreads();
    if (!merge) {
      // the other half has not published: publish this one, then count;
      // whichever half counts second combines.  The partial state goes out
      // as device-coherent stores (they write through the XCD's L2) and each
      // lane waits for its own to complete before the barrier, so no
      // device-scope fence (a write-back and invalidate of the whole L2,
      // which would drop the key/value blocks the XCD's other workgroups
      // are reading) is needed.
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            __hip_atomic_store(&mine[(4 * (4 * u + r4) + x) * 256 + tid], st.oacc[u][4 * r4 + x],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&mine[kPartO + tid], st.m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&mine[kPartO + 256 + tid], st.l_run, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);   // this lane's stores have completed
      __syncthreads();
      if (tid == 0)
        *flag = __hip_atomic_fetch_add(&done[item], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      merge = *flag;
      if (!merge) return;
    }
    // The other half's state was complete before its count, which this half
    // has seen; device-coherent loads read it past any stale L2 copy.
    // Combine in fixed half order (half 0 first), so the result does not
    // depend on which half finished first: with M = max(m0, m1),
    //   O = O1 * 2^(m1 - M) + O0 * 2^(m0 - M),  l likewise.
    const float m_o = __hip_atomic_load(&other[kPartO + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float l_o =
        __hip_atomic_load(&other[kPartO + 256 + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float m0 = part ? m_o : st.m_run, m1 = part ? st.m_run : m_o;
    const float l0 = part ? l_o : st.l_run, l1 = part ? st.l_run : l_o;
    const float mm = fmaxf(m0, m1);
    const bool any = mm > -INFINITY;
    const float a0 = any ? __builtin_amdgcn_exp2f(m0 - mm) : 0.f;
    const float a1 = any ? __builtin_amdgcn_exp2f(m1 - mm) : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float ov[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          ov[x] = __hip_atomic_load(&other[(4 * (4 * u + r4) + x) * 256 + tid], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float own = st.oacc[u][4 * r4 + x];
          const float v0 = part ? ov[x] : own, v1 = part ? own : ov[x];
          st.oacc[u][4 * r4 + x] = fmaf(v1, a1, v0 * a0);
        }
      }
    st.l_run = fmaf(l1, a1, l0 * a0);
    st.m_run = mm;
  }
  store_rows(st, out, lse, h, i, q_rows, q_valid);
}

// Persistent (max_units unbounded): each workgroup pops units from its XCD's
// queue until all queues are empty; with max_units = 1 and one workgroup per
// unit it is the plain one-item-per-workgroup launch.  Either way every
// workgroup exits once the queues are empty (every workgroup reaches that exit; no workgroup waits on another:
// the half that combines only reads what the other half already published).
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ col_slot,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
    float* __restrict__ lse, const int32_t* __restrict__ items, const int32_t* __restrict__ xq,
    int32_t* __restrict__ ctr, int split, float* __restrict__ partial, int32_t* __restrict__ done,
    int max_units, uint64_t* __restrict__ wg_clock, int nqb, int nkb, int64_t q_rows,
    int64_t q_valid, int64_t kv_valid, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) uint16_t kl[kB * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t vl[kB * kD];
  __shared__ int next_item, flag;
  const uint64_t t_start = wg_clock ? __builtin_amdgcn_s_memrealtime() : 0;
  const int home = xcc_id();
  for (int n = 0; n < max_units; ++n) {
    if (threadIdx.x == 0) next_item = pop_item(items, xq, ctr, home);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(next_item);   // uniform: scalar loads below
    __syncthreads();
    if (item < 0) break;
    attend_item(item, split, partial, done, &flag, kl, vl, q, row_ptr, col_idx, col_slot, k, v, out,
                lse, nqb, nkb, q_rows, q_valid, kv_valid, scale_log2);
  }
  if (wg_clock && threadIdx.x == 0) {
    wg_clock[2 * blockIdx.x] = t_start;
    wg_clock[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

template <int D, int BLK>
hipError_t f32_launch(const Dims& g, const void* q, const int32_t* row_ptr,
                      const int32_t* col_idx, const int32_t* col_slot, const void* k,
                      const void* v, void* out, float* lse, const int32_t* items, float sm,
                      hipStream_t s) {
  hipLaunchKernelGGL((attn_f32_kernel<D, BLK>), dim3(g.H * g.nqb), dim3(BLK), 0, s,
                     (const float*)q, row_ptr, col_idx, col_slot, (const float*)k,
                     (const float*)v, (float*)out, lse, items, g.nqb, g.nkb, g.q_rows,
                     g.q_valid, g.kv_rows, g.kv_valid, sm);
  return hipGetLastError();
}

}  // namespace

namespace {
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }
// units (up to two per item), xq, ctr, done
size_t queue_bytes(int rows) { return round256(sizeof(int32_t) * ((size_t)3 * rows + 2 * kXcd + 1)); }
size_t partial_bytes(int rows) { return sizeof(float) * (size_t)rows * 2 * kSlotFloats; }

// Items are split in halves when whole items would leave the last round of
// the persistent grid (two workgroups per CU) more than 5% idle: items of
// near-equal length then finish together, one round short of the whole
// grid.  Halving doubles the rounds and so halves that idle fraction.
bool split_items(const Dims& g) {
  if (g.dtype != SA_BF16) return false;
  const int64_t rows = (int64_t)g.H * g.nqb, slots = 2 * (int64_t)cu_count();
  const int64_t rounds = (rows + slots - 1) / slots;
  return (double)(rounds * slots) > 1.05 * (double)rows;
}


// Finest head grouping whose (range, head group, half) groups fit in LDS.
QueueShape queue_shape(const Dims& g) {
  int hs = 0;
  while (2 * (kXcd + ((g.H - 1) >> hs) + 1) > kQueueMaxGroups) ++hs;
  return {g.nqb, hs};
}
}  // namespace

bool attn_supported(int dtype, int d, int B) {
  if (dtype == SA_BF16) return d == kD && B == kB;
  return (d == 64 || d == 128) && (B == 64 || B == 128);
}

size_t attn_queue_ws_bytes(const Dims& g) { return queue_bytes(g.H * g.nqb); }

size_t attn_ws_bytes(const Dims& g) {
  const int rows = g.H * g.nqb;
  return queue_bytes(rows) + (split_items(g) ? partial_bytes(rows) : 0);
}

int attn_workgroups(const Dims& g, int schedule) {
  const int rows = g.H * g.nqb;
  if (g.dtype != SA_BF16) return rows;
  const int units = (split_items(g) ? 2 : 1) * rows;
  return schedule == SA_SCHEDULE_PER_UNIT ? units : std::min(units, 2 * cu_count());
}

hipError_t launch_attn(const Dims& g, const void* q, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* col_slot, const void* k,
                       const void* v, void* out, float* lse, void* ws, size_t ws_bytes,
                       float sm_scale, int schedule, uint64_t* wg_clock, hipStream_t s) {
  const int rows = g.H * g.nqb;
  int32_t* units = static_cast<int32_t*>(ws);
  int32_t* xq = units + 2 * rows;
  int32_t* ctr = xq + kXcd + 1;
  int32_t* done = ctr + kXcd;
  // halves only when the workspace holds their partial states (it was sized
  // on this device by attn_ws_bytes)
  const int split = split_items(g) && ws_bytes >= queue_bytes(rows) + partial_bytes(rows);
  float* partial = split ? reinterpret_cast<float*>(static_cast<char*>(ws) + queue_bytes(rows)) : nullptr;
  hipLaunchKernelGGL(queue_kernel, dim3(1), dim3(kQueueThreads), 0, s, row_ptr, rows,
                     queue_shape(g), split, units, xq, ctr, done);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.dtype == SA_BF16) {
    if (g.d != kD || g.B != kB) return hipErrorInvalidValue;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    // persistent: two resident workgroups per CU, no more than there are units
    const int nunits = (split ? 2 : 1) * rows;
    const bool per_unit = schedule == SA_SCHEDULE_PER_UNIT;
    const int grid = per_unit ? nunits : std::min(nunits, 2 * cu_count());
    hipLaunchKernelGGL(attn_bf16_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t*)q,
                       row_ptr, col_idx, col_slot, (const uint16_t*)k, (const uint16_t*)v,
                       (uint16_t*)out, lse, units, xq, ctr, split, partial, done,
                       per_unit ? 1 : INT_MAX, wg_clock, g.nqb, g.nkb, g.q_rows, g.q_valid,
                       g.kv_valid, scale_log2);
    return hipGetLastError();
  }
  if (g.d == 64 && g.B == 64) return f32_launch<64, 64>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, units, sm_scale, s);
  if (g.d == 64 && g.B == 128) return f32_launch<64, 128>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, units, sm_scale, s);
  if (g.d == 128 && g.B == 64) return f32_launch<128, 64>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, units, sm_scale, s);
  if (g.d == 128 && g.B == 128) return f32_launch<128, 128>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, units, sm_scale, s);
  return hipErrorInvalidValue;
}

}  // namespace sa
