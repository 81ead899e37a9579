// Attention over the selected key blocks only ("Dynamic Sparsity in
// Large-Scale Video DiT Training", section "The idea": sparse attention
// kernels that never build the full score matrix; neighbouring queries, one
// query block, share one selected key/value set) with work items ordered
// longest-first so uneven per-head sparsity does not leave CUs idle (same
// page, "Once the work is uneven"; the Top-p sparse-attention abstract, mlsift
// listing: rank-level stragglers).
//
// queue_kernel : one workgroup sorts the (head, query block) items by their
//                selected-block count, largest first, ties by item id
//                (bitonic sort of packed 32-bit keys in LDS).  Workgroups of
//                the attention grid take items in that order, so the hardware
//                dispatcher hands the longest items out first.
// attn_f32     : fp32 path (one thread per query, 32-key LDS sub-tiles,
//                online softmax in fp32).
// attn_bf16    : bf16 MFMA path, d = 128, block = 128.  One workgroup of four
//                waves per item; wave w owns queries 32w..32w+31.  Per key
//                block: K (row-major) and V (transposed, XOR-swizzled 4-key
//                groups) are staged in LDS; S^T = K Q^T with
//                v_mfma_f32_32x32x16_bf16 so that each lane holds one query's
//                scores (row max = local max + one cross-half exchange);
//                online softmax in the exp2 domain; P^T goes straight from the
//                accumulator registers into the B operand of O^T = V^T P^T.
#include <float.h>
#include <math.h>

#include "sa_common.h"

namespace sa {
namespace {

// ---------------------------------------------------------------------------
// work queue
// ---------------------------------------------------------------------------
constexpr int kQueueThreads = 1024;
constexpr int kQueueMax = 32768;

__global__ __launch_bounds__(kQueueThreads) void queue_kernel(const int32_t* __restrict__ row_ptr,
                                                              int rows, int nkb, int n2,
                                                              int idbits,
                                                              int32_t* __restrict__ items) {
  __shared__ uint32_t key[kQueueMax];
  const int t = threadIdx.x;
  const uint32_t idmask = (1u << idbits) - 1u;
  for (int r = t; r < n2; r += kQueueThreads) {
    if (r < rows) {
      const uint32_t c = (uint32_t)(row_ptr[r + 1] - row_ptr[r]);
      key[r] = (((uint32_t)nkb - min(c, (uint32_t)nkb)) << idbits) | (uint32_t)r;
    } else {
      key[r] = 0xffffffffu;
    }
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = t; p < (n2 >> 1); p += kQueueThreads) {
        const int a = 2 * stride * (p / stride) + (p % stride);
        const int b = a + stride;
        const uint32_t ka = key[a], kb = key[b];
        const bool up = (a & size) == 0;
        if ((ka > kb) == up) {
          key[a] = kb;
          key[b] = ka;
        }
      }
      __syncthreads();
    }
  }
  for (int r = t; r < rows; r += kQueueThreads) items[r] = (int32_t)(key[r] & idmask);
}

__global__ void identity_queue_kernel(int rows, int32_t* __restrict__ items) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < rows) items[r] = r;
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
  const int item = items[blockIdx.x];
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
constexpr int kD = 128, kB = 128;
constexpr int kKsStride = kD + 8;   // K tile row stride in bf16 (272 bytes)
constexpr int kVtStride = kB + 8;   // V^T tile row stride in bf16 (272 bytes)

__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const int32_t* __restrict__ col_slot,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
    float* __restrict__ lse, const int32_t* __restrict__ items, int nqb, int nkb,
    int64_t q_rows, int64_t q_valid, int64_t kv_rows, int64_t kv_valid, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kB * kKsStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kD * kVtStride];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, g = lane >> 5;
  const int item = items[blockIdx.x];
  const int h = item / nqb, i = item % nqb;
  const int64_t qrow = (int64_t)i * kB + 32 * wave + lq;   // this lane's query row

  // Q fragments (B operand of S^T = K Q^T): d = 16s + 8g .. +8
  bf16x8 qf[8];
  {
    const uint16_t* qp = q + ((int64_t)h * q_rows + qrow) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[u][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

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
    const uint16_t* kb = k + blk * (kB * kD);
    const uint16_t* vb = v + blk * (kB * kD);

    // global -> registers: K as 8 x 16 B row chunks, V as 2 x (4 rows x 8 d)
    uint4 kr[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c16 = tid + 256 * it;
      kr[it] = *reinterpret_cast<const uint4*>(kb + (c16 >> 4) * kD + (c16 & 15) * 8);
    }
    uint4 vr[2][4];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int sub = tid + 256 * it, dc = sub & 15, kg = sub >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vr[it][r] = *reinterpret_cast<const uint4*>(vb + (4 * kg + r) * kD + 8 * dc);
    }
    __syncthreads();   // everyone is done reading the previous tiles
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c16 = tid + 256 * it;
      *reinterpret_cast<uint4*>(ks + (c16 >> 4) * kKsStride + (c16 & 15) * 8) = kr[it];
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int sub = tid + 256 * it, dc = sub & 15, kg = sub >> 4;
      const int kgs = kg ^ dc;   // swizzle: d >> 3 == dc for these 8 rows
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[it][0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[it][1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[it][2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[it][3]);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int c = x >> 1;
        uint2 pr;
        if (x & 1) {
          pr.x = (w0[c] >> 16) | (w1[c] & 0xffff0000u);
          pr.y = (w2[c] >> 16) | (w3[c] & 0xffff0000u);
        } else {
          pr.x = (w0[c] & 0xffffu) | (w1[c] << 16);
          pr.y = (w2[c] & 0xffffu) | (w3[c] << 16);
        }
        *reinterpret_cast<uint2*>(vt + (8 * dc + x) * kVtStride + 4 * kgs) = pr;
      }
    }
    __syncthreads();

    // S^T tile t: keys 32t.., this lane's query; reg r -> key 32t + 8(r/4) + 4g + r%4
    f32x16 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks + (32 * t + lq) * kKsStride + 16 * s + 8 * g);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t], 0, 0, 0);
      }
    }

    const int64_t lim = kv_valid - (int64_t)j * kB;   // keys >= lim are padding
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
        const float x = (kk < lim) ? sacc[t][r] * scale_log2 : -INFINITY;
        sacc[t][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - mn);
    m_run = mn;
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[t][r] - mn);
        sacc[t][r] = p;
        ps += p;
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;

    // O^T += V^T P^T; k-step (t, h2) covers keys 32t + 16h2 .. +16
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint32_t pw[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          pw[x] = pack_bf16x2(sacc[t][8 * h2 + 2 * x], sacc[t][8 * h2 + 2 * x + 1]);
        bf16x8 pf;
        __builtin_memcpy(&pf, pw, 16);
        const int kga = 8 * t + 4 * h2 + g, kgb = kga + 2;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int d = 32 * u + lq;
          const int sw = (d >> 3) & 15;
          const uint2 va = *reinterpret_cast<const uint2*>(vt + d * kVtStride + 4 * (kga ^ sw));
          const uint2 vb2 = *reinterpret_cast<const uint2*>(vt + d * kVtStride + 4 * (kgb ^ sw));
          const uint32_t vw[4] = {va.x, va.y, vb2.x, vb2.y};
          bf16x8 vf;
          __builtin_memcpy(&vf, vw, 16);
          oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[u], 0, 0, 0);
        }
      }
    }
  }

  // finalise: O[query][d], reg r of d-tile u -> d = 32u + 8(r/4) + 4g + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool live = qrow < q_valid && l_tot > 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
  uint16_t* op = out + ((int64_t)h * q_rows + qrow) * kD;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      uint2 w;
      w.x = pack_bf16x2(oacc[u][4 * r4 + 0] * inv, oacc[u][4 * r4 + 1] * inv);
      w.y = pack_bf16x2(oacc[u][4 * r4 + 2] * inv, oacc[u][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + 32 * u + 8 * r4 + 4 * g) = w;
    }
  if (lse && g == 0)
    lse[(int64_t)h * q_rows + qrow] =
        live ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
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

hipError_t launch_queue(const Dims& g, const int32_t* row_ptr, int32_t* items, hipStream_t s) {
  const int rows = g.H * g.nqb;
  int n2 = 1, idbits = 0;
  while (n2 < rows) n2 <<= 1;
  while ((1 << idbits) < rows) ++idbits;
  int cbits = 0;
  while ((1 << cbits) <= g.nkb) ++cbits;
  if (n2 <= kQueueMax && idbits + cbits <= 31) {   // real keys stay below the sentinel
    hipLaunchKernelGGL(queue_kernel, dim3(1), dim3(kQueueThreads), 0, s, row_ptr, rows, g.nkb,
                       n2, idbits, items);
  } else {
    hipLaunchKernelGGL(identity_queue_kernel, dim3((rows + 255) / 256), dim3(256), 0, s, rows,
                       items);
  }
  return hipGetLastError();
}

bool attn_supported(int dtype, int d, int B) {
  if (dtype == SA_BF16) return d == kD && B == kB;
  return (d == 64 || d == 128) && (B == 64 || B == 128);
}

hipError_t launch_attn(const Dims& g, const void* q, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* col_slot, const void* k,
                       const void* v, void* out, float* lse, const int32_t* items,
                       float sm_scale, hipStream_t s) {
  const int rows = g.H * g.nqb;
  if (g.dtype == SA_BF16) {
    if (g.d != kD || g.B != kB) return hipErrorInvalidValue;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(attn_bf16_kernel, dim3(rows), dim3(256), 0, s, (const uint16_t*)q,
                       row_ptr, col_idx, col_slot, (const uint16_t*)k, (const uint16_t*)v,
                       (uint16_t*)out, lse, items, g.nqb, g.nkb, g.q_rows, g.q_valid, g.kv_rows,
                       g.kv_valid, scale_log2);
    return hipGetLastError();
  }
  if (g.d == 64 && g.B == 64) return f32_launch<64, 64>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, items, sm_scale, s);
  if (g.d == 64 && g.B == 128) return f32_launch<64, 128>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, items, sm_scale, s);
  if (g.d == 128 && g.B == 64) return f32_launch<128, 64>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, items, sm_scale, s);
  if (g.d == 128 && g.B == 128) return f32_launch<128, 128>(g, q, row_ptr, col_idx, col_slot, k, v, out, lse, items, sm_scale, s);
  return hipErrorInvalidValue;
}

}  // namespace sa
