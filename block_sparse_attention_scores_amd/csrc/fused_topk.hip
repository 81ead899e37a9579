// Critical-KV estimation and sparse attention in one pass ("Dynamic Sparsity
// in Large-Scale Video DiT Training", section "The idea": kernels that fuse
// the estimation of the critical keys and values with the sparse attention,
// keep the intermediates on chip and never build the full score matrix).
//
// One workgroup per (head, query block) item:
//   1. scores of the item's query block against every key block of its head
//      from the block means or their rank-r projections (fp64, L2-resident
//      inputs of the pooling pass), held in registers;
//   2. the top-k of those scores (ties to the lower block id) by an 8-bit
//      radix search for the k-th largest order-preserving key, with block-wide
//      histograms in LDS;
//   3. the kept block ids, ascending, into an LDS list (and, when asked, the
//      row's mask words for checking);
//   4. attention over that list (attend_blocks, the same core as the three-call
//      path's forward), straight from the full K and V.
// No score matrix, mask or CSR goes to memory (the optional mask output
// aside).  Every item keeps exactly min(k, nKB) blocks, so the grid needs no
// work queue: workgroups are mapped to items so that each XCD takes a
// contiguous run of items (the hardware deals workgroups to the XCDs in
// turn), which keeps neighbouring query blocks of a head, whose block sets
// overlap, in one L2.
#include <float.h>
#include <limits.h>
#include <math.h>

#include "attend_bf16.h"

namespace sa {
namespace {

using namespace bf16mma;

constexpr int kThreads = 256;
constexpr int kMaxPer = 16;            // nKB <= 4096 = 256 threads x 16 keys
constexpr int kFusedXcd = 8;

// fp64 -> uint64 whose unsigned order is the numeric order (finite values)
__device__ __forceinline__ uint64_t order_key(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

struct FusedLds {
  uint16_t ids[4096];                  // kept block ids, ascending
  int hist[256];
  int red[kThreads / kWave + 1];
  int digit, need;
  uint32_t bits[128];                  // the row's mask words (optional output)
  double qrow[128];                    // the item's query-block vector (mean or projection)
};

__global__ __launch_bounds__(kThreads, 2) void fused_topk_kernel(
    const double* __restrict__ qx, const double* __restrict__ kx, int dim, double scale,
    int top_k, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint32_t* __restrict__ mask_bits, int items, int per_xcd, int nqb, int nkb, int W,
    int64_t q_rows, int64_t q_valid, int64_t kv_valid, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) uint16_t kl[kB * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t vl[kB * kD];
  __shared__ FusedLds sh;
  // contiguous items per XCD: workgroup b runs on XCD b % 8
  const int item = (blockIdx.x % kFusedXcd) * per_xcd + blockIdx.x / kFusedXcd;
  if (item >= items) return;
  const int h = item / nqb, i = item % nqb;
  const int t = threadIdx.x;

  // ---- 1. scores: thread t owns key blocks t*per .. t*per+per-1 ----------
  for (int c = t; c < dim; c += kThreads) sh.qrow[c] = qx[(int64_t)item * dim + c];
  for (int w = t; w < W; w += kThreads) sh.bits[w] = 0u;
  __syncthreads();
  const int per = (nkb + kThreads - 1) / kThreads;
  const int j0 = t * per;
  uint64_t key[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    key[u] = 0;   // below every real key
    const int j = j0 + u;
    if (u < per && j < nkb) {
      const double* kr = kx + ((int64_t)h * nkb + j) * dim;
      double acc = 0.0;
      for (int c = 0; c < dim; ++c) acc = fma(sh.qrow[c], kr[c], acc);
      key[u] = order_key(acc * scale + 0.0);   // + 0.0: -0 ties with +0, as numbers do
    }
  }
  const int n_keep = min(top_k, nkb);

  // ---- 2. k-th largest key, 8 bits at a time from the top ----------------
  // Invariant: `need` of the keys that match `prefix` on the bits already
  // fixed must still be kept, counting from the largest.
  uint64_t prefix = 0, pmask = 0;
  int need = n_keep;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    sh.hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u)
      if (u < per && j0 + u < nkb && (key[u] & pmask) == prefix)
        atomicAdd(&sh.hist[(key[u] >> shift) & 0xff], 1);
    __syncthreads();
    if (t < kWave) {
      // lane l holds bins 4l .. 4l+3; suffix sums from the top bin down
      const int b0 = 4 * t;
      const int c0 = sh.hist[b0], c1 = sh.hist[b0 + 1], c2 = sh.hist[b0 + 2], c3 = sh.hist[b0 + 3];
      const int mine = c0 + c1 + c2 + c3;
      // inclusive scan from the high lanes: above[l] = sum of lanes > l
      int incl = mine;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_down(incl, off, kWave);
        if (t + off < kWave) incl += o;
      }
      const int above = incl - mine;
      // the digit: the largest bin whose suffix count reaches `need`
      const int s3 = above + c3, s2 = s3 + c2, s1 = s2 + c1, s0 = s1 + c0;
      int d = -1, before = 0;
      if (s3 >= need && above < need) { d = b0 + 3; before = above; }
      else if (s2 >= need && s3 < need) { d = b0 + 2; before = s3; }
      else if (s1 >= need && s2 < need) { d = b0 + 1; before = s2; }
      else if (s0 >= need && s1 < need) { d = b0; before = s1; }
      if (d >= 0) {
        sh.digit = d;
        sh.need = need - before;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sh.digit << shift;
    pmask |= (uint64_t)0xff << shift;
    need = sh.need;
  }
  // prefix is the k-th largest key; the first `need` keys equal to it (by
  // block id) are kept along with every larger key

  // ---- 3. kept ids, ascending, into LDS -----------------------------------
  int eq = 0;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u)
    if (u < per && j0 + u < nkb && key[u] == prefix) ++eq;
  int eq_all;
  int eq_before = block_inclusive_scan(eq, sh.red, &eq_all) - eq;
  int kept = 0;
  uint32_t keep_bits = 0;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    if (u < per && j0 + u < nkb) {
      bool keep = key[u] > prefix;
      if (key[u] == prefix) {
        keep = eq_before < need;
        ++eq_before;
      }
      if (keep) {
        keep_bits |= 1u << u;
        ++kept;
      }
    }
  }
  int kept_all;
  int pos = block_inclusive_scan(kept, sh.red, &kept_all) - kept;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u)
    if (keep_bits >> u & 1u) {
      const int j = j0 + u;
      sh.ids[pos++] = (uint16_t)j;
      if (mask_bits) atomicOr(&sh.bits[j >> 5], 1u << (j & 31));
    }
  __syncthreads();
  if (mask_bits)
    for (int w = t; w < W; w += kThreads) mask_bits[(int64_t)item * W + w] = sh.bits[w];

  // ---- 4. attention over the kept blocks ----------------------------------
  AttnState st;
  attend_blocks(st, LdsBlockList{sh.ids, h, nkb}, 0, kept_all, kl, vl, q, k, v, h, i, q_rows,
                kv_valid, scale_log2);
  store_rows(st, out, lse, h, i, q_rows, q_valid);
}

}  // namespace

hipError_t launch_fused_topk(const Dims& g, const double* qx, const double* kx, int dim,
                             double scale, int top_k, const void* q, const void* k, const void* v,
                             void* out, float* lse, uint32_t* mask_bits, float sm_scale,
                             hipStream_t s) {
  if (g.dtype != SA_BF16 || g.d != kD || g.B != kB || g.nkb > kThreads * kMaxPer || dim > 128)
    return hipErrorInvalidValue;
  const int items = g.H * g.nqb;
  const int per_xcd = (items + kFusedXcd - 1) / kFusedXcd;
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(fused_topk_kernel, dim3(per_xcd * kFusedXcd), dim3(kThreads), 0, s, qx, kx,
                     dim, scale, top_k, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (uint16_t*)out, lse, mask_bits, items, per_xcd, g.nqb,
                     g.nkb, g.W, g.q_rows, g.q_valid, g.kv_valid, scale_log2);
  return hipGetLastError();
}

}  // namespace sa
