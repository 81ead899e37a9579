// Critical-KV estimation and sparse attention in one pass ("Dynamic Sparsity
// in Large-Scale Video DiT Training", section "The idea": kernels that fuse
// the estimation of the critical keys and values with the sparse attention,
// keep the intermediates on chip and never build the full score matrix).
//
// Per (head, query block) item, one workgroup:
//   1. scores of the item's query block against every key block of its head
//      from the block means or their rank-r projections (fp64, L2-resident
//      inputs of the pooling pass), held in registers;
//   2. the kept set, as an order-preserving uint64 key per block and a cut:
//      - top-k: the key is the score; the k-th largest key is found by an
//        8-bit radix search (block-wide 256-bin histograms in LDS);
//      - top-p with a top-k floor (the Top-p sparse-attention abstract): the
//        key is the block's softmax mass (fp64, max-subtracted); the same
//        radix search, with each bin also summing its masses as 2^-62 fixed
//        point (exact, order-free integer sums), finds the block at which the
//        cumulative mass in key order first reaches p; the floor then raises
//        the count to min(k, nKB) by the counting search;
//      blocks above the cut key are kept, and of those equal to it the
//      lowest ids (the ranking's tie rule);
//   3. the kept block ids, ascending, into an LDS list (and, when asked, the
//      row's mask words for checking);
//   4. attention over that list (attend_blocks, the same core as the three-call
//      path's forward), straight from the full K and V.
// No score matrix, mask or CSR goes to memory (the optional mask output
// aside).  Items go head by head.  Top-k items all keep min(k, nKB) blocks:
// one workgroup per item, mapped so that each XCD takes a contiguous run of
// items (the hardware deals workgroups to the XCDs in turn), which keeps
// neighbouring query blocks of a head, whose block sets overlap, in one L2.
// Top-p items keep different numbers of blocks (from a few to nearly all
// between heads): two persistent workgroups per CU take items from their
// XCD's contiguous range through a counter, and from the other ranges once
// theirs is empty; each takes its first item without the counter, so the
// workgroups do not all queue on the counters at the start (measured: 2-3%
// faster than the one-item grid on the 40-head layer and the 720p rank
// share, 0.6% slower at 480p).
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "attend_bf16.h"

namespace sa {
namespace {

using namespace bf16mma;

constexpr int kThreads = 256;
constexpr int kMaxPer = 16;            // nKB <= 4096 = 256 threads x 16 keys
constexpr int kFusedXcd = 8;

// Next item for a persistent workgroup.  Range x holds the items
// [x*items/8, (x+1)*items/8) (head-major, so the workgroups on one XCD share
// a head's key/value blocks in its L2) and belongs to the workgroups b with
// b % 8 == x, which the hardware deals to XCD x; ctr[x] is the range's
// cursor.  A workgroup takes from its own range first, then from the
// others'.  -1 once every range is exhausted.
__device__ __forceinline__ int fused_pop(int32_t* ctr, int items, int home) {
  for (int k = 0; k < kFusedXcd; ++k) {
    const int x = (home + k) & (kFusedXcd - 1);
    const int lo = (int)((int64_t)x * items / kFusedXcd);
    const int n = (int)((int64_t)(x + 1) * items / kFusedXcd) - lo;
    if (n <= 0) continue;
    if (__hip_atomic_load(&ctr[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
    const int idx = atomicAdd(&ctr[x], 1);
    if (idx < n) return lo + idx;
  }
  return -1;
}

// Sets each range's cursor past the first tickets, which the workgroups
// take without atomics: workgroup b starts with item b / 8 of range b % 8.
__global__ void fused_clear_kernel(int32_t* ctr, int grid) {
  const int x = threadIdx.x;
  if (x < kFusedXcd) ctr[x] = (grid - x + kFusedXcd - 1) / kFusedXcd;
}

// fp64 -> uint64 whose unsigned order is the numeric order (finite values)
__device__ __forceinline__ uint64_t order_key(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// The mass behind a top-p key (a non-negative fp64), as 2^-62 fixed point:
// a whole row sums to at most 2^62 plus the rounding of nKB terms.
__device__ __forceinline__ uint64_t fixed_mass(uint64_t key) {
  const double m = __longlong_as_double((long long)(key & 0x7fffffffffffffffull));
  return __double2ull_rn(m * 0x1p62);
}

struct FusedLds {
  uint16_t ids[4096];                  // kept block ids, ascending
  int hist[256];
  unsigned long long hmass[256];       // top-p: each bin's fixed-point mass
  int red[kThreads / kWave + 1];
  double redd[kThreads / kWave + 1];
  uint64_t redu[kThreads / kWave + 1];
  int digit, need, count_before, eq;
  uint64_t mass_before;
  uint32_t bits[128];                  // the row's mask words (optional output)
  double qrow[128];                    // the item's query-block vector (mean or projection)
};

// The `need`-th largest of the row's keys (thread t holds keys of blocks
// j0 .. j0+per-1, below nkb), 8 bits at a time from the top.  Returns the cut
// key; *need_out is how many keys equal to it are kept (the lowest ids).
// Invariant: `need` of the keys that match `prefix` on the bits already fixed
// must still be kept, counting from the largest.
__device__ __forceinline__ uint64_t kth_key(const uint64_t (&key)[kMaxPer], int per, int j0,
                                            int nkb, int need, FusedLds& sh, int* need_out) {
  const int t = threadIdx.x;
  uint64_t prefix = 0, pmask = 0;
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
  *need_out = need;
  return prefix;
}

// Top-p cut over mass keys: the block, in key order (ties to the lower id),
// at which the cumulative fixed-point mass first reaches P, for
// 0 < P <= the row's total.  Returns m_p, the number of blocks up to and
// including it; *cut and *need_out give the kept set as kth_key does.
// Invariant: the keys above `prefix` (numerically, on the bits already fixed)
// hold fixed mass `above` < P, and those matching it reach P.
__device__ __forceinline__ int top_p_cut(const uint64_t (&key)[kMaxPer], int per, int j0, int nkb,
                                         uint64_t P, FusedLds& sh, uint64_t* cut, int* need_out) {
  const int t = threadIdx.x;
  uint64_t prefix = 0, pmask = 0, above = 0;
  int n_above = 0, eq = 0;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    sh.hist[t] = 0;
    sh.hmass[t] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u)
      if (u < per && j0 + u < nkb && (key[u] & pmask) == prefix) {
        const int b = (key[u] >> shift) & 0xff;
        atomicAdd(&sh.hist[b], 1);
        atomicAdd(&sh.hmass[b], (unsigned long long)fixed_mass(key[u]));
      }
    __syncthreads();
    if (t < kWave) {
      const int b0 = 4 * t;
      const int c0 = sh.hist[b0], c1 = sh.hist[b0 + 1], c2 = sh.hist[b0 + 2], c3 = sh.hist[b0 + 3];
      const uint64_t m0 = sh.hmass[b0], m1 = sh.hmass[b0 + 1], m2 = sh.hmass[b0 + 2],
                     m3 = sh.hmass[b0 + 3];
      const int cmine = c0 + c1 + c2 + c3;
      const uint64_t mmine = m0 + m1 + m2 + m3;
      int cinc = cmine;
      uint64_t minc = mmine;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int oc = __shfl_down(cinc, off, kWave);
        const uint64_t om = __shfl_down(minc, off, kWave);
        if (t + off < kWave) {
          cinc += oc;
          minc += om;
        }
      }
      // mass and count of the keys ranked before this lane's top bin
      const uint64_t base = above + (minc - mmine);
      const int cbase = cinc - cmine;
      const uint64_t s3 = base + m3, s2 = s3 + m2, s1 = s2 + m1, s0 = s1 + m0;
      // the digit: the first bin from the top whose suffix mass reaches P
      int d = -1, eqd = 0, cb = 0;
      uint64_t mb = 0;
      if (base < P && s3 >= P) { d = b0 + 3; mb = base; cb = cbase; eqd = c3; }
      else if (s3 < P && s2 >= P) { d = b0 + 2; mb = s3; cb = cbase + c3; eqd = c2; }
      else if (s2 < P && s1 >= P) { d = b0 + 1; mb = s2; cb = cbase + c3 + c2; eqd = c1; }
      else if (s1 < P && s0 >= P) { d = b0; mb = s1; cb = cbase + c3 + c2 + c1; eqd = c0; }
      if (d >= 0) {
        sh.digit = d;
        sh.mass_before = mb;
        sh.count_before = cb;
        sh.eq = eqd;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)sh.digit << shift;
    pmask |= (uint64_t)0xff << shift;
    above = sh.mass_before;
    n_above += sh.count_before;
    eq = sh.eq;
  }
  // `eq` keys equal the cut key, each of fixed mass q > 0 (the cut adds mass):
  // the first j of them (by id) bring the cumulative mass to P
  const uint64_t q = fixed_mass(prefix);
  int j = eq;
  if (q > 0) {
    const uint64_t jj = (P - above + q - 1) / q;
    j = jj < 1 ? 1 : (jj > (uint64_t)eq ? eq : (int)jj);
  }
  *cut = prefix;
  *need_out = j;
  return n_above + j;
}

template <bool kTopP>
__global__ __launch_bounds__(kThreads, 2) void fused_select_kernel(
    const double* __restrict__ qx, const double* __restrict__ kx, int dim, double scale,
    double top_p, int top_k, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint32_t* __restrict__ mask_bits, int heads, int nqb, int nkb, int W, int64_t q_rows,
    int64_t q_valid, int64_t kv_valid, float scale_log2, int persistent, int32_t* ctr) {
  __shared__ __attribute__((aligned(1024))) uint16_t kl[kB * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t vl[kB * kD];
  __shared__ FusedLds sh;
  __shared__ int next_item;
  const int items = heads * nqb;
  const int home = persistent ? (int)(blockIdx.x % kFusedXcd) : 0;
  const int per_xcd = (items + kFusedXcd - 1) / kFusedXcd;
  const int t = threadIdx.x;
  for (int n = 0;; ++n) {
  int item;
  if (persistent) {
    if (t == 0) {
      if (n == 0) {
        // the first ticket, taken statically (the range cursors start past them)
        const int lo = (int)((int64_t)home * items / kFusedXcd);
        const int cnt = (int)((int64_t)(home + 1) * items / kFusedXcd) - lo;
        const int idx = blockIdx.x / kFusedXcd;
        next_item = idx < cnt ? lo + idx : fused_pop(ctr, items, home);
      } else {
        next_item = fused_pop(ctr, items, home);
      }
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(next_item);
    __syncthreads();
  } else {
    // one item per workgroup, contiguous items per XCD: workgroup b runs on
    // XCD b % 8
    item = n == 0 ? (blockIdx.x % kFusedXcd) * per_xcd + blockIdx.x / kFusedXcd : -1;
    if (item >= items) item = -1;
  }
  if (item < 0) break;
  const int h = item / nqb, i = item % nqb;

  // ---- 1. scores: thread t owns key blocks t*per .. t*per+per-1 ----------
  for (int c = t; c < dim; c += kThreads) sh.qrow[c] = qx[(int64_t)item * dim + c];
  for (int w = t; w < W; w += kThreads) sh.bits[w] = 0u;
  __syncthreads();
  const int per = (nkb + kThreads - 1) / kThreads;
  const int j0 = t * per;
  double sc[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    sc[u] = 0.0;
    const int j = j0 + u;
    if (u < per && j < nkb) {
      const double* kr = kx + ((int64_t)h * nkb + j) * dim;
      double acc = 0.0;
      for (int c = 0; c < dim; ++c) acc = fma(sh.qrow[c], kr[c], acc);
      sc[u] = acc * scale + 0.0;   // + 0.0: -0 ties with +0, as numbers do
    }
  }

  // ---- 2. the cut ----------------------------------------------------------
  uint64_t key[kMaxPer];
  uint64_t cut;
  int need;
  if constexpr (kTopP) {
    // softmax masses: max-subtracted, each thread's terms in block order, then
    // a fixed reduction tree
    double mx = -DBL_MAX;
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u)
      if (u < per && j0 + u < nkb) mx = fmax(mx, sc[u]);
    mx = block_reduce(mx, sh.redd, [](double a, double b) { return fmax(a, b); });
    double part = 0.0;
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u)
      if (u < per && j0 + u < nkb) {
        sc[u] = exp(sc[u] - mx);
        part += sc[u];
      }
    const double tot = block_reduce(part, sh.redd, [](double a, double b) { return a + b; });
    uint64_t mine = 0;
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) {
      key[u] = 0;   // below every real key
      if (u < per && j0 + u < nkb) {
        key[u] = order_key(sc[u] / tot);
        mine += fixed_mass(key[u]);
      }
    }
    const uint64_t total =
        block_reduce(mine, sh.redu, [](uint64_t a, uint64_t b) { return a + b; });
    // p >= 1, or a prefix that never reaches p through rounding: every block
    int m = nkb;
    const uint64_t P = top_p <= 0.0 ? 1ull : (uint64_t)fmax(1.0, rint(top_p * 0x1p62));
    if (top_p < 1.0 && P <= total) m = top_p_cut(key, per, j0, nkb, P, sh, &cut, &need);
    const int floor_k = min(top_k, nkb);
    if (m == nkb || floor_k > m) cut = kth_key(key, per, j0, nkb, max(m, floor_k), sh, &need);
  } else {
#pragma unroll
    for (int u = 0; u < kMaxPer; ++u) key[u] = (u < per && j0 + u < nkb) ? order_key(sc[u]) : 0;
    cut = kth_key(key, per, j0, nkb, min(top_k, nkb), sh, &need);
  }
  // kept: every key above `cut`, and the first `need` keys equal to it by id

  // ---- 3. kept ids, ascending, into LDS -----------------------------------
  int eq = 0;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u)
    if (u < per && j0 + u < nkb && key[u] == cut) ++eq;
  int eq_all;
  int eq_before = block_inclusive_scan(eq, sh.red, &eq_all) - eq;
  int kept = 0;
  uint32_t keep_bits = 0;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    if (u < per && j0 + u < nkb) {
      bool keep = key[u] > cut;
      if (key[u] == cut) {
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
  __syncthreads();   // LDS is reused by the next item
  }
}

}  // namespace

hipError_t launch_fused(const Dims& g, const double* qx, const double* kx, int dim, double scale,
                        int mode, double top_p, int top_k, const void* q, const void* k,
                        const void* v, void* out, float* lse, uint32_t* mask_bits, float sm_scale,
                        int32_t* ctr, hipStream_t s) {
  if (g.dtype != SA_BF16 || g.d != kD || g.B != kB || g.nkb > kThreads * kMaxPer || dim > 128 ||
      (mode != SA_TOP_P && mode != SA_TOP_K))
    return hipErrorInvalidValue;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  // Top-p rows keep different numbers of blocks: two persistent workgroups
  // per CU take items from per-XCD queues (and steal).  Top-k rows are all
  // the same length: one workgroup per item, handed out by the dispatcher.
  const int persistent = mode == SA_TOP_P;
  const int64_t items = (int64_t)g.H * g.nqb;
  const int64_t per_xcd = (items + kFusedXcd - 1) / kFusedXcd;
  if (per_xcd * kFusedXcd > INT_MAX) return hipErrorInvalidValue;
  const int grid = persistent ? (int)std::min<int64_t>(items, 2 * (int64_t)cus)
                              : (int)(per_xcd * kFusedXcd);
  if (persistent) {
    hipLaunchKernelGGL(fused_clear_kernel, dim3(1), dim3(64), 0, s, ctr, grid);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  auto kern = mode == SA_TOP_P ? fused_select_kernel<true> : fused_select_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s, qx, kx,
                     dim, scale, top_p, top_k, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (uint16_t*)out, lse, mask_bits, g.H, g.nqb, g.nkb, g.W,
                     g.q_rows, g.q_valid, g.kv_valid, scale_log2, persistent, ctr);
  return hipGetLastError();
}

}  // namespace sa
