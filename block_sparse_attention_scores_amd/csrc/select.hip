// Per-row block selection: Top-p routing with a Top-k safety floor, or a fixed
// top-k (the Top-p sparse-attention abstract, mlsift listing, tag "sequence
// parallelism"; "Dynamic Sparsity in Large-Scale Video DiT Training", section
// "The idea": rank the pairs and keep the critical ones).
//
// One workgroup per (head, query block) row.  The row's scores are staged in
// LDS; top-p mode turns them into softmax masses (fp64, max-subtracted, sum in
// a fixed order).  A bitonic sort in LDS orders (value descending, block id
// ascending); the cumulative mass comes from a block-wide scan in fp64.  The
// kept set is written as a bitmask row plus its count.
#include <float.h>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kSelThreads = 256;
constexpr int kMaxKB = 4096;

// a goes before b: larger value first, then lower block id
__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const double* __restrict__ S, int nkb, int W, int mode, double top_p, int top_k,
    uint32_t* __restrict__ bits_out, int32_t* __restrict__ counts) {
  __shared__ double key[kMaxKB];
  __shared__ int idx[kMaxKB];
  __shared__ uint32_t bits[kMaxKB / 32];
  __shared__ double red[kSelThreads / kWave + 1];
  __shared__ int redi[kSelThreads / kWave + 1];

  const int row = blockIdx.x, t = threadIdx.x;
  int n2 = 1;
  while (n2 < nkb) n2 <<= 1;
  const double* s = S + (int64_t)row * nkb;

  if (mode == SA_TOP_P) {
    double mx = -DBL_MAX;
    for (int j = t; j < nkb; j += kSelThreads) mx = fmax(mx, s[j]);
    mx = block_reduce(mx, red, [](double a, double b) { return fmax(a, b); });
    double part = 0.0;
    for (int j = t; j < nkb; j += kSelThreads) {
      const double e = exp(s[j] - mx);
      key[j] = e;
      part += e;
    }
    const double tot = block_reduce(part, red, [](double a, double b) { return a + b; });
    for (int j = t; j < n2; j += kSelThreads) {
      key[j] = (j < nkb) ? key[j] / tot : -1.0;
      idx[j] = (j < nkb) ? j : 0x7fffffff;
    }
  } else {
    for (int j = t; j < n2; j += kSelThreads) {
      key[j] = (j < nkb) ? s[j] : -DBL_MAX;
      idx[j] = (j < nkb) ? j : 0x7fffffff;
    }
  }
  for (int w = t; w < W; w += kSelThreads) bits[w] = 0u;
  __syncthreads();

  // bitonic sort of n2 (value, id) pairs into "before" order
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = t; p < (n2 >> 1); p += kSelThreads) {
        const int a = 2 * stride * (p / stride) + (p % stride);
        const int b = a + stride;
        const bool up = (a & size) == 0;
        const double va = key[a], vb = key[b];
        const int ia = idx[a], ib = idx[b];
        const bool sw = up ? before(vb, ib, va, ia) : before(va, ia, vb, ib);
        if (sw) {
          key[a] = vb; key[b] = va;
          idx[a] = ib; idx[b] = ia;
        }
      }
      __syncthreads();
    }
  }

  int m;
  const int kf = min(top_k, nkb);
  if (mode == SA_TOP_P) {
    if (top_p >= 1.0) {
      m = nkb;
    } else {
      // inclusive scan over the sorted masses: each thread owns a contiguous
      // chunk; count positions whose cumulative mass is still below p
      const int per = (nkb + kSelThreads - 1) / kSelThreads;
      const int lo = min(nkb, t * per), hi = min(nkb, lo + per);
      double local = 0.0;
      for (int j = lo; j < hi; ++j) local += key[j];
      double total;
      const double incl = block_inclusive_scan(local, red, &total);
      double run = incl - local;
      int below = 0;
      for (int j = lo; j < hi; ++j) {
        run += key[j];
        below += (run < top_p) ? 1 : 0;
      }
      below = block_reduce(below, redi, [](int a, int b) { return a + b; });
      m = min(nkb, 1 + below);
    }
    m = max(m, kf);
  } else {
    m = kf;
  }

  for (int pidx = t; pidx < m; pidx += kSelThreads) {
    const int j = idx[pidx];
    if ((unsigned)j < (unsigned)nkb) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // the count is the popcount of the written row, so the CSR built from it
  // always matches the mask (even if non-finite scores broke the ordering)
  int c = 0;
  for (int w = t; w < W; w += kSelThreads) {
    bits_out[(int64_t)row * W + w] = bits[w];
    c += __popc(bits[w]);
  }
  c = block_reduce(c, redi, [](int a, int b) { return a + b; });
  if (t == 0) counts[row] = c;
}

}  // namespace

hipError_t launch_select(const Dims& g, const double* scores, int mode, double top_p,
                         int top_k, uint32_t* bits, int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(g.H * g.nqb), dim3(kSelThreads), 0, s, scores, g.nkb,
                     g.W, mode, top_p, top_k, bits, counts);
  return hipGetLastError();
}

}  // namespace sa
