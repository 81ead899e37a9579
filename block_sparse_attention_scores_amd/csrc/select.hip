// Per-row block selection: Top-p routing with a Top-k safety floor, or a fixed
// top-k (the Top-p sparse-attention abstract, mlsift listing, tag "sequence
// parallelism"; "Dynamic Sparsity in Large-Scale Video DiT Training", section
// "The idea": rank the pairs and keep the critical ones).
//
// One single-wave workgroup per (head, query block) row.  Top-p mode turns
// the row's scores into softmax masses (fp64, max-subtracted, sum in a fixed
// order).  The kept set is the first m blocks in the order (value
// descending, block id ascending); for top-p, m is the shortest prefix whose
// cumulative mass (fp64) reaches p, raised to the floor.  It is written as a
// bitmask row plus its count.
//
// Rows of up to 1024 blocks stay in registers (select_reg_kernel).  Rows of
// up to 256 blocks are sorted there (lane l holds sorted positions l, l+64,
// ...; strides under 64 exchange across lanes by DPP moves, or ds_bpermute
// for 16 and 32, larger ones swap registers).  Only the keys are sorted; the
// kept blocks then follow from each lane's unsorted keys and the cut key.
// Rows of 257 to 1024 blocks skip the sort: the cut key is found by a bitwise
// search over the key space (the top-p cut from mass sums, the top-k cut and
// the floor from counts).  Longer rows go through an LDS sort of (value, id)
// pairs (select_kernel).
#include <float.h>

#include "sa_common.h"

namespace sa {
namespace {

// a goes before b: larger value first, then lower block id
__device__ __forceinline__ bool before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// LDS (dynamic): key[n2] fp64, idx[n2] int32, bits[W] uint32, n2 = pow2 >= nkb
template <int kSelThreads>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const double* __restrict__ S, int nkb, int n2, int W, int mode, double top_p, int top_k,
    uint32_t* __restrict__ bits_out, int32_t* __restrict__ counts) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sel_lds[];
  double* key = reinterpret_cast<double*>(sel_lds);
  int* idx = reinterpret_cast<int*>(key + n2);
  uint32_t* bits = reinterpret_cast<uint32_t*>(idx + n2);
  __shared__ double red[kSelThreads / kWave + 1];
  __shared__ int redi[kSelThreads / kWave + 1];

  const int row = blockIdx.x, t = threadIdx.x;
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

// Order-preserving map of an fp64 value onto uint64 (larger value, larger
// key); -0.0 is folded onto +0.0 so that equal values compare equal.
__device__ __forceinline__ uint64_t order_key(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v + 0.0);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}
__device__ __forceinline__ double key_value(uint64_t k) {
  const uint64_t u = (k >> 63) ? (k & ~(1ull << 63)) : ~k;
  return __longlong_as_double((long long)u);
}
// Value of lane (l ^ S) for S below 64.  Strides 1, 2 and 8 are a single DPP
// move (quad_perm / row_ror:8); stride 4 picks between row_ror:4 and
// row_ror:12 by lane bit 2; 16 and 32 go through ds_bpermute.
template <int S>
__device__ __forceinline__ int xor_lane(int v) {
  if constexpr (S == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
  } else if constexpr (S == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);
  } else if constexpr (S == 4) {
    const int a = __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true);
    const int b = __builtin_amdgcn_mov_dpp(v, 0x12C, 0xF, 0xF, true);
    return (threadIdx.x & 4) ? a : b;
  } else if constexpr (S == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);
  } else {
    return __shfl_xor(v, S, kWave);
  }
}
template <int S>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v) {
  const int lo = xor_lane<S>((int)(uint32_t)v);
  const int hi = xor_lane<S>((int)(uint32_t)(v >> 32));
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// One compare-exchange stage of the bitonic network (block size SIZE, partner
// distance STRIDE) over positions e = l + 64 k, into descending key order.
// Only keys move: equal keys are interchangeable, and block ids are resolved
// afterwards from each lane's unsorted keys (select_reg_kernel).
template <int K, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stage(uint64_t (&key)[K], int l) {
  if constexpr (STRIDE >= kWave) {
    constexpr int ks = STRIDE / kWave;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (k & ks) continue;
      const int kb = k | ks;
      const bool up = ((kWave * k) & SIZE) == 0;   // SIZE >= 128: lane bits do not matter
      const bool sw = up ? key[kb] > key[k] : key[k] > key[kb];
      if (sw) {
        const uint64_t tk = key[k]; key[k] = key[kb]; key[kb] = tk;
      }
    }
  } else {
    const bool lower = (l & STRIDE) == 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t pk = xor_lane<STRIDE>(key[k]);
      const bool up = ((l + kWave * k) & SIZE) == 0;
      // the lower position of a descending pair keeps the larger key
      key[k] = (lower == up) ? (key[k] > pk ? key[k] : pk) : (key[k] > pk ? pk : key[k]);
    }
  }
}

// The whole network for 64 K keys: sizes 2, 4, ..., 64 K, each with strides
// SIZE/2 down to 1.
template <int K, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic(uint64_t (&key)[K], int l) {
  if constexpr (SIZE <= kWave * K) {
    if constexpr (STRIDE == 0) {
      bitonic<K, SIZE * 2, SIZE>(key, l);
    } else {
      bitonic_stage<K, SIZE, STRIDE>(key, l);
      bitonic<K, SIZE, STRIDE / 2>(key, l);
    }
  }
}

// Largest key kc with at least m valid keys >= kc: the key at position m - 1
// of the descending order, found bit by bit from the top (ballot counts).
template <int K>
__device__ __forceinline__ uint64_t key_at_rank(const uint64_t (&key)[K], int m) {
  uint64_t kq = 0;
  for (int b = 63; b >= 0; --b) {
    const uint64_t cand = kq | (1ull << b);
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) cnt += __popcll(__ballot(key[k] >= cand));   // padding key 0 < cand
    if (cnt >= m) kq = cand;
  }
  return kq;
}

template <int K>  // elements per lane; the sort length is 64 * K
__global__ __launch_bounds__(kWave) void select_reg_kernel(
    const double* __restrict__ S, int nkb, int W, int mode, double top_p, int top_k,
    uint32_t* __restrict__ bits_out, int32_t* __restrict__ counts) {
  // Rows of up to 256 blocks are sorted; longer rows find the cut key by a
  // bitwise search instead (no sort: 64 reductions over the unsorted keys).
  constexpr bool kSearch = K >= 8;
  __shared__ uint64_t okey[kSearch ? 1 : kWave * K];   // unsorted keys, element j at j
  const int row = blockIdx.x, l = threadIdx.x;
  const double* s = S + (int64_t)row * nkb;

  uint64_t key[K];
  double mass[K];   // softmax mass of block j = l + 64 k (top-p mode)
  if (mode == SA_TOP_P) {
    double mx = -DBL_MAX;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = l + kWave * k;
      mass[k] = j < nkb ? s[j] : -DBL_MAX;
      mx = fmax(mx, mass[k]);
    }
    mx = wave_reduce(mx, [](double a, double b) { return fmax(a, b); });
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = l + kWave * k;
      mass[k] = j < nkb ? exp(mass[k] - mx) : 0.0;
      part += mass[k];
    }
    const double tot = wave_reduce(part, [](double a, double b) { return a + b; });
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = l + kWave * k;
      mass[k] = j < nkb ? mass[k] / tot : 0.0;
      key[k] = j < nkb ? order_key(mass[k]) : 0ull;   // padding sorts last
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = l + kWave * k;
      mass[k] = 0.0;
      key[k] = j < nkb ? order_key(s[j]) : 0ull;
    }
  }

  const int kf = min(top_k, nkb);
  int m;
  uint64_t kc = 0;   // the cut key: that of position m - 1 in descending order
  if constexpr (kSearch) {
    // Top-p: the cut is at the largest key kp whose blocks with keys >= kp
    // hold mass >= p (the mass of the keys above any larger candidate stays
    // below p).  Ties at kp are taken in block-id order until the cumulative
    // mass reaches p.  A total below p through rounding keeps every block.
    bool at_kp = false;
    if (mode == SA_TOP_P && top_p < 1.0) {
      uint64_t kp = 0;
      for (int b = 63; b >= 0; --b) {
        const uint64_t cand = kp | (1ull << b);
        double part = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) part += key[k] >= cand ? mass[k] : 0.0;
        if (wave_reduce(part, [](double a, double b2) { return a + b2; }) >= top_p) kp = cand;
      }
      if (kp == 0) {
        m = nkb;
      } else {
        double part = 0.0;
        int gt = 0, eq = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          part += key[k] > kp ? mass[k] : 0.0;
          gt += __popcll(__ballot(key[k] > kp));
          eq += __popcll(__ballot(key[k] == kp));
        }
        double cs = wave_reduce(part, [](double a, double b2) { return a + b2; });
        const double pk = key_value(kp);
        int r = 1;
        for (cs += pk; r < eq && cs < top_p; ++r) cs += pk;
        m = gt + r;
        at_kp = true;
        kc = kp;
      }
    } else {
      m = mode == SA_TOP_P ? nkb : kf;
    }
    if (mode == SA_TOP_P && m < kf) {
      m = kf;
      at_kp = false;
    }
    if (!at_kp) kc = key_at_rank<K>(key, m);
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) okey[l + kWave * k] = key[k];

    // bitonic sort of the keys into descending order over positions e = l + 64 k
    bitonic<K, 2, 1>(key, l);

    if (mode == SA_TOP_P) {
      if (top_p >= 1.0) {
        m = nkb;
      } else {
        // cumulative mass in sorted order; count the positions still below p
        double carry = 0.0;
        int below = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int e = l + kWave * k;
          const double ms = e < nkb ? key_value(key[k]) : 0.0;
          const double cs = carry + wave_inclusive_scan(ms);
          below += __popcll(__ballot(e < nkb && cs < top_p));
          carry = __shfl(cs, kWave - 1, kWave);
        }
        m = min(nkb, 1 + below);
      }
      m = max(m, kf);
    } else {
      m = kf;
    }
    const int sk = (m - 1) / kWave, sl = (m - 1) % kWave;   // m >= 1
    uint64_t kk = 0;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (k == sk) kk = key[k];
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)kk, sl, kWave);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(kk >> 32), sl, kWave);
    kc = ((uint64_t)hi << 32) | lo;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) key[k] = okey[l + kWave * k];   // back to unsorted
  }

  // The kept set is the first m positions of the (key descending, block id
  // ascending) order: every block whose key exceeds the cut key kc, then the
  // r lowest-id blocks whose key equals it.  Each lane tests its unsorted
  // blocks j = l + 64 k; a ballot over k is mask words 2k, 2k+1.
  uint64_t gt[K], eq[K];
  int above = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = l + kWave * k;
    gt[k] = __ballot(j < nkb && key[k] > kc);
    eq[k] = __ballot(j < nkb && key[k] == kc);
    above += __popcll(gt[k]);
  }
  int r = m - above;   // ties at the cut to keep, lowest ids first
  const uint64_t below_me = (l == 0) ? 0ull : (~0ull >> (kWave - l));
  int c = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const bool tie_kept = ((eq[k] >> l) & 1ull) && __popcll(eq[k] & below_me) < r;
    const uint64_t b = gt[k] | __ballot(tie_kept);
    r -= __popcll(eq[k]);
    if (l == 0) {
      if (2 * k < W) bits_out[(int64_t)row * W + 2 * k] = (uint32_t)b;
      if (2 * k + 1 < W) bits_out[(int64_t)row * W + 2 * k + 1] = (uint32_t)(b >> 32);
    }
    c += __popcll(b);
  }
  // the count is the popcount of the written row, so the CSR built from it
  // always matches the mask
  if (l == 0) counts[row] = c;
}

}  // namespace

hipError_t launch_select(const Dims& g, const double* scores, int mode, double top_p,
                         int top_k, uint32_t* bits, int32_t* counts, hipStream_t s) {
  int n2 = 1;
  while (n2 < g.nkb) n2 <<= 1;
  const size_t lds = (size_t)n2 * (sizeof(double) + sizeof(int)) + (size_t)g.W * sizeof(uint32_t);
  const dim3 grid(g.H * g.nqb);
#define SA_SEL_REG(K)                                                                     \
  hipLaunchKernelGGL(select_reg_kernel<K>, grid, dim3(kWave), 0, s, scores, g.nkb, g.W, mode, \
                     top_p, top_k, bits, counts)
  if (n2 <= 64) {
    SA_SEL_REG(1);
  } else if (n2 <= 128) {
    SA_SEL_REG(2);
  } else if (n2 <= 256) {
    SA_SEL_REG(4);
  } else if (n2 <= 512) {
    SA_SEL_REG(8);
  } else if (n2 <= 1024) {
    SA_SEL_REG(16);
  } else {
    hipLaunchKernelGGL(select_kernel<256>, grid, dim3(256), lds, s, scores, g.nkb, n2, g.W,
                       mode, top_p, top_k, bits, counts);
  }
#undef SA_SEL_REG
  return hipGetLastError();
}

}  // namespace sa
