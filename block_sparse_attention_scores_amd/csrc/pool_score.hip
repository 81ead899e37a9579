// Block pooling (mean of the valid rows of every query and key block) and the
// block-score matrix, the cheap surrogate that ranks key blocks for each query
// block ("Dynamic Sparsity in Large-Scale Video DiT Training", section "The
// idea": a cheap surrogate instead of the full scores; a per-head low-rank
// predictor of inner dimension sixteen).
//
// pool_kernel: HBM-bound streaming read of Q and K in one launch.  One
// workgroup per (block, head); every thread issues all of its 16-byte loads
// before accumulating, sums in fp64, and the per-row-lane partial sums are
// combined in LDS in a fixed order (deterministic).  With the low-rank
// predictor the workgroup also projects its mean through W (fp64).
//
// score_kernel: S = scale * X Y^T per head in fp64 (X = pooled or projected
// query blocks, Y = key blocks), 64x64 tiles staged through LDS.
#include "sa_common.h"

namespace sa {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static void add(double* acc, const uint4& v) {
    acc[0] += (double)__uint_as_float(v.x);
    acc[1] += (double)__uint_as_float(v.y);
    acc[2] += (double)__uint_as_float(v.z);
    acc[3] += (double)__uint_as_float(v.w);
  }
};
template <>
struct Elem<uint16_t> {  // bf16 storage
  static constexpr int kPerChunk = 8;
  __device__ static void add(double* acc, const uint4& v) {
    acc[0] += (double)bf16_lo(v.x);
    acc[1] += (double)bf16_hi(v.x);
    acc[2] += (double)bf16_lo(v.y);
    acc[3] += (double)bf16_hi(v.y);
    acc[4] += (double)bf16_lo(v.z);
    acc[5] += (double)bf16_hi(v.z);
    acc[6] += (double)bf16_lo(v.w);
    acc[7] += (double)bf16_hi(v.w);
  }
};

constexpr int kPoolThreads = 256;

template <typename T, int D, int BLK>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int nqb, int nkb, int64_t q_rows,
    int64_t q_valid, int64_t kv_rows, int64_t kv_valid, const float* __restrict__ wq,
    const float* __restrict__ wk, int rank, double* __restrict__ qbar,
    double* __restrict__ kbar, double* __restrict__ qt, double* __restrict__ kt) {
  constexpr int EPC = Elem<T>::kPerChunk;      // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                 // chunks per row
  constexpr int RL = kPoolThreads / CPR;       // row lanes
  constexpr int IT = BLK / RL;                 // rows per row lane
  static_assert(kPoolThreads % CPR == 0 && BLK % RL == 0, "pool tiling");
  __shared__ double part[RL * D];
  __shared__ double mean[D];

  const int h = blockIdx.y;
  const bool is_q = (int)blockIdx.x < nqb;
  const int blk = is_q ? blockIdx.x : blockIdx.x - nqb;
  const T* x = is_q ? q : k;
  const int64_t rows = is_q ? q_rows : kv_rows;
  const int64_t valid = is_q ? q_valid : kv_valid;
  const int64_t first = (int64_t)blk * BLK;
  const int n = (int)min((int64_t)BLK, valid - first);

  const int t = threadIdx.x, c = t % CPR, rl = t / CPR;
  const T* base = x + ((int64_t)h * rows + first) * D + c * EPC;
  uint4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = rl + it * RL;
    v[it] = (r < n) ? *reinterpret_cast<const uint4*>(base + (int64_t)r * D) : make_uint4(0, 0, 0, 0);
  }
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int it = 0; it < IT; ++it) Elem<T>::add(acc, v[it]);  // padded loads are +0.0
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[rl * D + c * EPC + e] = acc[e];
  __syncthreads();

  const int nb = is_q ? nqb : nkb;
  double* out = is_q ? qbar : kbar;
  if (t < D) {
    double s = 0.0;
    for (int r = 0; r < RL; ++r) s += part[r * D + t];
    const double m = s / (double)n;
    out[((int64_t)h * nb + blk) * D + t] = m;
    mean[t] = m;
  }
  if (rank > 0) {
    __syncthreads();
    if (t < rank) {
      const float* w = (is_q ? wq : wk) + (int64_t)h * D * rank;
      double s = 0.0;
      for (int cc = 0; cc < D; ++cc) s += mean[cc] * (double)w[cc * rank + t];
      (is_q ? qt : kt)[((int64_t)h * nb + blk) * rank + t] = s;
    }
  }
}

// S[h, i, j] = scale * sum_c X[h, i, c] * Y[h, j, c]  (fp64, c ascending)
constexpr int kTile = 64, kKc = 16;
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ X,
                                                    const double* __restrict__ Y, int nx,
                                                    int ny, int inner, double scale,
                                                    double* __restrict__ S) {
  __shared__ double xs[kTile][kKc + 1];
  __shared__ double ys[kTile][kKc + 1];
  const int h = blockIdx.z;
  const int i0 = blockIdx.y * kTile, j0 = blockIdx.x * kTile;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  const double* xh = X + (int64_t)h * nx * inner;
  const double* yh = Y + (int64_t)h * ny * inner;
  double acc[4][4] = {};
  for (int c0 = 0; c0 < inner; c0 += kKc) {
    for (int e = t; e < kTile * kKc; e += 256) {
      const int r = e / kKc, cc = e % kKc;
      const bool okc = c0 + cc < inner;
      xs[r][cc] = (i0 + r < nx && okc) ? xh[(int64_t)(i0 + r) * inner + c0 + cc] : 0.0;
      ys[r][cc] = (j0 + r < ny && okc) ? yh[(int64_t)(j0 + r) * inner + c0 + cc] : 0.0;
    }
    __syncthreads();
    const int kc = min(kKc, inner - c0);
    for (int cc = 0; cc < kc; ++cc) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = xs[ty * 4 + u][cc];
        b[u] = ys[tx * 4 + u][cc];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma(a[u], b[w], acc[u][w]);
    }
    __syncthreads();
  }
  double* sh = S + (int64_t)h * nx * ny;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty * 4 + u;
    if (i >= nx) continue;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = j0 + tx * 4 + w;
      if (j < ny) sh[(int64_t)i * ny + j] = scale * acc[u][w];
    }
  }
}

template <typename T, int D, int BLK>
hipError_t pool_launch(const Dims& g, const void* q, const void* k, const float* wq,
                       const float* wk, double* qbar, double* kbar, double* qt, double* kt,
                       hipStream_t s) {
  dim3 grid(g.nqb + g.nkb, g.H);
  hipLaunchKernelGGL((pool_kernel<T, D, BLK>), grid, dim3(kPoolThreads), 0, s,
                     (const T*)q, (const T*)k, g.nqb, g.nkb, g.q_rows, g.q_valid, g.kv_rows,
                     g.kv_valid, wq, wk, g.rank, qbar, kbar, qt, kt);
  return hipGetLastError();
}

template <typename T>
hipError_t pool_dispatch(const Dims& g, const void* q, const void* k, const float* wq,
                         const float* wk, double* qbar, double* kbar, double* qt, double* kt,
                         hipStream_t s) {
  if (g.d == 128 && g.B == 128) return pool_launch<T, 128, 128>(g, q, k, wq, wk, qbar, kbar, qt, kt, s);
  if (g.d == 128 && g.B == 64) return pool_launch<T, 128, 64>(g, q, k, wq, wk, qbar, kbar, qt, kt, s);
  if (g.d == 64 && g.B == 128) return pool_launch<T, 64, 128>(g, q, k, wq, wk, qbar, kbar, qt, kt, s);
  if (g.d == 64 && g.B == 64) return pool_launch<T, 64, 64>(g, q, k, wq, wk, qbar, kbar, qt, kt, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pool(const Dims& g, const void* q, const void* k, const float* wq,
                       const float* wk, double* qbar, double* kbar, double* qt, double* kt,
                       hipStream_t s) {
  if (g.dtype == SA_BF16) return pool_dispatch<uint16_t>(g, q, k, wq, wk, qbar, kbar, qt, kt, s);
  return pool_dispatch<float>(g, q, k, wq, wk, qbar, kbar, qt, kt, s);
}

hipError_t launch_scores(const Dims& g, const double* qx, const double* kx, int inner,
                         double scale, double* scores, hipStream_t s) {
  dim3 grid((g.nkb + kTile - 1) / kTile, (g.nqb + kTile - 1) / kTile, g.H);
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, inner, scale,
                     scores);
  return hipGetLastError();
}

}  // namespace sa
