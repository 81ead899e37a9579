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
// query blocks, Y = key blocks) on the fp64 matrix cores.  score_lds_kernel:
// the same scores, bit for bit, for inner 64 or 128 with the operand rows of
// a 64 x 64 block staged in LDS (a quarter of the L2 reads).
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
  // buffer descriptor over the block's valid rows only: rows at or past n read
  // as 0 without a branch, so every load is issued up front
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(x + ((int64_t)h * rows + first) * D), (short)0,
      (int)(n * D * (int)sizeof(T)), 0x00020000);
  const int off = (rl * D + c * EPC) * (int)sizeof(T);
  uint4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it)
    v[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, off, it * RL * D * (int)sizeof(T), 0));
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int it = 0; it < IT; ++it) Elem<T>::add(acc, v[it]);  // rows past n read as +0.0
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

// S[h, i, j] = scale * sum_c X[h, i, c] * Y[h, j, c] in fp64 on the matrix
// cores (v_mfma_f64_16x16x4_f64).  One wave per 16 x 16 output tile, four
// tiles along j per workgroup.  The inner index (padded with zeros to 4*KPL)
// is dealt to the four 16-lane groups in pairs: at steps 2c and 2c+1, lane
// group g supplies indices 8c + 2g and 8c + 2g + 1 of its row of X (A operand,
// row = lane % 16) and of its row of Y (B operand, column = lane % 16), so
// each 16-byte load of a wave covers 64 contiguous bytes of 16 rows.  Output
// element q of lane l is S[4*q + l/16][l % 16] of the tile.  Rows and columns
// past the edge load 0 and are not stored.
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

template <int KPL>  // steps per lane group: inner <= 4 * KPL
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ X,
                                                    const double* __restrict__ Y, int nx,
                                                    int ny, int inner, double scale,
                                                    double* __restrict__ S) {
  static_assert(KPL % 2 == 0, "pairs of doubles per load");
  const int h = blockIdx.z, wv = threadIdx.x / kWave, l = lane_id();
  const int i0 = blockIdx.y * 16, j0 = (blockIdx.x * 4 + wv) * 16;
  if (j0 >= ny) return;  // whole wave; no barriers below
  const int r = l % 16, g = l / 16;
  const int xi = i0 + r, yj = j0 + r;
  const double* xp = X + ((int64_t)h * nx + xi) * inner;
  const double* yp = Y + ((int64_t)h * ny + yj) * inner;
  f64x2 a[KPL / 2], b[KPL / 2];
  if (inner == 4 * KPL) {  // no padding; rows are 16-byte aligned
    const f64x2* xv = reinterpret_cast<const f64x2*>(xp);
    const f64x2* yv = reinterpret_cast<const f64x2*>(yp);
#pragma unroll
    for (int s = 0; s < KPL / 2; ++s) {
      a[s] = xi < nx ? xv[4 * s + g] : f64x2{0.0, 0.0};
      b[s] = yj < ny ? yv[4 * s + g] : f64x2{0.0, 0.0};
    }
  } else {
#pragma unroll
    for (int s = 0; s < KPL / 2; ++s) {
      const int c0 = 8 * s + 2 * g, c1 = c0 + 1;
      a[s].x = (xi < nx && c0 < inner) ? xp[c0] : 0.0;
      a[s].y = (xi < nx && c1 < inner) ? xp[c1] : 0.0;
      b[s].x = (yj < ny && c0 < inner) ? yp[c0] : 0.0;
      b[s].y = (yj < ny && c1 < inner) ? yp[c1] : 0.0;
    }
  }
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < KPL / 2; ++s) {
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s].x, b[s].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s].y, b[s].y, acc, 0, 0, 0);
  }
  const int j = j0 + r;
  if (j < ny) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + 4 * q + g;
      if (i < nx) S[((int64_t)h * nx + i) * ny + j] = scale * acc[q];
    }
  }
}

// The same scores for inner = 64 or 128, a 64 x 64 block of S per workgroup:
// the 64 rows of X and of Y pass through LDS in chunks of 32 inner indices,
// so each is read once per block instead of once per 16 x 16 tile (a quarter
// of the L2 reads).  Wave w owns row tile w and the four column tiles; each
// tile takes exactly the MFMA sequence of score_kernel (steps 2s and 2s+1 on
// inner indices 8s + 2g and 8s + 2g + 1), so the scores are bit-identical.
constexpr int kScoreChunk = 32;                 // inner indices per LDS chunk
constexpr int kScoreRow = kScoreChunk + 2;      // padded LDS row (doubles)

template <int NC>  // chunks: inner = 32 NC
__global__ __launch_bounds__(256) void score_lds_kernel(const double* __restrict__ X,
                                                        const double* __restrict__ Y, int nx,
                                                        int ny, double scale,
                                                        double* __restrict__ S) {
  constexpr int inner = kScoreChunk * NC;
  __shared__ __attribute__((aligned(16))) double xs[64 * kScoreRow];
  __shared__ __attribute__((aligned(16))) double ys[64 * kScoreRow];
  const int h = blockIdx.z, w = threadIdx.x / kWave, l = lane_id();
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int r = l % 16, g = l / 16;
  // staging: thread t copies inner indices 8(t%4) .. +8 of every chunk of row
  // t/4 of X and of Y; all chunks are loaded up front (one load latency)
  const int sr = threadIdx.x / 4, sc = 8 * (threadIdx.x % 4);
  const bool xin = i0 + sr < nx, yin = j0 + sr < ny;
  const double* xp = X + ((int64_t)h * nx + i0 + sr) * inner + sc;
  const double* yp = Y + ((int64_t)h * ny + j0 + sr) * inner + sc;
  f64x2 xr[NC][4], yr[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xr[c][e] = xin ? *reinterpret_cast<const f64x2*>(xp + kScoreChunk * c + 2 * e) : f64x2{0.0, 0.0};
      yr[c][e] = yin ? *reinterpret_cast<const f64x2*>(yp + kScoreChunk * c + 2 * e) : f64x2{0.0, 0.0};
    }
  f64x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c > 0) __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<f64x2*>(xs + sr * kScoreRow + sc + 2 * e) = xr[c][e];
      *reinterpret_cast<f64x2*>(ys + sr * kScoreRow + sc + 2 * e) = yr[c][e];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kScoreChunk / 8; ++s) {
      const f64x2 a = *reinterpret_cast<const f64x2*>(xs + (16 * w + r) * kScoreRow + 8 * s + 2 * g);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const f64x2 b = *reinterpret_cast<const f64x2*>(ys + (16 * ct + r) * kScoreRow + 8 * s + 2 * g);
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a.x, b.x, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a.y, b.y, acc[ct], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int j = j0 + 16 * ct + r;
    if (j >= ny) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + 16 * w + 4 * q + g;
      if (i < nx) S[((int64_t)h * nx + i) * ny + j] = scale * acc[ct][q];
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
  if (inner == 64 || inner == 128) {
    const dim3 grid((g.nkb + 63) / 64, (g.nqb + 63) / 64, g.H);
    if (inner == 64)
      hipLaunchKernelGGL(score_lds_kernel<2>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, scale, scores);
    else
      hipLaunchKernelGGL(score_lds_kernel<4>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, scale, scores);
    return hipGetLastError();
  }
  const dim3 grid((g.nkb + 63) / 64, (g.nqb + 15) / 16, g.H);
  if (inner <= 8) {
    hipLaunchKernelGGL(score_kernel<2>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, inner, scale, scores);
  } else if (inner <= 16) {
    hipLaunchKernelGGL(score_kernel<4>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, inner, scale, scores);
  } else if (inner <= 32) {
    hipLaunchKernelGGL(score_kernel<8>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, inner, scale, scores);
  } else if (inner <= 64) {
    hipLaunchKernelGGL(score_kernel<16>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, inner, scale, scores);
  } else if (inner <= 128) {
    hipLaunchKernelGGL(score_kernel<32>, grid, dim3(256), 0, s, qx, kx, g.nqb, g.nkb, inner, scale, scores);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sa
