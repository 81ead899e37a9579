// CSR block lists of a bit-packed block mask (the materialised mask of the
// Top-p sparse-attention abstract, mlsift listing, tag "sequence
// parallelism").  Rows are (head, query block) head-major; the columns of a
// row are its selected key blocks in ascending order.
//
//   count_kernel   : popcount of each mask row (only for an external mask;
//                    the selector writes the counts itself)
//   scan_kernel    : one workgroup, exclusive scan of the counts -> row_ptr
//   compact_kernel : one wave per row; word popcounts are prefix-summed across
//                    the wave and each lane expands its word's set bits into
//                    ascending column ids
#include "sa_common.h"

namespace sa {
namespace {

__device__ __forceinline__ uint32_t word_mask(int w, int nkb) {
  const int lo = w * 32;
  if (lo + 32 <= nkb) return 0xffffffffu;
  const int n = nkb - lo;
  return n <= 0 ? 0u : ((1u << n) - 1u);
}

__global__ __launch_bounds__(256) void count_kernel(const uint32_t* __restrict__ bits, int rows,
                                                    int nkb, int W, int32_t* __restrict__ counts) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= rows) return;
  int c = 0;
  for (int w = lane_id(); w < W; w += kWave)
    c += __popc(bits[(int64_t)row * W + w] & word_mask(w, nkb));
  c = wave_reduce(c, [](int a, int b) { return a + b; });
  if (lane_id() == 0) counts[row] = c;
}

constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ counts,
                                                            int rows, int32_t* __restrict__ row_ptr) {
  __shared__ int red[kScanThreads / kWave + 1];
  const int t = threadIdx.x;
  const int per = (rows + kScanThreads - 1) / kScanThreads;
  const int lo = min(rows, t * per), hi = min(rows, lo + per);
  int local = 0;
  for (int r = lo; r < hi; ++r) local += counts[r];
  int total;
  int run = block_inclusive_scan(local, red, &total) - local;
  for (int r = lo; r < hi; ++r) {
    row_ptr[r] = run;
    run += counts[r];
  }
  if (t == 0) row_ptr[rows] = total;
}

__global__ __launch_bounds__(256) void compact_kernel(const uint32_t* __restrict__ bits, int rows,
                                                      int nkb, int W,
                                                      const int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= rows) return;
  const int l = lane_id();
  int base = row_ptr[row];
  for (int w0 = 0; w0 < W; w0 += kWave) {
    const int w = w0 + l;
    uint32_t word = (w < W) ? (bits[(int64_t)row * W + w] & word_mask(w, nkb)) : 0u;
    const int c = __popc(word);
    const int incl = wave_inclusive_scan(c);
    int pos = base + incl - c;
    while (word) {
      const int b = __ffs(word) - 1;
      col_idx[pos++] = w * 32 + b;
      word &= word - 1u;
    }
    base += __shfl(incl, kWave - 1, kWave);
  }
}

}  // namespace

hipError_t launch_count_bits(const Dims& g, const uint32_t* bits, int32_t* counts,
                             hipStream_t s) {
  const int rows = g.H * g.nqb;
  hipLaunchKernelGGL(count_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, bits, rows, g.nkb,
                     g.W, counts);
  return hipGetLastError();
}

hipError_t launch_csr(const Dims& g, const uint32_t* bits, const int32_t* counts,
                      int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
  const int rows = g.H * g.nqb;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, rows, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, bits, rows, g.nkb,
                     g.W, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace sa
