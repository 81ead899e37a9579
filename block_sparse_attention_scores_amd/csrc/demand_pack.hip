// Per-head KV demand union and packed gather ("SparSP: Exploiting
// Communication Sparsity for Sequence-Parallel Video DiTs", Abstract:
// demand-directed KV routing moves only the KV blocks some query block
// requests; on one GPU this is the union of the requested blocks and their
// contiguous gather, i.e. the send buffer of that routing).
//
//   mark_kernel  : one workgroup per head; flags every block named by the
//                  head's CSR entries in LDS, writes the head's demand bits
//                  and its demand count
//   slots_kernel : one workgroup per head; the head's first slot is the sum of
//                  the counts of the heads before it; a wave-ballot prefix over
//                  the demand bits numbers the head's blocks in ascending id;
//                  writes demand_ptr, demand_idx and col_slot of every entry
//   pack_kernel  : grid-stride bitwise copy of the demanded K and V blocks,
//                  16-byte loads all issued before the stores
#include <algorithm>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kMaxKB = 4096;

__global__ __launch_bounds__(1024) void mark_kernel(const int32_t* __restrict__ row_ptr,
                                                    const int32_t* __restrict__ col_idx,
                                                    int nqb, int nkb, int W,
                                                    uint32_t* __restrict__ dem_bits,
                                                    int32_t* __restrict__ head_count) {
  __shared__ uint32_t flag[kMaxKB];
  __shared__ int red[1024 / kWave + 1];
  const int h = blockIdx.x, t = threadIdx.x;
  for (int j = t; j < nkb; j += blockDim.x) flag[j] = 0u;
  __syncthreads();
  const int e0 = row_ptr[h * nqb], e1 = row_ptr[(h + 1) * nqb];
  for (int e = e0 + t; e < e1; e += blockDim.x) {
    const int c = col_idx[e];
    if ((unsigned)c < (unsigned)nkb) flag[c] = 1u;   // ids outside the row are ignored
  }
  __syncthreads();
  int c = 0;
  for (int w = t; w < W; w += blockDim.x) {
    uint32_t word = 0;
    for (int b = 0; b < 32 && w * 32 + b < nkb; ++b) word |= flag[w * 32 + b] << b;
    dem_bits[(int64_t)h * W + w] = word;
    c += __popc(word);
  }
  c = block_reduce(c, red, [](int a, int b) { return a + b; });
  if (t == 0) head_count[h] = c;
}

__global__ __launch_bounds__(1024) void slots_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int H, int nqb,
    int nkb, int W, const uint32_t* __restrict__ dem_bits, const int32_t* __restrict__ head_count,
    int64_t cap, int32_t* __restrict__ demand_ptr, int32_t* __restrict__ demand_idx,
    int32_t* __restrict__ col_slot, int32_t* __restrict__ dev_status) {
  __shared__ int slot_of[kMaxKB];
  __shared__ int wbase[kMaxKB / 32];
  __shared__ int red[1024 / kWave + 1];
  const int h = blockIdx.x, t = threadIdx.x;
  int base = 0;
  for (int i = 0; i < h; ++i) base += head_count[i];

  // exclusive prefix of word popcounts (W <= 128 words, first wave)
  if (t < kWave) {
    int run = 0;
    for (int w0 = 0; w0 < W; w0 += kWave) {
      const int w = w0 + t;
      const int c = (w < W) ? __popc(dem_bits[(int64_t)h * W + w]) : 0;
      const int incl = wave_inclusive_scan(c);
      if (w < W) wbase[w] = run + incl - c;
      run += __shfl(incl, kWave - 1, kWave);
    }
  }
  __syncthreads();
  for (int j = t; j < nkb; j += blockDim.x) {
    const uint32_t word = dem_bits[(int64_t)h * W + (j >> 5)];
    const uint32_t bit = 1u << (j & 31);
    int s = -1;
    if (word & bit) {
      s = base + wbase[j >> 5] + __popc(word & (bit - 1u));
      demand_idx[s] = j;
    }
    slot_of[j] = s;
  }
  __syncthreads();
  const int e0 = row_ptr[h * nqb], e1 = row_ptr[(h + 1) * nqb];
  for (int e = e0 + t; e < e1; e += blockDim.x) {
    const int c = col_idx[e];
    const int sl = ((unsigned)c < (unsigned)nkb) ? slot_of[c] : -1;
    col_slot[e] = ((int64_t)sl < cap) ? sl : -1;   // -1: not packed (capacity)
  }
  if (t == 0) {
    demand_ptr[h] = base;
    if (h == H - 1) {
      const int total = base + head_count[h];
      demand_ptr[H] = total;
      dev_status[0] = ((int64_t)total > cap) ? (int32_t)SA_ERR_CAPACITY : 0;
    }
  }
}

// Copies 2 * min(total, cap) blocks (K and V) of B*d elements of `eb` bytes.
// Work unit = one (tensor, slot) block; `kChunks` 16-byte chunks per thread.
template <int kBytesPerBlock>
__global__ __launch_bounds__(256) void pack_kernel(const int32_t* __restrict__ demand_ptr,
                                                   const int32_t* __restrict__ demand_idx,
                                                   int H, int nkb, const uint8_t* __restrict__ k,
                                                   const uint8_t* __restrict__ v,
                                                   uint8_t* __restrict__ kp,
                                                   uint8_t* __restrict__ vp, int64_t cap) {
  constexpr int kChunks = kBytesPerBlock / (16 * 256);
  static_assert(kChunks * 16 * 256 == kBytesPerBlock, "block size");
  const int64_t total = min((int64_t)demand_ptr[H], cap);
  for (int64_t u = blockIdx.x; u < 2 * total; u += gridDim.x) {
    const int64_t slot = u >> 1;
    const bool is_v = u & 1;
    // head of this slot: last h with demand_ptr[h] <= slot
    int lo = 0, hi = H - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)demand_ptr[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    const int j = demand_idx[slot];
    const uint8_t* src = (is_v ? v : k) + ((int64_t)lo * nkb + j) * kBytesPerBlock;
    uint8_t* dst = (is_v ? vp : kp) + slot * kBytesPerBlock;
    uint4 r[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      r[c] = *reinterpret_cast<const uint4*>(src + (int64_t)(c * 256 + threadIdx.x) * 16);
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      *reinterpret_cast<uint4*>(dst + (int64_t)(c * 256 + threadIdx.x) * 16) = r[c];
  }
}

}  // namespace

hipError_t launch_demand(const Dims& g, const int32_t* row_ptr, const int32_t* col_idx,
                         uint32_t* dem_bits, int32_t* head_count, int32_t* demand_ptr,
                         int32_t* demand_idx, int32_t* col_slot, int64_t cap,
                         int32_t* dev_status, hipStream_t s) {
  hipLaunchKernelGGL(mark_kernel, dim3(g.H), dim3(1024), 0, s, row_ptr, col_idx, g.nqb, g.nkb,
                     g.W, dem_bits, head_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(slots_kernel, dim3(g.H), dim3(1024), 0, s, row_ptr, col_idx, g.H, g.nqb,
                     g.nkb, g.W, dem_bits, head_count, cap, demand_ptr, demand_idx, col_slot,
                     dev_status);
  return hipGetLastError();
}

hipError_t launch_pack(const Dims& g, const int32_t* demand_ptr, const int32_t* demand_idx,
                       const void* k, const void* v, void* kp, void* vp, int64_t cap,
                       hipStream_t s) {
  const int64_t bytes = (int64_t)g.B * g.d * (g.dtype == SA_BF16 ? 2 : 4);
  const int64_t most = std::min<int64_t>(cap, (int64_t)g.H * g.nkb);
  if (most <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(2 * most, 8192);
#define SA_PACK(NB)                                                                        \
  hipLaunchKernelGGL(pack_kernel<NB>, dim3(grid), dim3(256), 0, s, demand_ptr, demand_idx, \
                     g.H, g.nkb, (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)kp,       \
                     (uint8_t*)vp, cap)
  switch (bytes) {
    case 8192: SA_PACK(8192); break;     // 64 x 64 bf16
    case 16384: SA_PACK(16384); break;   // 64 x 128 bf16, 64 x 64 fp32
    case 32768: SA_PACK(32768); break;   // 128 x 128 bf16, 64 x 128 fp32
    case 65536: SA_PACK(65536); break;   // 128 x 128 fp32
    default: return hipErrorInvalidValue;
  }
#undef SA_PACK
  return hipGetLastError();
}

}  // namespace sa
