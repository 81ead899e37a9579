// Per-head KV demand union and packed gather ("SparSP: Exploiting
// Communication Sparsity for Sequence-Parallel Video DiTs", Abstract:
// demand-directed KV routing moves only the KV blocks some query block
// requests; on one GPU this is the union of the requested blocks and their
// contiguous gather, i.e. the send buffer of that routing).
//
//   mark_kernel  : one workgroup per (head, group of 8 query-block rows);
//                  flags the blocks its CSR entries name in LDS and writes the
//                  group's partial demand words
//   slots_kernel : one workgroup per head; ORs the partial words of every
//                  head up to its own, so the head's first slot is the sum of
//                  the counts of the heads before it; a wave-ballot prefix
//                  over the demand words numbers the head's blocks in
//                  ascending id; writes demand_ptr, demand_idx and the
//                  head's slot map
//   pack_kernel  : grid-stride bitwise copy of the demanded K and V blocks,
//                  16-byte loads all issued before the stores; the same
//                  workgroups then fill col_slot of every CSR entry from the
//                  slot maps
#include <algorithm>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int kMaxKB = 4096;
constexpr int kMarkThreads = 256;
constexpr int kMarkRows = 8;   // query-block rows per mark workgroup

__global__ __launch_bounds__(kMarkThreads) void mark_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int nqb, int nkb,
    int W, int groups, uint32_t* __restrict__ part) {
  __shared__ uint32_t flag[kMaxKB / 4];   // one byte per key block
  const int c = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  uint8_t* f8 = reinterpret_cast<uint8_t*>(flag);
  for (int w = t; w < (nkb + 3) / 4; w += kMarkThreads) flag[w] = 0u;
  __syncthreads();
  const int r0 = h * nqb + c * kMarkRows, r1 = h * nqb + min(nqb, (c + 1) * kMarkRows);
  const int e0 = row_ptr[r0], e1 = row_ptr[r1];
  for (int e = e0 + t; e < e1; e += kMarkThreads) {
    const int j = col_idx[e];
    if ((unsigned)j < (unsigned)nkb) f8[j] = 1;   // ids outside the row are ignored
  }
  __syncthreads();
  for (int w = t; w < W; w += kMarkThreads) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int fw = 8 * w + q;                    // flag word: blocks 4 fw .. 4 fw + 3
      const uint32_t x = (4 * fw < nkb) ? flag[fw] : 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) word |= ((x >> (8 * b)) & 1u) << (4 * q + b);
    }
    part[((int64_t)h * groups + c) * W + w] = word;
  }
}

__global__ __launch_bounds__(1024) void slots_kernel(
    int H, int nkb, int W, int groups, const uint32_t* __restrict__ part, int64_t cap,
    int32_t* __restrict__ demand_ptr, int32_t* __restrict__ demand_idx,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ dev_status) {
  __shared__ uint32_t dem[kMaxKB / 32];
  __shared__ int wbase[kMaxKB / 32 + 1];
  __shared__ int red[1024 / kWave + 1];
  const int h = blockIdx.x, t = threadIdx.x;
  // demand words of heads 0..h; the counts of the heads before h give its base
  int before = 0;
  for (int u = t; u < (h + 1) * W; u += blockDim.x) {
    const int hh = u / W, w = u % W;
    uint32_t word = 0;
    for (int c = 0; c < groups; ++c) word |= part[((int64_t)hh * groups + c) * W + w];
    if (hh < h) before += __popc(word);
    else dem[w] = word;
  }
  const int base = block_reduce(before, red, [](int a, int b) { return a + b; });
  __syncthreads();
  // exclusive prefix of the head's word popcounts (first wave)
  if (t < kWave) {
    int run = 0;
    for (int w0 = 0; w0 < W; w0 += kWave) {
      const int w = w0 + t;
      const int c = (w < W) ? __popc(dem[w]) : 0;
      const int incl = wave_inclusive_scan(c);
      if (w < W) wbase[w] = run + incl - c;
      run += __shfl(incl, kWave - 1, kWave);
    }
    if (t == 0) wbase[W] = run;   // the head's count
  }
  __syncthreads();
  for (int j = t; j < nkb; j += blockDim.x) {
    const uint32_t word = dem[j >> 5];
    const uint32_t bit = 1u << (j & 31);
    int sl = -1;
    if (word & bit) {
      sl = base + wbase[j >> 5] + __popc(word & (bit - 1u));
      demand_idx[sl] = j;
    }
    slot_of[(int64_t)h * nkb + j] = ((int64_t)sl < cap) ? sl : -1;   // -1: not packed
  }
  if (t == 0) {
    demand_ptr[h] = base;
    if (h == H - 1) {
      const int total = base + wbase[W];
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
                                                   int H, int nqb, int nkb,
                                                   const uint8_t* __restrict__ k,
                                                   const uint8_t* __restrict__ v,
                                                   uint8_t* __restrict__ kp,
                                                   uint8_t* __restrict__ vp, int64_t cap,
                                                   const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col_idx,
                                                   const int32_t* __restrict__ slot_of,
                                                   int32_t* __restrict__ col_slot) {
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
  // slot of every CSR entry (-1 where the block did not fit the capacity)
  for (int r = blockIdx.x; r < H * nqb; r += gridDim.x) {
    const int32_t* so = slot_of + (int64_t)(r / nqb) * nkb;
    const int e1 = row_ptr[r + 1];
    for (int e = row_ptr[r] + threadIdx.x; e < e1; e += blockDim.x) {
      const int c = col_idx[e];
      col_slot[e] = ((unsigned)c < (unsigned)nkb) ? so[c] : -1;
    }
  }
}

}  // namespace

int mark_groups(const Dims& g) { return (g.nqb + kMarkRows - 1) / kMarkRows; }

hipError_t launch_demand(const Dims& g, const int32_t* row_ptr, const int32_t* col_idx,
                         uint32_t* part, int32_t* slot_of, int32_t* demand_ptr,
                         int32_t* demand_idx, int64_t cap, int32_t* dev_status, hipStream_t s) {
  const int groups = mark_groups(g);
  hipLaunchKernelGGL(mark_kernel, dim3(groups, g.H), dim3(kMarkThreads), 0, s, row_ptr, col_idx,
                     g.nqb, g.nkb, g.W, groups, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(slots_kernel, dim3(g.H), dim3(1024), 0, s, g.H, g.nkb, g.W, groups, part,
                     cap, demand_ptr, demand_idx, slot_of, dev_status);
  return hipGetLastError();
}

hipError_t launch_pack(const Dims& g, const int32_t* demand_ptr, const int32_t* demand_idx,
                       const void* k, const void* v, void* kp, void* vp, int64_t cap,
                       const int32_t* row_ptr, const int32_t* col_idx, const int32_t* slot_of,
                       int32_t* col_slot, hipStream_t s) {
  const int64_t bytes = (int64_t)g.B * g.d * (g.dtype == SA_BF16 ? 2 : 4);
  const int64_t most = std::min<int64_t>(cap, (int64_t)g.H * g.nkb);
  // enough workgroups for the copies, and at least a few per CU for col_slot
  const int grid = (int)std::min<int64_t>(std::max<int64_t>(2 * most, 1024), 8192);
#define SA_PACK(NB)                                                                         \
  hipLaunchKernelGGL(pack_kernel<NB>, dim3(grid), dim3(256), 0, s, demand_ptr, demand_idx,  \
                     g.H, g.nqb, g.nkb, (const uint8_t*)k, (const uint8_t*)v, (uint8_t*)kp, \
                     (uint8_t*)vp, cap, row_ptr, col_idx, slot_of, col_slot)
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
