// bf16 MFMA building blocks shared by the attention kernels (gfx950, d = 128,
// blocks of 128 rows): buffer descriptors, accumulator -> bf16 fragments,
// direct HBM -> LDS block loads into XOR-swizzled rows, transposing LDS reads.
#pragma once

#include <type_traits>

#include "sa_common.h"

namespace sa {
namespace bf16mma {

constexpr int kD = 128, kB = 128;
constexpr int kTileBytes = kB * kD * 2;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer, 32-bit dword data format (gfx9 CDNA descriptor word 3)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 8 consecutive fp32 accumulator values -> bf16x8 (v_cvt_pk_bf16_f32, RNE)
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& a, int base) {
  f32x8 v;
#pragma unroll
  for (int x = 0; x < 8; ++x) v[x] = a[base + x];
  return __builtin_convertvector(v, bf16x8);
}

// Blocks go from global memory straight into LDS (buffer_load ... lds,
// 16 bytes per lane, no staging registers).  One such load of a wave fills 1 KiB
// of LDS, four 256-byte rows, lane L at byte 16 L; the lane chooses which
// 16-byte chunk of its row it fetches, so each row is stored with its chunks
// permuted (XOR swizzle) and the MFMA operand reads below hit 64 distinct banks:
//   K: logical chunk c of row r sits at chunk c ^ (r & 15)
//   V: logical chunk c of row r sits at chunk c ^ (4 (r & 3))
// A block of 32 KiB is 32 such loads, 8 per wave.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;

__device__ __forceinline__ void dma_block(const uint16_t* src, uint16_t* lds, int wave,
                                          const int (&voff)[4]) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, kTileBytes);
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const int i = 8 * wave + ii;   // rows 4i .. 4i+3
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + i * 512), 16, voff[ii & 3],
                                             i * 1024, 0, 0);
  }
}

// 8 bytes at LDS byte address `addr`, transposed within 16-lane groups
// (ds_read_b64_tr_b16): element e of lane j is element j%4 of what lane
// 4e + j/4 of the group addressed.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* base, int addr) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)(lds_void*)base + addr));
  return __builtin_bit_cast(u32x2, v);
}

// f(integral_constant<int, n>) for n = N .. End - 1, expanded at compile time
template <int N, int End, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N < End) {
    f(std::integral_constant<int, N>{});
    static_for<N + 1, End>(f);
  }
}

}  // namespace bf16mma
}  // namespace sa
