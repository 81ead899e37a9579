// Matrix-pipe throughput probe (measurement context only; no part of the
// attention path uses it).  Every wave runs `iters` rounds of eight
// independent v_mfma_f32_32x32x16_bf16 on register operands, with no memory
// traffic in the loop, then stores one value per lane so that the work cannot
// be removed.  FLOPs per launch: workgroups * 4 waves * iters * 8 * 32768.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    a[x] = (__bf16)(1.0f / 1024.0f * (float)((lane + x) & 7));
    b[x] = (__bf16)(1.0f / 1024.0f * (float)((lane + 3 * x) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// out: device buffer of workgroups * 256 floats.  Returns 0, or -1 for bad
// arguments, -2 if the launch failed.
extern "C" int sa_probe_mfma_bf16(int workgroups, int iters, float* out, void* stream) {
  if (workgroups < 1 || iters < 1 || !out) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
