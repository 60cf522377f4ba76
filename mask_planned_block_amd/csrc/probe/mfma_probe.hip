// Measurement helper (libmpb_probe.so, not part of the attention path): a
// bf16 MFMA throughput probe for gfx950.
//
// Every wavefront issues `iters` rounds of eight independent
// v_mfma_f32_32x32x16_bf16 (the instruction the attention kernels use) on
// register operands, so the matrix pipe never waits on a dependency or on
// memory.  Timing the launch gives the dense bf16 MFMA rate the chip sustains
// at the clock it runs under this load: the measured counterpart of the
// published peak that the attention roofline is quoted against.
#include <hip/hip_runtime.h>

#include "../../../include/mpb_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.0009765625f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(0.0009765625f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" mpb_status mpb_mfma_probe(int32_t workgroups, int32_t iters, float* out,
                                     void* stream) {
  if (workgroups < 1 || iters < 1 || !out) return MPB_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? MPB_OK : MPB_ERR_DEVICE;
}
