// Practical MFMA ceiling: a loop of independent bf16 MFMAs with no memory
// traffic, the measured counterpart of the nominal dense peak that the
// fused kernels are reported against.
#include "mk_params.h"

namespace mk {

// Every wave keeps 8 independent 32x32x16 accumulators busy for `iters`
// rounds (8 MFMAs of 32768 FLOP each per round); one value per workgroup
// goes to sink so the work cannot be dropped.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *sink) {
  typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
  const float s = (float)(threadIdx.x & 7) * 0.125f;
  bf8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(s + (float)i);
    b[i] = (__bf16)(s - (float)i);
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][15];
  if (threadIdx.x == 0) sink[blockIdx.x & 255] = t;
}

hipError_t launch_mfma_loop(int grid, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace mk
