// Issue-rate calibration of exp2, the transcendental the softmax runs once
// per logit (the second roof of the attention kernel, beside the matrix
// cores).  Every lane runs kCalibChains independent chains x <- exp2(-x), two
// waves per SIMD when the grid is resident, so that nothing but the issue
// rate of v_exp_f32 (and the clock the device holds while running it) bounds
// the launch.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kCalibBlocks = 2048, kCalibThreads = 256, kCalibChains = 8;

__global__ __launch_bounds__(kCalibThreads) void calib_exp2_kernel(float* __restrict__ out, int iters) {
  float x[kCalibChains];
#pragma unroll
  for (int j = 0; j < kCalibChains; ++j) x[j] = 0.25f + 0.01f * (float)(j + threadIdx.x % 7);
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < kCalibChains; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kCalibChains; ++j) s += x[j];
  out[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = s;
}

hipError_t launch_calib_exp2(float* out, int iters, hipStream_t s) {
  hipLaunchKernelGGL(calib_exp2_kernel, dim3(kCalibBlocks), dim3(kCalibThreads), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace pa
