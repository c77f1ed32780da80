// Measurement helper (not part of the block): a v_mfma_f32_16x16x32_bf16
// throughput kernel, so that MFMA fractions can be quoted against the rate the
// chip sustains as well as against its published peak.  Each wave runs 8
// independent accumulator chains (no MFMA waits on its own previous result
// within 8 issues) for `iters` rounds; every thread writes one float so the
// work is kept.
#include "vswin_kernels.h"

namespace vswin {

__global__ void __launch_bounds__(512) mfma_rate_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(i - lane));
  }
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = s;
}

hipError_t mfma_rate(float* out, int blocks, int iters, hipStream_t st) {
  mfma_rate_kernel<<<dim3((unsigned)blocks), dim3(512), 0, st>>>(out, iters);
  return hipGetLastError();
}

}  // namespace vswin
