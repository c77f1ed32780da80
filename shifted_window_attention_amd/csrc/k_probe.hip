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

// Whether MFMA and VALU work overlap on a SIMD.  Per round a wave issues 8
// independent v_mfma_f32_16x16x32_bf16 (MFMA part) and/or 8 independent
// chains of v_exp_f32 then v_fma_f32 (VALU part): mode 0 MFMA part only,
// 1 VALU part only, 2 even waves MFMA part / odd waves VALU part, 3 both parts
// in every wave.  Timed by the caller: if the two units ran concurrently,
// mode 3 would take max(t0, t1) and mode 2 half of that; run back to back
// they take t0 + t1 and half of that.
__global__ void __launch_bounds__(512) issue_probe_kernel(float* __restrict__ out, int iters, int mode) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool do_m = mode == 0 || mode == 3 || (mode == 2 && (wave & 1) == 0);
  const bool do_v = mode == 1 || mode == 3 || (mode == 2 && (wave & 1) == 1);
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(i - lane));
  }
  f32x4_t acc[8];
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    v[j] = 1e-3f * (float)(lane + j);
  }
  for (int it = 0; it < iters; ++it) {
    if (do_m) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    if (do_v) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(__builtin_amdgcn_exp2f(v[j]), 0.5f, -0.25f);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][3] + v[j];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = s;
}

hipError_t issue_probe(float* out, int blocks, int iters, int mode, hipStream_t st) {
  issue_probe_kernel<<<dim3((unsigned)blocks), dim3(512), 0, st>>>(out, iters, mode);
  return hipGetLastError();
}

hipError_t mfma_rate(float* out, int blocks, int iters, hipStream_t st) {
  mfma_rate_kernel<<<dim3((unsigned)blocks), dim3(512), 0, st>>>(out, iters);
  return hipGetLastError();
}

}  // namespace vswin
