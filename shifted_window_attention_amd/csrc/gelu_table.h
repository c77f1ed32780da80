// GELU as a table in LDS, shared by the two fused MLP kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace vswin {

// GELU(x) = x Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2, as a piecewise linear
// function in intercept-slope form: kPhiN bins of width h = 2 kPhiX / kPhiN
// = 0.0176 over [-kPhiX, kPhiX), entry k + 1 of bin k holding (c, d) with
// GELU(x) ~ c + d x through the bin's end points, plus entry 0 = (0, 0) for
// x < -kPhiX and entry kPhiN + 1 = (0, 1) for x >= kPhiX, reached by
// clamping the bin index.  Error <= max|GELU''| h^2 / 8 = 0.80 * 3.1e-4 / 8
// < 3.1e-5 inside (GELU'' = phi(x) (2 - x^2)), and |x| (1 - Phi(|x|)) <
// 1.6e-5 outside.  A lookup is one FMA for the index, a clamp, a convert,
// one 8-byte LDS read and one FMA.
constexpr int kPhiN = 512;
constexpr float kPhiX = 4.5f;
constexpr int kGeluEntries = kPhiN + 2;

// the table, built by the nthr threads of a workgroup (a barrier must follow)
__device__ __forceinline__ void gelu_table_build(float2* t, int tid, int nthr) {
  for (int i = tid; i < kGeluEntries; i += nthr) {
    float2 e = make_float2(0.f, i == 0 ? 0.f : 1.f);   // the two tails
    if (i >= 1 && i <= kPhiN) {
      const float h = 2.0f * kPhiX / kPhiN;
      const float x0 = -kPhiX + h * (i - 1), x1 = x0 + h;
      const float g0 = x0 * 0.5f * (1.0f + erff(x0 * 0.70710678118654752f));
      const float g1 = x1 * 0.5f * (1.0f + erff(x1 * 0.70710678118654752f));
      const float d = (g1 - g0) / h;
      e = make_float2(g0 - d * x0, d);
    }
    t[i] = e;
  }
}

__device__ __forceinline__ float gelu_tab(const float2* t, float x) {
  const float uu = __builtin_amdgcn_fmed3f(__builtin_fmaf(x, kPhiN / (2.0f * kPhiX), kPhiN / 2.0f + 1.0f), 0.0f,
                                           (float)kPhiN + 1.5f);
  const float2 e = t[(int)uu];
  return __builtin_fmaf(x, e.y, e.x);
}

// The same function on the scaled coordinate u = 64 x + kGeluU0 (a bin is
// 1/64 wide: kPhiNu = 576 bins over [-4.5, 4.5)), for a caller whose
// matrix product already yields u: the fc1 operand scaled by 64 (a power of
// two, exact in bf16) and its accumulator started at 64 b + kGeluU0.  Entry
// k + 1 of bin k holds (c', d') with GELU ~ c' + d' u, i.e. c' = c - d U0 / 64,
// d' = d / 64 for the bin's line c + d x; entry 0 = (0, 0) below the range,
// entry kPhiNu + 1 = (-U0 / 64, 1 / 64) (GELU = x) above it.  Error <= 0.80 *
// (1/64)^2 / 8 < 2.5e-5 inside, < 1.6e-5 outside.  A lookup is a clamp, a
// convert, one 8-byte LDS read and one FMA.
constexpr int kPhiNu = 576;
constexpr float kGeluU0 = kPhiNu / 2 + 1;
constexpr int kGeluEntriesU = kPhiNu + 2;

__device__ __forceinline__ void gelu_table_build_u(float2* t, int tid, int nthr) {
  for (int i = tid; i < kGeluEntriesU; i += nthr) {
    float2 e = i == 0 ? make_float2(0.f, 0.f) : make_float2(-kGeluU0 / 64.0f, 1.0f / 64.0f);   // the two tails
    if (i >= 1 && i <= kPhiNu) {
      const float h = 1.0f / 64.0f;
      const float x0 = -4.5f + h * (i - 1), x1 = x0 + h;
      const float g0 = x0 * 0.5f * (1.0f + erff(x0 * 0.70710678118654752f));
      const float g1 = x1 * 0.5f * (1.0f + erff(x1 * 0.70710678118654752f));
      const float d = (g1 - g0) / h;
      const float c = g0 - d * x0;
      e = make_float2(c - d * (kGeluU0 / 64.0f), d / 64.0f);
    }
    t[i] = e;
  }
}

__device__ __forceinline__ float gelu_tab_u(const float2* t, float u) {
  const float2 e = t[(int)__builtin_amdgcn_fmed3f(u, 0.0f, (float)kPhiNu + 1.5f)];
  return __builtin_fmaf(u, e.y, e.x);
}

}  // namespace vswin
