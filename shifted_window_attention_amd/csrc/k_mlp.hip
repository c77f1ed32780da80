// Second half of the Video Swin block (eq. 1): y = z^ + MLP(LN2(z^)),
// MLP = Linear(C, 4C) -> GELU -> Linear(4C, C), fused in one kernel so the
// 4C-wide hidden activations never leave the chip.
//
// One workgroup handles 64 tokens: LN2 of its z^ rows (fp32) into a bf16 LDS
// tile, then for each chunk of 64 hidden units: H = GELU(A W1_c^T + b1_c)
// (MFMA, kept in LDS as bf16) and acc += H W2_c^T (MFMA, fp32 registers);
// finally y = z^ + acc + b2 rounded to bf16.  The next chunk's weights are
// fetched into registers while the current chunk computes.
//
// GELU uses erf from the Abramowitz & Stegun formula 7.1.26 (Hastings'
// approximation, |error| <= 1.5e-7): erf(x) = 1 - (a1 t + ... + a5 t^5)
// exp(-x^2), t = 1 / (1 + p x) for x >= 0, odd extension for x < 0.
#include "vswin_kernels.h"

namespace vswin {

__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, ax, 1.0f));
  float p = 1.061405429f;
  p = __builtin_fmaf(p, t, -1.453152027f);
  p = __builtin_fmaf(p, t, 1.421413741f);
  p = __builtin_fmaf(p, t, -0.284496736f);
  p = __builtin_fmaf(p, t, 0.254829592f);
  p *= t;
  // exp(-x^2) = exp2(-x^2 log2 e)
  const float e = __builtin_amdgcn_exp2f(-(ax * ax) * 1.4426950408889634f);
  const float r = __builtin_fmaf(-p, e, 1.0f);
  return copysignf(r, x);
}

__device__ __forceinline__ float gelu_fast(float x) {
  return 0.5f * x * (1.0f + erf_as7126(x * 0.70710678118654752f));
}

template <int C>
__global__ void __launch_bounds__(256) mlp_fused_kernel(const float* __restrict__ zh, const bf16_t* __restrict__ g2,
                                                        const bf16_t* __restrict__ b2ln, const bf16_t* __restrict__ W1,
                                                        const bf16_t* __restrict__ b1, const bf16_t* __restrict__ W2,
                                                        const bf16_t* __restrict__ bo, bf16_t* __restrict__ y,
                                                        int64_t L, float eps) {
  constexpr int BM = 64, HC = 64, HID = 4 * C, NCH = HID / HC;
  constexpr int LDA = C + 8, LDH = HC + 8;
  constexpr int NT2 = C / 32;            // GEMM2 feature tiles of 16 per wave (C/2 features)
  constexpr int W1CH = HC * C / 8;       // 16-byte chunks of one W1 chunk
  constexpr int W2CH = C * HC / 8;
  constexpr int RW1 = (W1CH + 255) / 256, RW2 = (W2CH + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) bf16_t Hs[BM * LDH];
  __shared__ __attribute__((aligned(16))) bf16_t W1s[HC * LDA];
  __shared__ __attribute__((aligned(16))) bf16_t W2s[C * LDH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, g4 = lane >> 4, fk = g4 * 8;
  const int64_t m0 = (int64_t)blockIdx.x * BM;

  u32x4_t r1[RW1], r2[RW2];
  auto fetch = [&](int hc) {
#pragma unroll
    for (int i = 0; i < RW1; ++i) {
      const int c = tid + 256 * i;
      if (c < W1CH) {
        const int r = c / (C / 8), k = (c % (C / 8)) * 8;
        r1[i] = *reinterpret_cast<const u32x4_t*>(W1 + (int64_t)(hc * HC + r) * C + k);
      }
    }
#pragma unroll
    for (int i = 0; i < RW2; ++i) {
      const int c = tid + 256 * i;
      if (c < W2CH) {
        const int r = c / (HC / 8), k = (c % (HC / 8)) * 8;
        r2[i] = *reinterpret_cast<const u32x4_t*>(W2 + (int64_t)r * HID + hc * HC + k);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < RW1; ++i) {
      const int c = tid + 256 * i;
      if (c < W1CH) {
        const int r = c / (C / 8), k = (c % (C / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(&W1s[r * LDA + k]) = r1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < RW2; ++i) {
      const int c = tid + 256 * i;
      if (c < W2CH) {
        const int r = c / (HC / 8), k = (c % (HC / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(&W2s[r * LDH + k]) = r2[i];
      }
    }
  };

  fetch(0);
  // ---- LN2: 4 lanes per token row, C/4 values each
  {
    constexpr int PER = C / 4;
    const int row = tid >> 2, part = tid & 3;
    const int64_t m = m0 + row;
    float v[PER];
    if (m < L) {
      const float* src = zh + m * C + part * PER;
#pragma unroll
      for (int i = 0; i < PER; i += 4) {
        const float4 t = *reinterpret_cast<const float4*>(src + i);
        v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) v[i] = 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += v[i];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const float mean = s * (1.0f / C);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) { const float dd = v[i] - mean; q += dd * dd; }
    q += __shfl_xor(q, 1);
    q += __shfl_xor(q, 2);
    const float rstd = 1.0f / sqrtf(q * (1.0f / C) + eps);
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      float gg[4], bb[4], o[4];
      load4(g2, part * PER + i, gg);
      load4(b2ln, part * PER + i, bb);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = (v[i + k] - mean) * rstd * gg[k] + bb[k];
      u32x2_t pk;
      pk[0] = pack_bf16x2(o[0], o[1]);
      pk[1] = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<u32x2_t*>(&As[row * LDA + part * PER + i]) = pk;
    }
  }
  stash();
  __syncthreads();

  f32x4_t acc2[2][NT2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT2; ++j) acc2[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int hc = 0; hc < NCH; ++hc) {
    if (hc + 1 < NCH) fetch(hc + 1);
    // GEMM1: wave tile 32 tokens x 32 hidden; D = W1_c rows x A rows^T
    f32x4_t acc1[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc1[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < C; k += 32) {
      bf16x8_t af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 32 + i * 16 + fr) * LDA + k + fk]);
        wf[i] = *reinterpret_cast<const bf16x8_t*>(&W1s[(wn * 32 + i * 16 + fr) * LDA + k + fk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc1[i][j], 0, 0, 0);
    }
    // bias + GELU -> Hs[token][hidden]; lane: token fr, hidden 4*g4 .. +3
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int hcol = wn * 32 + j * 16 + 4 * g4;
        float bb[4] = {0.f, 0.f, 0.f, 0.f}, o[4];
        if (b1) load4(b1, hc * HC + hcol, bb);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = gelu_fast(acc1[i][j][k] + bb[k]);
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[0], o[1]);
        pk[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2_t*>(&Hs[(wm * 32 + i * 16 + fr) * LDH + hcol]) = pk;
      }
    __syncthreads();
    // GEMM2: wave tile 32 tokens x C/2 features; D = W2_c rows x H rows^T
#pragma unroll
    for (int k = 0; k < HC; k += 32) {
      bf16x8_t hf[2], wf[NT2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        hf[i] = *reinterpret_cast<const bf16x8_t*>(&Hs[(wm * 32 + i * 16 + fr) * LDH + k + fk]);
#pragma unroll
      for (int j = 0; j < NT2; ++j)
        wf[j] = *reinterpret_cast<const bf16x8_t*>(&W2s[(wn * (C / 2) + j * 16 + fr) * LDH + k + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT2; ++j)
          acc2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], hf[i], acc2[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (hc + 1 < NCH) {
      stash();
      __syncthreads();
    }
  }
  // ---- y = z^ + acc + b2; lane: token fr, features 4*g4 .. +3 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 32 + i * 16 + fr;
    if (m >= L) continue;
#pragma unroll
    for (int j = 0; j < NT2; ++j) {
      const int n = wn * (C / 2) + j * 16 + 4 * g4;
      float r[4], bb[4], o[4];
      load4(zh, m * C + n, r);
      if (bo) load4(bo, n, bb);
      else bb[0] = bb[1] = bb[2] = bb[3] = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = r[k] + acc2[i][j][k] + bb[k];
      store4(y, m * C + n, o);
    }
  }
}

bool mlp_fused_supported(vswin_dtype dt, int C, int hid) {
  return dt == VSWIN_BF16 && hid == 4 * C && (C == 96 || C == 128);
}

hipError_t mlp_fused(const float* zh, const void* g2, const void* b2ln, const void* W1, const void* b1,
                     const void* W2, const void* bo, void* y, int64_t L, int C, float eps, hipStream_t st) {
  if (L <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((L + 63) / 64);
  if (C == 96)
    hipLaunchKernelGGL(mlp_fused_kernel<96>, dim3(blocks), dim3(256), 0, st, zh, (const bf16_t*)g2,
                       (const bf16_t*)b2ln, (const bf16_t*)W1, (const bf16_t*)b1, (const bf16_t*)W2,
                       (const bf16_t*)bo, (bf16_t*)y, L, eps);
  else if (C == 128)
    hipLaunchKernelGGL(mlp_fused_kernel<128>, dim3(blocks), dim3(256), 0, st, zh, (const bf16_t*)g2,
                       (const bf16_t*)b2ln, (const bf16_t*)W1, (const bf16_t*)b1, (const bf16_t*)W2,
                       (const bf16_t*)bo, (bf16_t*)y, L, eps);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vswin
