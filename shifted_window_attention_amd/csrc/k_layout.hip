// Permutation and normalisation kernels of the Video Swin block:
//   * LayerNorm over C fused with the pad + roll + partition gather (the
//     LN -> pad -> roll -> window_partition order of the mmaction2 block);
//   * plain LayerNorm over rows (LN2, patch-merge LN, final LN);
//   * the inverse scatter (reverse partition + roll back + crop, optional
//     residual) and the index-map export.
// All are HBM-bound: one read and one write per element.  Rows are handled
// by LPR lanes each (16 lanes for C <= 192, a whole wave above), channel
// pairs are loaded as 4-byte (bf16) or 8-byte (fp32) vectors.
#include "vswin_kernels.h"

namespace vswin {

template <typename T> struct Pair;
template <> struct Pair<float> {
  __device__ __forceinline__ static void load(const float* p, int64_t i, float& a, float& b) {
    const float2 t = *reinterpret_cast<const float2*>(p + i); a = t.x; b = t.y;
  }
  __device__ __forceinline__ static void store(float* p, int64_t i, float a, float b) {
    *reinterpret_cast<float2*>(p + i) = make_float2(a, b);
  }
};
template <> struct Pair<bf16_t> {
  __device__ __forceinline__ static void load(const bf16_t* p, int64_t i, float& a, float& b) {
    const uint32_t t = *reinterpret_cast<const uint32_t*>(p + i); a = bflo(t); b = bfhi(t);
  }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float a, float b) {
    *reinterpret_cast<uint32_t*>(p + i) = pack_bf16x2(a, b);
  }
};

// rows: output rows.  gather: output row = window slot, input row = its source
// token (zeros for pad slots).  apply_ln = 0 turns it into a plain gather.
template <typename TIN, typename TOUT, int LPR, int KP>
__global__ void __launch_bounds__(256) ln_rows_kernel(const TIN* __restrict__ x, const TOUT* __restrict__ g,
                                                      const TOUT* __restrict__ b, TOUT* __restrict__ y,
                                                      int64_t rows, int C, float eps, int gather,
                                                      WinGeo geo, int apply_ln) {
  warm_args(x, g, b, y, rows, C, eps, gather, geo, apply_ln);
  const int li = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= rows) return;
  int64_t src = row;
  if (gather) {
    int lab;
    const int r = (int)row;
    const int w = r / geo.N;
    src = slot_source(geo, w, r - w * geo.N, lab);
  }
  const int npairs = C >> 1;
  TOUT* yr = y + row * C;
  if (src < 0) {
    for (int k = 0; k < KP; ++k) {
      const int p = li + k * LPR;
      if (p < npairs) Pair<TOUT>::store(yr, 2 * p, 0.f, 0.f);
    }
    return;
  }
  const TIN* xr = x + src * C;
  float v[2 * KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int p = li + k * LPR;
    if (p < npairs) Pair<TIN>::load(xr, 2 * p, v[2 * k], v[2 * k + 1]);
    else { v[2 * k] = 0.f; v[2 * k + 1] = 0.f; }
  }
  if (!apply_ln) {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int p = li + k * LPR;
      if (p < npairs) Pair<TOUT>::store(yr, 2 * p, v[2 * k], v[2 * k + 1]);
    }
    return;
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 2 * KP; ++k) s += v[k];
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, LPR);
  const float mean = s / (float)C;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int p = li + k * LPR;
    if (p < npairs) {
      const float d0 = v[2 * k] - mean, d1 = v[2 * k + 1] - mean;
      q += d0 * d0 + d1 * d1;
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) q += __shfl_xor(q, m, LPR);
  const float rstd = 1.0f / sqrtf(q / (float)C + eps);
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int p = li + k * LPR;
    if (p < npairs) {
      float g0, g1, b0, b1;
      Pair<TOUT>::load(g, 2 * p, g0, g1);
      Pair<TOUT>::load(b, 2 * p, b0, b1);
      Pair<TOUT>::store(yr, 2 * p, (v[2 * k] - mean) * rstd * g0 + b0,
                        (v[2 * k + 1] - mean) * rstd * g1 + b1);
    }
  }
}

// ---------------------------------------------------------------------------
// 16-byte vector variants (C % 8 == 0): LPR lanes per row, each carrying KC
// chunks of 8 channels (chunks li, li + LPR, ...), so every access is a 16-byte
// (bf16) or two 16-byte (fp32) vectors and a wave covers 64 / LPR rows.
// ---------------------------------------------------------------------------
template <typename T> struct Vec8;
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, int64_t i, float v[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p + i), b = *reinterpret_cast<const float4*>(p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, int64_t i, const float v[8]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct Vec8<bf16_t> {
  __device__ __forceinline__ static void load(const bf16_t* p, int64_t i, float v[8]) {
    const u32x4_t t = *reinterpret_cast<const u32x4_t*>(p + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[2 * e] = bflo(t[e]); v[2 * e + 1] = bfhi(t[e]); }
  }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, const float v[8]) {
    u32x4_t t;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<u32x4_t*>(p + i) = t;
  }
};

template <typename TIN, typename TOUT, int LPR, int KC>
__global__ void __launch_bounds__(256) ln_rows_v8_kernel(const TIN* __restrict__ x, const TOUT* __restrict__ g,
                                                         const TOUT* __restrict__ b, TOUT* __restrict__ y,
                                                         int64_t rows, int C, float eps, int gather,
                                                         WinGeo geo, int apply_ln) {
  warm_args(x, g, b, y, rows, C, eps, gather, geo, apply_ln);
  const int li = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= rows) return;
  int64_t src = row;
  if (gather) {
    int lab;
    src = row_source(geo, (int)row, lab);
  }
  TOUT* yr = y + row * C;
  float v[KC][8];
  if (src < 0) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k][e] = 0.f;
      Vec8<TOUT>::store(yr, 8 * (li + k * LPR), v[k]);
    }
    return;
  }
  const TIN* xr = x + src * C;
#pragma unroll
  for (int k = 0; k < KC; ++k) Vec8<TIN>::load(xr, 8 * (li + k * LPR), v[k]);
  if (apply_ln) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[k][e];
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, LPR);
    const float mean = s / (float)C;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < KC; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[k][e] - mean;
        q += d * d;
      }
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) q += __shfl_xor(q, m, LPR);
    const float rstd = 1.0f / sqrtf(q / (float)C + eps);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float gg[8], bb[8];
      Vec8<TOUT>::load(g, 8 * (li + k * LPR), gg);
      Vec8<TOUT>::load(b, 8 * (li + k * LPR), bb);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k][e] = (v[k][e] - mean) * rstd * gg[e] + bb[e];
    }
  }
#pragma unroll
  for (int k = 0; k < KC; ++k) Vec8<TOUT>::store(yr, 8 * (li + k * LPR), v[k]);
}

// (LPR, KC) for C = 8 * LPR * KC with LPR a power of two <= 64, KC <= 8;
// false when C has no such split (the 4-byte kernels serve it)
static bool v8_split(int C, int& lpr, int& kc) {
  if (C % 8) return false;
  const int ch = C / 8;
  for (int k = 1; k <= 8; ++k) {
    if (ch % k) continue;
    const int l = ch / k;
    if (l <= 64 && (l & (l - 1)) == 0 && (l >= 4 || k == ch)) {
      lpr = l;
      kc = k;
      return true;
    }
  }
  return false;
}

template <typename TIN, typename TOUT, int LPR, int KC>
static void launch_ln_v8(const TIN* x, const TOUT* g, const TOUT* b, TOUT* y, int64_t rows, int C, float eps,
                         int gather, const WinGeo& geo, int apply_ln, hipStream_t st) {
  const int64_t blocks = (rows + (256 / LPR) - 1) / (256 / LPR);
  hipLaunchKernelGGL((ln_rows_v8_kernel<TIN, TOUT, LPR, KC>), dim3((unsigned)blocks), dim3(256), 0, st, x, g, b,
                     y, rows, C, eps, gather, geo, apply_ln);
}

template <typename TIN, typename TOUT>
static bool try_ln_v8(const TIN* x, const TOUT* g, const TOUT* b, TOUT* y, int64_t rows, int C, float eps,
                      int gather, const WinGeo& geo, int apply_ln, hipStream_t st) {
  int lpr, kc;
  if (!v8_split(C, lpr, kc)) return false;
#define VSWIN_V8(L, K)                                                       \
  if (lpr == L && kc == K) {                                                 \
    launch_ln_v8<TIN, TOUT, L, K>(x, g, b, y, rows, C, eps, gather, geo, apply_ln, st); \
    return true;                                                             \
  }
  VSWIN_V8(4, 1) VSWIN_V8(8, 1) VSWIN_V8(16, 1) VSWIN_V8(32, 1) VSWIN_V8(64, 1)
  VSWIN_V8(4, 3) VSWIN_V8(8, 3) VSWIN_V8(16, 3) VSWIN_V8(32, 3) VSWIN_V8(64, 3)
  VSWIN_V8(64, 2) VSWIN_V8(64, 4) VSWIN_V8(64, 6) VSWIN_V8(64, 8)
#undef VSWIN_V8
  return false;
}

template <typename TIN, typename TOUT, int LPR, int KP>
static void launch_ln_kp(const TIN* x, const TOUT* g, const TOUT* b, TOUT* y, int64_t rows, int C, float eps,
                         int gather, const WinGeo& geo, int apply_ln, hipStream_t st) {
  const int64_t blocks = (rows + (256 / LPR) - 1) / (256 / LPR);
  hipLaunchKernelGGL((ln_rows_kernel<TIN, TOUT, LPR, KP>), dim3((unsigned)blocks), dim3(256), 0, st, x, g, b, y,
                     rows, C, eps, gather, geo, apply_ln);
}

// Pairs per lane are a template constant so that each lane holds only the
// values of its own row slice in registers.
template <typename TIN, typename TOUT>
static hipError_t launch_ln(const TIN* x, const TOUT* g, const TOUT* b, TOUT* y, int64_t rows, int C,
                            float eps, int gather, const WinGeo& geo, int apply_ln, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (try_ln_v8<TIN, TOUT>(x, g, b, y, rows, C, eps, gather, geo, apply_ln, st)) return hipGetLastError();
  const int npairs = C / 2;
#define VSWIN_LN(LPR, KP) \
  launch_ln_kp<TIN, TOUT, LPR, KP>(x, g, b, y, rows, C, eps, gather, geo, apply_ln, st)
  if (npairs <= 96) {                // C <= 192: 16 lanes per row, <= 6 pairs per lane
    const int kp = (npairs + 15) / 16;
    if (kp <= 1) VSWIN_LN(16, 1);
    else if (kp <= 2) VSWIN_LN(16, 2);
    else if (kp <= 3) VSWIN_LN(16, 3);
    else if (kp <= 4) VSWIN_LN(16, 4);
    else VSWIN_LN(16, 6);
  } else {                           // C <= 4096: a wave per row
    const int kp = (npairs + 63) / 64;
    if (kp <= 2) VSWIN_LN(64, 2);
    else if (kp <= 3) VSWIN_LN(64, 3);
    else if (kp <= 4) VSWIN_LN(64, 4);
    else if (kp <= 6) VSWIN_LN(64, 6);
    else if (kp <= 8) VSWIN_LN(64, 8);
    else if (kp <= 12) VSWIN_LN(64, 12);
    else if (kp <= 16) VSWIN_LN(64, 16);
    else VSWIN_LN(64, 32);
  }
#undef VSWIN_LN
  return hipGetLastError();
}

hipError_t ln_gather(vswin_dtype dt, const void* x, const void* g, const void* b, void* y, int64_t slots,
                     int C, float eps, const WinGeo& geo, int apply_ln, hipStream_t st) {
  if (dt == VSWIN_BF16)
    return launch_ln<bf16_t, bf16_t>((const bf16_t*)x, (const bf16_t*)g, (const bf16_t*)b, (bf16_t*)y,
                                     slots, C, eps, 1, geo, apply_ln, st);
  return launch_ln<float, float>((const float*)x, (const float*)g, (const float*)b, (float*)y, slots, C,
                                 eps, 1, geo, apply_ln, st);
}

hipError_t ln_rows(vswin_dtype in_dt, vswin_dtype out_dt, const void* x, const void* g, const void* b,
                   void* y, int64_t rows, int C, float eps, hipStream_t st) {
  WinGeo geo{};
  if (in_dt == VSWIN_FP32 && out_dt == VSWIN_BF16)
    return launch_ln<float, bf16_t>((const float*)x, (const bf16_t*)g, (const bf16_t*)b, (bf16_t*)y, rows,
                                    C, eps, 0, geo, 1, st);
  if (in_dt == VSWIN_FP32 && out_dt == VSWIN_FP32)
    return launch_ln<float, float>((const float*)x, (const float*)g, (const float*)b, (float*)y, rows, C,
                                   eps, 0, geo, 1, st);
  if (in_dt == VSWIN_BF16 && out_dt == VSWIN_BF16)
    return launch_ln<bf16_t, bf16_t>((const bf16_t*)x, (const bf16_t*)g, (const bf16_t*)b, (bf16_t*)y,
                                     rows, C, eps, 0, geo, 1, st);
  return launch_ln<bf16_t, float>((const bf16_t*)x, (const float*)g, (const float*)b, (float*)y, rows, C,
                                  eps, 0, geo, 1, st);
}

// ---------------------------------------------------------------------------
// inverse scatter: y[src] = windows[slot] (+ residual[src]); pads dropped.
// One thread per (slot, group of 4 channels).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) reverse_kernel(const T* __restrict__ win, const T* __restrict__ res,
                                                      T* __restrict__ y, int64_t slots, int C, WinGeo geo) {
  warm_args(win, res, y, slots, C, geo);
  const int c4 = C >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= slots * c4) return;
  const int64_t s = i / c4;
  const int c = (int)(i - s * c4) * 4;
  int lab;
  const int w = (int)s / geo.N;
  const int64_t src = slot_source(geo, w, (int)s - w * geo.N, lab);
  if (src < 0) return;
  float v[4];
  load4(win, s * C + c, v);
  if (res) {
    float r[4];
    load4(res, src * C + c, r);
    for (int k = 0; k < 4; ++k) v[k] += r[k];
  }
  store4(y, src * C + c, v);
}

// 16-byte variant: LPR lanes per slot row, KC chunks of 8 channels per lane
template <typename T, int LPR, int KC>
__global__ void __launch_bounds__(256) reverse_v8_kernel(const T* __restrict__ win, const T* __restrict__ res,
                                                         T* __restrict__ y, int64_t slots, int C, WinGeo geo) {
  warm_args(win, res, y, slots, C, geo);
  const int li = threadIdx.x % LPR;
  const int64_t s = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (s >= slots) return;
  int lab;
  const int64_t src = row_source(geo, (int)s, lab);
  if (src < 0) return;
  float v[KC][8];
#pragma unroll
  for (int k = 0; k < KC; ++k) Vec8<T>::load(win, s * C + 8 * (li + k * LPR), v[k]);
  if (res) {
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float r[8];
      Vec8<T>::load(res, src * C + 8 * (li + k * LPR), r);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k][e] += r[e];
    }
  }
#pragma unroll
  for (int k = 0; k < KC; ++k) Vec8<T>::store(y, src * C + 8 * (li + k * LPR), v[k]);
}

template <typename T>
static bool try_reverse_v8(const T* win, const T* res, T* y, int64_t slots, int C, const WinGeo& geo,
                           hipStream_t st) {
  int lpr, kc;
  if (!v8_split(C, lpr, kc)) return false;
#define VSWIN_V8(L, K)                                                                              \
  if (lpr == L && kc == K) {                                                                        \
    hipLaunchKernelGGL((reverse_v8_kernel<T, L, K>), dim3((unsigned)((slots + (256 / L) - 1) / (256 / L))), \
                       dim3(256), 0, st, win, res, y, slots, C, geo);                               \
    return true;                                                                                    \
  }
  VSWIN_V8(4, 1) VSWIN_V8(8, 1) VSWIN_V8(16, 1) VSWIN_V8(32, 1) VSWIN_V8(64, 1)
  VSWIN_V8(4, 3) VSWIN_V8(8, 3) VSWIN_V8(16, 3) VSWIN_V8(32, 3) VSWIN_V8(64, 3)
  VSWIN_V8(64, 2) VSWIN_V8(64, 4) VSWIN_V8(64, 6) VSWIN_V8(64, 8)
#undef VSWIN_V8
  return false;
}

hipError_t reverse_scatter(vswin_dtype dt, const void* win, const void* res, void* y, int64_t slots, int C,
                           const WinGeo& geo, hipStream_t st) {
  const int64_t n = slots * (C / 4);
  if (n <= 0) return hipSuccess;
  if (dt == VSWIN_BF16 ? try_reverse_v8<bf16_t>((const bf16_t*)win, (const bf16_t*)res, (bf16_t*)y, slots, C, geo, st)
                       : try_reverse_v8<float>((const float*)win, (const float*)res, (float*)y, slots, C, geo, st))
    return hipGetLastError();
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (dt == VSWIN_BF16)
    hipLaunchKernelGGL(reverse_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)win,
                       (const bf16_t*)res, (bf16_t*)y, slots, C, geo);
  else
    hipLaunchKernelGGL(reverse_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)win,
                       (const float*)res, (float*)y, slots, C, geo);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) index_map_kernel(int32_t* __restrict__ map, uint8_t* __restrict__ region,
                                                        int64_t slots, WinGeo geo) {
  warm_args(map, region, slots, geo);
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= slots) return;
  int lab;
  const int w = (int)s / geo.N;
  const int64_t src = slot_source(geo, w, (int)s - w * geo.N, lab);
  map[s] = (int32_t)src;
  if (region) region[s] = (uint8_t)lab;
}

hipError_t index_map(int32_t* map, uint8_t* region, int64_t slots, const WinGeo& geo, hipStream_t st) {
  if (slots <= 0) return hipSuccess;
  hipLaunchKernelGGL(index_map_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, st, map, region,
                     slots, geo);
  return hipGetLastError();
}

}  // namespace vswin
