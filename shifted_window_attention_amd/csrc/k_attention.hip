// Window attention of the Video Swin block (§3.2, eq. 2), generic path:
//   per (window, head): S = (q k^T) / sqrt(d) + B[idx(i, j)], masked pairs
//   excluded (or -100 added with the MASK_M100 flag), P = softmax_j(S),
//   O = P v, heads concatenated as h*d + e.
//
// SIMT fp32 arithmetic for any dtype / head_dim <= 64 / window of up to 2048
// tokens, two passes (row max, then exp-sum and P v); it serves the shapes
// neither MFMA kernel does (bf16: k_attn_mfma.hip; fp32: k_attn_f32.hip).
#include "vswin_kernels.h"

#include <math.h>

namespace vswin {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kGenMaxN = 2048;

// ---------------------------------------------------------------------------
// generic kernel
// ---------------------------------------------------------------------------
template <typename T, int DMAX>
__global__ void __launch_bounds__(256) attn_generic_kernel(const AttnArgs a) {
  warm_args(a);
  __shared__ int kf[kGenMaxN];
  __shared__ int klab[kGenMaxN];
  const int item = blockIdx.x;
  const int w = item / a.heads;
  const int h = item - w * a.heads;
  const WinGeo& g = a.geo;
  const int N = a.N, d = a.d;
  const int wr = w % g.nws;
  const int wpl = g.nwh * g.nww;
  const int wt = wr / wpl, rem = wr - wt * wpl, wh = rem / g.nww, ww = rem - (rem / g.nww) * g.nww;
  const int rt0 = wt * g.P, rh0 = wh * g.Mh, rw0 = ww * g.Mw;
  const int mhw = g.Mh * g.Mw;
  for (int n = threadIdx.x; n < N; n += 256) {
    const int pt = n / mhw, r2 = n - pt * mhw, ph = r2 / g.Mw, pw = r2 - ph * g.Mw;
    kf[n] = pt * a.rel.R + ph * a.rel.Rw + pw;
    klab[n] = slot_label_at(g, rt0 + pt, rh0 + ph, rw0 + pw);
  }
  __syncthreads();
  const T* Q = (const T*)a.q + (int64_t)item * N * d;
  const T* K = (const T*)a.k + (int64_t)item * N * d;
  const T* V = (const T*)a.v + (int64_t)item * N * d;
  const T* tab = (const T*)a.table;
  T* O = (T*)a.o;
  const float scale = 1.0f / sqrtf((float)d);
  for (int qi = threadIdx.x; qi < N; qi += 256) {
    float qv[DMAX], acc[DMAX];
#pragma unroll
    for (int e = 0; e < DMAX; ++e) {
      qv[e] = e < d ? Elem<T>::load(Q, (int64_t)qi * d + e) * scale : 0.f;
      acc[e] = 0.f;
    }
    const int qf = kf[qi] + a.rel.centre;
    const int ql = klab[qi];
    float mx = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
      float sum = 0.f;
      for (int j = 0; j < N; ++j) {
        const bool diff = a.use_mask && klab[j] != ql;
        if (diff && !a.mask_m100) continue;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DMAX; ++e)
          if (e < d) s = fmaf(qv[e], Elem<T>::load(K, (int64_t)j * d + e), s);
        s += Elem<T>::load(tab, (int64_t)(qf - kf[j]) * a.heads + h);
        if (diff) s -= 100.f;
        if (pass == 0) {
          mx = fmaxf(mx, s);
        } else {
          const float p = expf(s - mx);
          sum += p;
#pragma unroll
          for (int e = 0; e < DMAX; ++e)
            if (e < d) acc[e] = fmaf(p, Elem<T>::load(V, (int64_t)j * d + e), acc[e]);
        }
      }
      if (pass == 1) {
        const float inv = 1.0f / sum;
        for (int e = 0; e < d; ++e)
          Elem<T>::store(O, ((int64_t)w * N + qi) * a.C + h * d + e, acc[e] * inv);
      }
    }
  }
}

hipError_t attention_generic(vswin_dtype dt, const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  if (attention_f32_mfma_supported(dt, a)) return attention_f32_mfma(a, st);
  if (a.N > kGenMaxN || a.d > 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)items), block(256);
  if (dt == VSWIN_BF16) {
    if (a.d <= 32) hipLaunchKernelGGL((attn_generic_kernel<bf16_t, 32>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_generic_kernel<bf16_t, 64>), grid, block, 0, st, a);
  } else {
    if (a.d <= 16) hipLaunchKernelGGL((attn_generic_kernel<float, 16>), grid, block, 0, st, a);
    else if (a.d <= 32) hipLaunchKernelGGL((attn_generic_kernel<float, 32>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_generic_kernel<float, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace vswin
