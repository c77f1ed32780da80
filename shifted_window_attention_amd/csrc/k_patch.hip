// Gathers of the backbone's patch embedding and patch merging (§3.1 steps
// 1-2): exact permutations (with zero fill beyond the grid) that turn both
// layers into plain Linear layers on the MFMA GEMM.
#include "vswin_kernels.h"

namespace vswin {

// video (B, Cin, T, H, W) -> rows (B*T'*H'*W', Cin*pt*ph*pw), patch values in
// (c, kt, kh, kw) order, zeros beyond the video's end.
template <typename T>
__global__ void __launch_bounds__(256) patch_gather_kernel(const T* __restrict__ v, T* __restrict__ out, int B,
                                                           int Cin, int Tv, int Hv, int Wv, int pt, int ph,
                                                           int pw, int To, int Ho, int Wo) {
  const int K = Cin * pt * ph * pw;
  const int64_t total = (int64_t)B * To * Ho * Wo * K;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / K;
  int k = (int)(i - row * K);
  const int kw = k % pw; k /= pw;
  const int kh = k % ph; k /= ph;
  const int kt = k % pt;
  const int c = k / pt;
  int64_t r = row;
  const int wo = (int)(r % Wo); r /= Wo;
  const int ho = (int)(r % Ho); r /= Ho;
  const int to = (int)(r % To);
  const int b = (int)(r / To);
  const int t = to * pt + kt, h = ho * ph + kh, w = wo * pw + kw;
  float val = 0.f;
  if (t < Tv && h < Hv && w < Wv)
    val = Elem<T>::load(v, ((((int64_t)b * Cin + c) * Tv + t) * Hv + h) * Wv + w);
  Elem<T>::store(out, i, val);
}

// pw = 4: one thread per (b, c, t, h, w-group) of the patch-padded video
// moves the 4 consecutive w values of one patch row at once (one 8-byte
// load and store for bf16, 16 bytes for fp32); consecutive threads read
// consecutive w-groups.  32-bit index arithmetic (the launch checks the range).
template <typename T>
__global__ void __launch_bounds__(256) patch_gather4_kernel(const T* __restrict__ v, T* __restrict__ out, int Cin,
                                                            int Tv, int Hv, int Wv, int pt, int ph, int To, int Ho,
                                                            int Wo, int total) {
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= total) return;
  const int Tp = To * pt, Hp = Ho * ph;
  int r = i;
  const int wo = r % Wo; r /= Wo;
  const int h = r % Hp; r /= Hp;
  const int t = r % Tp; r /= Tp;
  const int c = r % Cin;
  const int b = r / Cin;
  const int K = Cin * pt * ph * 4;
  const int64_t row = (((int64_t)b * To + t / pt) * Ho + h / ph) * Wo + wo;
  T* dst = out + row * K + ((c * pt + t % pt) * ph + h % ph) * 4;
  const int w = wo * 4;
  float val[4] = {0.f, 0.f, 0.f, 0.f};
  if (t < Tv && h < Hv) {
    const T* src = v + ((((int64_t)b * Cin + c) * Tv + t) * Hv + h) * Wv + w;
    if (w + 4 <= Wv) {
      load4(src, 0, val);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (w + e < Wv) val[e] = Elem<T>::load(src, e);
    }
  }
  store4(dst, 0, val);
}

hipError_t patch_gather(vswin_dtype dt, const void* video, void* out, int B, int Cin, int T, int H, int W,
                        int pt, int ph, int pw, hipStream_t st) {
  const int To = (T + pt - 1) / pt, Ho = (H + ph - 1) / ph, Wo = (W + pw - 1) / pw;
  const int64_t total = (int64_t)B * To * Ho * Wo * Cin * pt * ph * pw;
  if (total <= 0) return hipSuccess;
  // pw = 4 with w-groups aligned to 4 elements: the vector kernel
  const int64_t total4 = (int64_t)B * Cin * (To * pt) * (Ho * ph) * Wo;
  const uintptr_t al = dt == VSWIN_BF16 ? 8 : 16;
  if (pw == 4 && W % 4 == 0 && total4 < 0x7fffffff && (uintptr_t)video % al == 0 && (uintptr_t)out % al == 0) {
    const unsigned b4 = (unsigned)((total4 + 255) / 256);
    if (dt == VSWIN_BF16)
      hipLaunchKernelGGL(patch_gather4_kernel<bf16_t>, dim3(b4), dim3(256), 0, st, (const bf16_t*)video,
                         (bf16_t*)out, Cin, T, H, W, pt, ph, To, Ho, Wo, (int)total4);
    else
      hipLaunchKernelGGL(patch_gather4_kernel<float>, dim3(b4), dim3(256), 0, st, (const float*)video, (float*)out,
                         Cin, T, H, W, pt, ph, To, Ho, Wo, (int)total4);
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dt == VSWIN_BF16)
    hipLaunchKernelGGL(patch_gather_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)video,
                       (bf16_t*)out, B, Cin, T, H, W, pt, ph, pw, To, Ho, Wo);
  else
    hipLaunchKernelGGL(patch_gather_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)video,
                       (float*)out, B, Cin, T, H, W, pt, ph, pw, To, Ho, Wo);
  return hipGetLastError();
}

// x (B, T, H, W, C) -> (B, T, H2, W2, 4C): the 2x2 group in (h, w) offset
// order (0,0), (1,0), (0,1), (1,1); zeros beyond the grid.  4 channels per
// thread.
template <typename T>
__global__ void __launch_bounds__(256) merge_gather_kernel(const T* __restrict__ x, T* __restrict__ out, int B,
                                                           int Tn, int H, int W, int C, int H2, int W2) {
  const int c4 = C / 4;
  const int64_t total = (int64_t)B * Tn * H2 * W2 * 4 * c4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  int64_t r = i;
  const int cc = (int)(r % c4); r /= c4;
  const int q = (int)(r % 4); r /= 4;
  const int j = (int)(r % W2); r /= W2;
  const int ii = (int)(r % H2); r /= H2;
  const int t = (int)(r % Tn);
  const int b = (int)(r / Tn);
  const int h = 2 * ii + (q & 1), w = 2 * j + (q >> 1);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (h < H && w < W) load4(x, ((((int64_t)b * Tn + t) * H + h) * W + w) * C + 4 * cc, v);
  store4(out, i * 4, v);
}

hipError_t merge_gather(vswin_dtype dt, const void* x, void* out, int B, int T, int H, int W, int C,
                        hipStream_t st) {
  const int H2 = (H + 1) / 2, W2 = (W + 1) / 2;
  const int64_t total = (int64_t)B * T * H2 * W2 * C;
  if (total <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dt == VSWIN_BF16)
    hipLaunchKernelGGL(merge_gather_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)x,
                       (bf16_t*)out, B, T, H, W, C, H2, W2);
  else
    hipLaunchKernelGGL(merge_gather_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)x,
                       (float*)out, B, T, H, W, C, H2, W2);
  return hipGetLastError();
}

}  // namespace vswin
