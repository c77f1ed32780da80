// Inference around the backbone:
//   * classification head: the mean of a clip's final tokens over
//     (T', H', W'), then Linear(C -> classes) (the 2D Swin page's global
//     average pooling and linear classifier on the 3D token grid);
//   * several views of a video (temporal clips x spatial crops, Table 1 of
//     the Video Swin Transformer page): the mean of the views' softmax
//     probabilities;
//   * 2D -> 3D inflation of an image model (§3.4, initialisation from an
//     image model): the patch kernel repeated over the pt temporal slots and
//     divided by pt; the relative-bias table repeated over the 2P - 1
//     temporal offsets (temporal offset outermost in the table's rows).
// All of it is memory- or latency-bound and small next to the blocks: plain
// coalesced loads, fp32 accumulation, fixed reduction orders (no atomics), so
// repeated calls give identical bits.
#include "vswin_kernels.h"

namespace vswin {

namespace {

constexpr int kHeadThreads = 256;
constexpr int kHeadClassesPerWg = 32;   // 8 per wave
constexpr int kFcSamples = 1;           // samples per classifier workgroup (more were slower)
constexpr int kViewThreads = 512;       // view average: 8 waves
constexpr int kViewMaxViews = 4096;     // (max, 1/sum) of every view in LDS

// VW consecutive elements as floats (16-byte loads for bf16 when VW = 8)
template <int VW>
__device__ __forceinline__ void loadv(const bf16_t* p, int64_t i, float* v) {
  if constexpr (VW == 8) {
    const u32x4_t t = *reinterpret_cast<const u32x4_t*>(p + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bflo(t[e]);
      v[2 * e + 1] = bfhi(t[e]);
    }
  } else {
    load4(p, i, v);
  }
}
template <int VW>
__device__ __forceinline__ void loadv(const float* p, int64_t i, float* v) {
  load4(p, i, v);
  if constexpr (VW == 8) load4(p, i + 4, v + 4);
}

// Partial channel sums of split s of sample b: token rows s L / S ..
// (s + 1) L / S - 1.  Thread t owns the VW channels of chunk t mod (C/VW) of
// every RPI-th row (RPI = 256 / (C/VW) row lanes when C/VW <= 256, else one
// row lane and chunks t, t + 256, ...); the row lanes meet in LDS at the end.
template <typename T, int VW>
__global__ void __launch_bounds__(kHeadThreads) head_pool_kernel(const T* __restrict__ x, float* __restrict__ part,
                                                                 int64_t L, int C, int S) {
  __shared__ float red[VW * kHeadThreads];
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t r0 = (int64_t)s * L / S, r1 = (int64_t)(s + 1) * L / S;
  const T* xb = x + (int64_t)b * L * C;
  float* pb = part + ((int64_t)b * S + s) * C;
  const int CPR = C / VW;
  if (CPR > kHeadThreads) {
    for (int j = tid; j < CPR; j += kHeadThreads) {
      float a[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) a[e] = 0.f;
#pragma unroll 4
      for (int64_t r = r0; r < r1; ++r) {
        float v[VW];
        loadv<VW>(xb, r * C + VW * j, v);
#pragma unroll
        for (int e = 0; e < VW; ++e) a[e] += v[e];
      }
#pragma unroll
      for (int e = 0; e < VW; e += 4)
        *reinterpret_cast<float4*>(pb + VW * j + e) = make_float4(a[e], a[e + 1], a[e + 2], a[e + 3]);
    }
    return;
  }
  const int RPI = kHeadThreads / CPR;
  const int j = tid % CPR, rl = tid / CPR;
  if (rl < RPI) {
    float a[VW];
#pragma unroll
    for (int e = 0; e < VW; ++e) a[e] = 0.f;
#pragma unroll 4
    for (int64_t r = r0 + rl; r < r1; r += RPI) {
      float v[VW];
      loadv<VW>(xb, r * C + VW * j, v);
#pragma unroll
      for (int e = 0; e < VW; ++e) a[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < VW; e += 4)
      *reinterpret_cast<float4*>(red + rl * C + VW * j + e) = make_float4(a[e], a[e + 1], a[e + 2], a[e + 3]);
  }
  __syncthreads();
  for (int c = tid; c < C; c += kHeadThreads) {
    float acc = 0.f;
    for (int q = 0; q < RPI; ++q) acc += red[q * C + c];
    pb[c] = acc;
  }
}

// pooled[b, c] = (sum of the S partial sums of channel c) / L
__global__ void __launch_bounds__(kHeadThreads) head_reduce_kernel(const float* __restrict__ part,
                                                                   float* __restrict__ pooled, int64_t L, int C,
                                                                   int S) {
  const int c = blockIdx.x * kHeadThreads + threadIdx.x, b = blockIdx.y;
  if (c >= C) return;
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) acc += part[((int64_t)b * S + s) * C + c];
  pooled[(int64_t)b * C + c] = acc * (1.0f / (float)L);
}

// logits[b, k] = pooled[b, :] . W[k, :] + bias[k] for the workgroup's 32
// classes (8 per wave) and kFcSamples samples: the samples' pooled vectors are
// staged in LDS; each weight fragment a lane loads serves all of them.
template <typename T>
__global__ void __launch_bounds__(kHeadThreads) head_fc_kernel(const float* __restrict__ pooled_g,
                                                               const T* __restrict__ w, const T* __restrict__ bias,
                                                               float* __restrict__ logits, int B, int C, int K) {
  extern __shared__ float pooled[];   // (kFcSamples, C)
  const int b0 = blockIdx.y * kFcSamples;
  const int nb = B - b0 < kFcSamples ? B - b0 : kFcSamples;
  for (int i = threadIdx.x; i < kFcSamples * C; i += kHeadThreads) {
    const int sb = i / C;
    pooled[i] = sb < nb ? pooled_g[(int64_t)b0 * C + i] : 0.f;
  }
  __syncthreads();
  constexpr int NK = kHeadClassesPerWg / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kb = blockIdx.x * kHeadClassesPerWg + wave * NK;
  float acc[NK][kFcSamples];
#pragma unroll
  for (int i = 0; i < NK; ++i)
#pragma unroll
    for (int j = 0; j < kFcSamples; ++j) acc[i][j] = 0.f;
  for (int c = 4 * lane; c < C; c += 256) {
    float wv[NK][4];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (kb + i < K) load4(w, (int64_t)(kb + i) * C + c, wv[i]);
      else wv[i][0] = wv[i][1] = wv[i][2] = wv[i][3] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kFcSamples; ++j) {
      const float4 p = *reinterpret_cast<const float4*>(pooled + j * C + c);
#pragma unroll
      for (int i = 0; i < NK; ++i) acc[i][j] += wv[i][0] * p.x + wv[i][1] * p.y + wv[i][2] * p.z + wv[i][3] * p.w;
    }
  }
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int k = kb + i;
    const float bk = (k < K && bias) ? Elem<T>::load(bias, k) : 0.f;
#pragma unroll
    for (int j = 0; j < kFcSamples; ++j) {
      float a = acc[i][j];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o);
      if (lane == 0 && k < K && j < nb) logits[(int64_t)(b0 + j) * K + k] = a + bk;
    }
  }
}

// probs[b, :] = mean over v of softmax(logits[b, v, :]); one workgroup per b.
// Each view's max and 1 / sum come from one wave (shuffle reductions), the
// waves taking views v, v + 8, ...; then every thread sums its classes over
// the views.
__global__ void __launch_bounds__(kViewThreads) view_avg_kernel(const float* __restrict__ logits,
                                                                float* __restrict__ probs, int V, int K) {
  extern __shared__ float2 ms[];   // per view: (max, 1 / sum of exp(z - max))
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int v = wave; v < V; v += kViewThreads / 64) {
    const float* z = logits + ((int64_t)b * V + v) * K;
    float m = -INFINITY;
    for (int k = lane; k < K; k += 64) m = fmaxf(m, z[k]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float sum = 0.f;
    for (int k = lane; k < K; k += 64) sum += expf(z[k] - m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) ms[v] = make_float2(m, 1.0f / sum);
  }
  __syncthreads();
  const float invV = 1.0f / (float)V;
  for (int k = threadIdx.x; k < K; k += kViewThreads) {
    float acc = 0.f;
    for (int v = 0; v < V; ++v) {
      const float2 t = ms[v];
      acc += expf(logits[((int64_t)b * V + v) * K + k] - t.x) * t.y;
    }
    probs[(int64_t)b * K + k] = acc * invV;
  }
}

// w3 (C, Cin, pt, ph, pw) from w2 (C, Cin, ph, pw): w2 / pt in every slot
template <typename T>
__global__ void __launch_bounds__(256) inflate_patch_kernel(const T* __restrict__ w2, T* __restrict__ w3,
                                                            int64_t total, int pt, int hw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t cc = i / ((int64_t)pt * hw);
  const int r = (int)(i - cc * pt * hw) % hw;
  Elem<T>::store(w3, i, Elem<T>::load(w2, cc * hw + r) / (float)pt);
}

// t3 = the n2 elements of t2, reps times over (a plain copy, any element size)
__global__ void __launch_bounds__(256) inflate_table_kernel(const uint16_t* __restrict__ t2,
                                                            uint16_t* __restrict__ t3, int64_t n2, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < total) t3[i] = t2[i % n2];
}

}  // namespace

int head_splits(int B, int64_t L) {
  // about 1024 workgroups over the batch (enough loads in flight for HBM),
  // at least 16 token rows each
  int64_t S = (1024 + B - 1) / (B > 0 ? B : 1);
  if (S > L / 16) S = L / 16;
  if (S < 1) S = 1;
  if (S > 256) S = 256;
  return (int)S;
}

size_t head_workspace_floats(int B, int64_t L, int C) {
  return (size_t)B * head_splits(B, L) * C + (size_t)B * C;
}

hipError_t head_fwd(vswin_dtype dt, const void* x, const void* w, const void* b, float* logits, float* work,
                    int B, int64_t L, int C, int K, hipStream_t st) {
  if (B == 0 || K == 0) return hipSuccess;
  const int S = head_splits(B, L);
  float* part = work;
  float* pooled = work + (size_t)B * S * C;
  const dim3 gp((unsigned)S, (unsigned)B), gr((unsigned)((C + kHeadThreads - 1) / kHeadThreads), (unsigned)B);
  const dim3 gf((unsigned)((K + kHeadClassesPerWg - 1) / kHeadClassesPerWg),
                (unsigned)((B + kFcSamples - 1) / kFcSamples));
  const size_t lds = (size_t)kFcSamples * C * sizeof(float);
  if (dt == VSWIN_BF16) {
    if (C % 8 == 0)
      hipLaunchKernelGGL((head_pool_kernel<bf16_t, 8>), gp, dim3(kHeadThreads), 0, st, (const bf16_t*)x, part, L, C, S);
    else
      hipLaunchKernelGGL((head_pool_kernel<bf16_t, 4>), gp, dim3(kHeadThreads), 0, st, (const bf16_t*)x, part, L, C, S);
  } else {
    if (C % 8 == 0)
      hipLaunchKernelGGL((head_pool_kernel<float, 8>), gp, dim3(kHeadThreads), 0, st, (const float*)x, part, L, C, S);
    else
      hipLaunchKernelGGL((head_pool_kernel<float, 4>), gp, dim3(kHeadThreads), 0, st, (const float*)x, part, L, C, S);
  }
  hipLaunchKernelGGL(head_reduce_kernel, gr, dim3(kHeadThreads), 0, st, part, pooled, L, C, S);
  if (dt == VSWIN_BF16) {
    const hipError_t e = ensure_dynamic_lds((const void*)head_fc_kernel<bf16_t>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(head_fc_kernel<bf16_t>, gf, dim3(kHeadThreads), lds, st, pooled, (const bf16_t*)w,
                       (const bf16_t*)b, logits, B, C, K);
  } else {
    const hipError_t e = ensure_dynamic_lds((const void*)head_fc_kernel<float>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(head_fc_kernel<float>, gf, dim3(kHeadThreads), lds, st, pooled, (const float*)w,
                       (const float*)b, logits, B, C, K);
  }
  return hipGetLastError();
}

int view_avg_max_views() { return kViewMaxViews; }

hipError_t view_avg(const float* logits, float* probs, int B, int V, int K, hipStream_t st) {
  if (B == 0 || K == 0) return hipSuccess;
  hipLaunchKernelGGL(view_avg_kernel, dim3((unsigned)B), dim3(kViewThreads), (size_t)V * sizeof(float2), st, logits,
                     probs, V, K);
  return hipGetLastError();
}

hipError_t inflate_patch(vswin_dtype dt, const void* w2, void* w3, int64_t C_Cin, int pt, int ph, int pw,
                         hipStream_t st) {
  const int64_t total = C_Cin * pt * ph * pw;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (dt == VSWIN_BF16)
    hipLaunchKernelGGL(inflate_patch_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t*)w2,
                       (bf16_t*)w3, total, pt, ph * pw);
  else
    hipLaunchKernelGGL(inflate_patch_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)w2, (float*)w3,
                       total, pt, ph * pw);
  return hipGetLastError();
}

hipError_t inflate_table(const void* t2, void* t3, int64_t n2_halves, int reps, hipStream_t st) {
  const int64_t total = n2_halves * reps;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(inflate_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)t2, (uint16_t*)t3, n2_halves, total);
  return hipGetLastError();
}

}  // namespace vswin
