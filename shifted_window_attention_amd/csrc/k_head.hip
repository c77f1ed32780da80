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
constexpr int kViewThreads = 512;       // view average: 8 waves
constexpr int kViewMaxViews = 4096;     // (max, 1/sum) of every view in LDS

// Partial channel sums of split s of sample b: token rows s L / S ..
// (s + 1) L / S - 1.  Thread t owns the 4 channels of chunk t mod (C/4) of
// every RPI-th row (RPI = 256 / (C/4) row lanes when C/4 <= 256, else one row
// lane and chunks t, t + 256, ...); the row lanes meet in LDS at the end.
template <typename T>
__global__ void __launch_bounds__(kHeadThreads) head_pool_kernel(const T* __restrict__ x, float* __restrict__ part,
                                                                 int64_t L, int C, int S) {
  __shared__ float red[4 * kHeadThreads];
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t r0 = (int64_t)s * L / S, r1 = (int64_t)(s + 1) * L / S;
  const T* xb = x + (int64_t)b * L * C;
  float* pb = part + ((int64_t)b * S + s) * C;
  const int CPR = C / 4;
  if (CPR > kHeadThreads) {
    for (int j = tid; j < CPR; j += kHeadThreads) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
      for (int64_t r = r0; r < r1; ++r) {
        float v[4];
        load4(xb, r * C + 4 * j, v);
        a0 += v[0]; a1 += v[1]; a2 += v[2]; a3 += v[3];
      }
      *reinterpret_cast<float4*>(pb + 4 * j) = make_float4(a0, a1, a2, a3);
    }
    return;
  }
  const int RPI = kHeadThreads / CPR;
  const int j = tid % CPR, rl = tid / CPR;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  if (rl < RPI) {
#pragma unroll 8
    for (int64_t r = r0 + rl; r < r1; r += RPI) {
      float v[4];
      load4(xb, r * C + 4 * j, v);
      a0 += v[0]; a1 += v[1]; a2 += v[2]; a3 += v[3];
    }
    *reinterpret_cast<float4*>(red + rl * C + 4 * j) = make_float4(a0, a1, a2, a3);
  }
  __syncthreads();
  for (int c = tid; c < C; c += kHeadThreads) {
    float acc = 0.f;
    for (int q = 0; q < RPI; ++q) acc += red[q * C + c];
    pb[c] = acc;
  }
}

// logits[b, k] = (sum of the S partial sums) / L . W[k, :] + bias[k] for the
// workgroup's 32 classes (8 per wave); the pooled vector sits in LDS.
template <typename T>
__global__ void __launch_bounds__(kHeadThreads) head_fc_kernel(const float* __restrict__ part, const T* __restrict__ w,
                                                               const T* __restrict__ bias, float* __restrict__ logits,
                                                               int64_t L, int C, int S, int K) {
  extern __shared__ float pooled[];
  const int b = blockIdx.y;
  const float inv = 1.0f / (float)L;
  for (int c = threadIdx.x; c < C; c += kHeadThreads) {
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) acc += part[((int64_t)b * S + s) * C + c];
    pooled[c] = acc * inv;
  }
  __syncthreads();
  constexpr int NK = kHeadClassesPerWg / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kb = blockIdx.x * kHeadClassesPerWg + wave * NK;
  float acc[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) acc[i] = 0.f;
  for (int c = 4 * lane; c < C; c += 256) {
    const float p0 = pooled[c], p1 = pooled[c + 1], p2 = pooled[c + 2], p3 = pooled[c + 3];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (kb + i < K) {
        float v[4];
        load4(w, (int64_t)(kb + i) * C + c, v);
        acc[i] += v[0] * p0 + v[1] * p1 + v[2] * p2 + v[3] * p3;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    float a = acc[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o);
    const int k = kb + i;
    if (lane == 0 && k < K) logits[(int64_t)b * K + k] = a + (bias ? Elem<T>::load(bias, k) : 0.f);
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
  // at least 8 token rows each
  int64_t S = (1024 + B - 1) / (B > 0 ? B : 1);
  if (S > L / 8) S = L / 8;
  if (S < 1) S = 1;
  if (S > 256) S = 256;
  return (int)S;
}

hipError_t head_fwd(vswin_dtype dt, const void* x, const void* w, const void* b, float* logits, float* part,
                    int B, int64_t L, int C, int K, hipStream_t st) {
  if (B == 0 || K == 0) return hipSuccess;
  const int S = head_splits(B, L);
  const size_t lds = (size_t)C * sizeof(float);
  if (dt == VSWIN_BF16) {
    hipLaunchKernelGGL(head_pool_kernel<bf16_t>, dim3((unsigned)S, (unsigned)B), dim3(kHeadThreads), 0, st,
                       (const bf16_t*)x, part, L, C, S);
    hipError_t e = ensure_dynamic_lds((const void*)head_fc_kernel<bf16_t>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(head_fc_kernel<bf16_t>, dim3((unsigned)((K + kHeadClassesPerWg - 1) / kHeadClassesPerWg),
                       (unsigned)B), dim3(kHeadThreads), lds, st, part, (const bf16_t*)w, (const bf16_t*)b, logits,
                       L, C, S, K);
  } else {
    hipLaunchKernelGGL(head_pool_kernel<float>, dim3((unsigned)S, (unsigned)B), dim3(kHeadThreads), 0, st,
                       (const float*)x, part, L, C, S);
    hipError_t e = ensure_dynamic_lds((const void*)head_fc_kernel<float>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(head_fc_kernel<float>, dim3((unsigned)((K + kHeadClassesPerWg - 1) / kHeadClassesPerWg),
                       (unsigned)B), dim3(kHeadThreads), lds, st, part, (const float*)w, (const float*)b, logits,
                       L, C, S, K);
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
