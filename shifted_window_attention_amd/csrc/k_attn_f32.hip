// Window attention in fp32 on the matrix cores (§3.2, eq. 2):
//   per (window, head): S = q k^T / sqrt(d) + B[idx(i, j)], masked pairs
//   excluded (or -100 added with the MASK_M100 flag), P = softmax_j(S),
//   O = P v, heads concatenated as h*d + e.
//
// One workgroup (4 waves) per (window, head) item; K and V (fp32, natural
// slot order) and the head's bias column go to LDS, and each wave owns
// 16-query tiles.  Both products run on v_mfma_f32_16x16x4_f32:
//   * S^T = K Q^T per 16-key tile (k = 4 head dims per instruction), so a
//     lane holds 4 keys of one query and the softmax state stays in the lane.
//     The K rows of a tile enter the product in the order 4i + g -> row
//     4g + i (a 4 x 4 transpose of the key index), so that register i of
//     lane group g holds key 4i + g: after the exponentials, register c of
//     every lane group is already the B operand of the P V product for keys
//     4c .. 4c + 3.
//   * O^T = V^T P^T, 16 head dims per output tile, a lane ends with 4
//     consecutive output features of one query (one 16-byte store).
// The softmax is exact in fp32: a first pass over the keys takes each row's
// maximum, the second recomputes the same scores (the same instruction
// sequence, so the same bits), subtracts it and accumulates exp, its sum and
// P V.  The shapes it does not serve (LDS bound, head dims that are not a
// multiple of 16) run on the SIMT kernel in k_attention.hip.
#include "vswin_kernels.h"

#include <math.h>

namespace vswin {

namespace {

constexpr int kF32Waves = 4;
constexpr size_t kF32Lds = 160 * 1024;

struct F32Lay {
  int NP;         // keys padded to 16
  int pitch;      // K / V row pitch in floats (d + 1: conflict-free column reads)
  uint32_t off_k, off_v, off_kf, off_lab, off_tab, bytes;
};

inline bool f32_layout(const AttnArgs& a, F32Lay& F) {
  F.NP = (a.N + 15) / 16 * 16;
  F.pitch = a.d + 1;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += (n + 15) & ~(size_t)15;
    return (uint32_t)o;
  };
  F.off_k = take((size_t)F.NP * F.pitch * 4);
  F.off_v = take((size_t)F.NP * F.pitch * 4);
  F.off_kf = take((size_t)F.NP * 4);
  F.off_lab = take((size_t)F.NP * 4);
  F.off_tab = take((size_t)a.rel.rows * 4);
  F.bytes = (uint32_t)off;
  return off <= kF32Lds;
}

template <int D>
__global__ void __launch_bounds__(64 * kF32Waves) attn_f32_mfma_kernel(const AttnArgs a, const F32Lay F) {
  warm_args(a, F);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* Ks = reinterpret_cast<float*>(smem + F.off_k);
  float* Vs = reinterpret_cast<float*>(smem + F.off_v);
  int* kf = reinterpret_cast<int*>(smem + F.off_kf);
  int* klab = reinterpret_cast<int*>(smem + F.off_lab);
  float* tab = reinterpret_cast<float*>(smem + F.off_tab);
  const int item = blockIdx.x;
  const int w = item / a.heads;
  const int h = item - w * a.heads;
  const WinGeo& g = a.geo;
  const int N = a.N, NP = F.NP, P = F.pitch;
  const int tid = threadIdx.x;

  // window origin in rolled coordinates; key offsets into the table and region labels
  const int wr = w % g.nws;
  const int wpl = g.nwh * g.nww;
  const int wt = wr / wpl, rem = wr - wt * wpl, wh = rem / g.nww, ww = rem - (rem / g.nww) * g.nww;
  const int rt0 = wt * g.P, rh0 = wh * g.Mh, rw0 = ww * g.Mw;
  const int mhw = g.Mh * g.Mw;
  for (int n = tid; n < NP; n += 64 * kF32Waves) {
    int off = 0, lab = -1;
    if (n < N) {
      const int pt = n / mhw, r2 = n - pt * mhw, ph = r2 / g.Mw, pw = r2 - ph * g.Mw;
      off = pt * a.rel.R + ph * a.rel.Rw + pw;
      lab = slot_label_at(g, rt0 + pt, rh0 + ph, rw0 + pw);
    }
    kf[n] = off;
    klab[n] = lab;
  }
  const float* Kg = reinterpret_cast<const float*>(a.k) + (int64_t)item * N * D;
  const float* Vg = reinterpret_cast<const float*>(a.v) + (int64_t)item * N * D;
  for (int x = tid; x < NP * D; x += 64 * kF32Waves) {
    const int n = x / D, e = x - n * D;
    Ks[n * P + e] = n < N ? Kg[x] : 0.f;
    Vs[n * P + e] = n < N ? Vg[x] : 0.f;
  }
  const float* Tg = reinterpret_cast<const float*>(a.table);
  for (int r = tid; r < a.rel.rows; r += 64 * kF32Waves) tab[r] = Tg[(int64_t)r * a.heads + h];
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6;
  const int fr = lane & 15, g4 = lane >> 4;
  const float scale = 1.0f / sqrtf((float)D);
  const float* Qg = reinterpret_cast<const float*>(a.q) + (int64_t)item * N * D;
  float* Og = reinterpret_cast<float*>(a.o);
  const int nkt = NP / 16;
  for (int qt = wv; qt < nkt; qt += kF32Waves) {
    const int q = 16 * qt + fr;
    const bool qok = q < N;
    // B operand of the score product: q[dim 4 kk + g4] of query fr
    float qv[D / 4];
#pragma unroll
    for (int kk = 0; kk < D / 4; ++kk) qv[kk] = qok ? Qg[(int64_t)q * D + 4 * kk + g4] * scale : 0.f;
    const int qf = (qok ? kf[q] : 0) + a.rel.centre;
    const int ql = qok ? klab[q] : -2;
    // scores of key tile kt for this lane: keys 16 kt + 4 i + g4, i = 0..3
    auto scores = [&](int kt, float s[4]) {
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // A operand row fr = key 16 kt + 4 (fr & 3) + (fr >> 2)
      const float* kr = Ks + (16 * kt + 4 * (fr & 3) + (fr >> 2)) * P + g4;
#pragma unroll
      for (int kk = 0; kk < D / 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[4 * kk], qv[kk], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kt + 4 * i + g4;
        float v = acc[i];
        if (key >= N) {
          v = -INFINITY;
        } else {
          v += tab[qf - kf[key]];
          if (a.use_mask && klab[key] != ql) v = a.mask_m100 ? v - 100.f : -INFINITY;
        }
        s[i] = v;
      }
    };
    float m = -INFINITY;
    for (int kt = 0; kt < nkt; ++kt) {
      float s[4];
      scores(kt, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, s[i]);
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (m == -INFINITY) m = 0.f;
    f32x4_t o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float sum = 0.f;
    for (int kt = 0; kt < nkt; ++kt) {
      float s[4];
      scores(kt, s);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = expf(s[i] - m);
        sum += p[i];
      }
      // O^T += V^T P^T over the tile's keys, 4 at a time: keys 16 kt + 4 c + g4
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float* vr = Vs + (16 * kt + 4 * c + g4) * P + fr;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[16 * dt], p[c], o[dt], 0, 0, 0);
      }
    }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    if (qok) {
      const float inv = 1.0f / sum;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        float4 r;
        r.x = o[dt][0] * inv;
        r.y = o[dt][1] * inv;
        r.z = o[dt][2] * inv;
        r.w = o[dt][3] * inv;
        *reinterpret_cast<float4*>(Og + ((int64_t)w * N + q) * a.C + h * D + 16 * dt + 4 * g4) = r;
      }
    }
  }
}

}  // namespace

bool attention_f32_mfma_supported(vswin_dtype dt, const AttnArgs& a) {
  if (dt != VSWIN_FP32 || (a.d != 16 && a.d != 32 && a.d != 64) || a.N <= 0) return false;
  F32Lay F;
  return f32_layout(a, F);
}

hipError_t attention_f32_mfma(const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  F32Lay F;
  if (!attention_f32_mfma_supported(VSWIN_FP32, a) || !f32_layout(a, F) || items > 0x7fffffff)
    return hipErrorInvalidValue;
  auto go = [&](const void* kern, auto launch) -> hipError_t {
    const hipError_t e = ensure_dynamic_lds(kern, F.bytes);
    if (e != hipSuccess) return e;
    launch();
    return hipGetLastError();
  };
  const dim3 grid((unsigned)items), block(64 * kF32Waves);
  if (a.d == 16)
    return go((const void*)attn_f32_mfma_kernel<16>, [&] { attn_f32_mfma_kernel<16><<<grid, block, F.bytes, st>>>(a, F); });
  if (a.d == 32)
    return go((const void*)attn_f32_mfma_kernel<32>, [&] { attn_f32_mfma_kernel<32><<<grid, block, F.bytes, st>>>(a, F); });
  return go((const void*)attn_f32_mfma_kernel<64>, [&] { attn_f32_mfma_kernel<64><<<grid, block, F.bytes, st>>>(a, F); });
}

}  // namespace vswin
