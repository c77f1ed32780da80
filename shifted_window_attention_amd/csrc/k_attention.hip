// Window attention of the Video Swin block (§3.2, eq. 2):
//   per (window, head): S = (q k^T) / sqrt(d) + B[idx(i, j)], masked pairs
//   excluded, P = softmax_j(S), O = P v, heads concatenated as h*d + e.
//
// attention_mfma -- the bf16 hot path (head_dim 32).  One workgroup per
// (window, head, query split); 4 waves, each owning up to 4 query tiles of 16.
//   * K (slot order) and V^T are staged once per workgroup in LDS; the head's
//     bias table is staged reversed, pre-scaled by log2(e), as fp16, followed
//     by a -inf zone that masked and dummy key groups point into.
//   * Key slots are permuted so that the 4 keys a lane holds in an MFMA
//     output fragment differ only in their temporal coordinate (kt = 4a + i):
//     their table rows are then r, r+R, r+2R, r+3R and one address with four
//     immediate offsets reads them.  Queries keep window order.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (k = head_dim): each lane holds
//     4 keys of one query, so per-query state (label, table address, running
//     sum, output) stays in the lane -- no cross-lane softmax reductions.
//   * scale, log2(e) and bias enter in one v_fma_mix (fp32 score, fp16 bias);
//     P = exp2(...) with no running max when a Cauchy-Schwarz bound
//     |score| <= alpha |q| max|k| + log2e max|B| shows exp2 cannot overflow
//     or underflow (softmax is shift invariant); otherwise a first pass
//     computes the exact row max.
//   * O^T = V^T P^T on MFMA with P^T already in B-operand layout; the row
//     sums come from a third MFMA against a ones operand, so the weights that
//     multiply V are exactly the ones that are summed.
//
// attention_generic -- SIMT fp32 arithmetic for any dtype / head_dim <= 64 /
// window; serves the fp32 workload and shapes the MFMA kernel does not.
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
  __shared__ int kf[kGenMaxN];
  __shared__ int klab[kGenMaxN];
  const int64_t item = blockIdx.x;
  const int64_t w = item / a.heads;
  const int h = (int)(item - w * a.heads);
  const WinGeo& g = a.geo;
  const int N = a.N, d = a.d;
  const int wr = (int)(w % g.nws);
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
  const T* Q = (const T*)a.q + item * N * d;
  const T* K = (const T*)a.k + item * N * d;
  const T* V = (const T*)a.v + item * N * d;
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
          Elem<T>::store(O, (w * N + qi) * (int64_t)a.C + h * d + e, acc[e] * inv);
      }
    }
  }
}

hipError_t attention_generic(vswin_dtype dt, const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
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

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kQT = 4;            // query tiles per wave
constexpr int kWaves = 4;
constexpr int kKLD = 40;          // K row pitch in LDS (elements): 80 bytes
constexpr int kDummyLab = 0x7fff0000;
constexpr int kNoQueryLab = 0x7ffe0000;

struct MfmaLaunch {
  int NT;        // key tiles of 16 (slots padded to NT*16)
  int VST;       // V^T row pitch (elements)
  int QTT;       // query tiles of 16
  int qsplit;    // workgroups per (window, head)
  int tps;       // query tiles per workgroup
  int tab_n;     // fp16 entries of table + -inf zone
  size_t lds;    // dynamic LDS bytes
  size_t off_vt, off_tab, off_kaddr, off_klab, off_red;
};

static MfmaLaunch mfma_launch(const AttnArgs& a) {
  MfmaLaunch L{};
  L.NT = (a.N + 15) / 16;
  const int nt2 = (L.NT + 1) & ~1;
  L.VST = nt2 * 16 + 4;          // (VST/2) mod 32 = 2 * odd: conflict-free 8-byte column reads
  L.QTT = L.NT;
  const int per_wg = kWaves * kQT;
  int qs = (L.QTT + per_wg - 1) / per_wg;
  if (const char* s = getenv("VSWIN_ATTN_QSPLIT")) {
    const int v = atoi(s);
    if (v >= qs && v <= L.QTT) qs = v;
  }
  L.qsplit = qs;
  L.tps = (L.QTT + qs - 1) / qs;
  L.tab_n = a.rel.rows + 3 * a.rel.R + 8;
  size_t off = (size_t)L.NT * 16 * kKLD * 2;
  L.off_vt = off;
  off += (size_t)32 * L.VST * 2;
  L.off_tab = off;
  off += ((size_t)L.tab_n * 2 + 15) & ~(size_t)15;
  L.off_kaddr = off;
  off += (size_t)L.NT * 4 * 4;
  L.off_klab = off;
  off += (size_t)L.NT * 4 * 4;
  L.off_red = off;
  off += 16;
  L.lds = off;
  return L;
}

bool attention_mfma_supported(vswin_dtype dt, const AttnArgs& a) {
  if (dt != VSWIN_BF16 || a.d != 32 || a.mask_m100) return false;
  if (a.geo.P % 4 != 0 || a.N > kMfmaMaxN) return false;
  // every group of 4 temporal positions (kt = 4a .. 4a+3) of every window
  // must share its temporal label and temporal pad status
  const WinGeo& g = a.geo;
  auto tkey = [&](int rt) {
    int ot = rt + g.st;
    if (ot >= g.Tp) ot -= g.Tp;
    const int pad = (ot >= g.T && !g.pad_visible) ? 1 : 0;
    return axis_label(rt, g.Tp, g.P, g.st) * 2 + pad;
  };
  for (int rt = 0; rt < g.Tp; rt += 4)
    for (int i = 1; i < 4; ++i)
      if (tkey(rt + i) != tkey(rt)) return false;
  return mfma_launch(a).lds <= 160 * 1024;
}

template <int MODE>   // 0: exp2(x)  1: row max only  2: exp2(x - rowmax)
__device__ __forceinline__ void attn_pass(const bf16_t* __restrict__ Ks, const bf16_t* __restrict__ Vt,
                                          const unsigned char* __restrict__ tabb, const int* __restrict__ kaddr,
                                          const int* __restrict__ klab, int NT, int N, int VST, int R2,
                                          int zone, bool wmasked, float alpha, const bool vq[kQT],
                                          const bf16x8_t qreg[kQT], const int qaddr[kQT], const int qlab[kQT],
                                          float mrow[kQT], f32x4_t acc0[kQT], f32x4_t acc1[kQT],
                                          f32x4_t accs[kQT]) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  bf16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int tp = 0; tp < NT; tp += 2) {
    const bool hasB = tp + 1 < NT;
    const bool sel = wmasked || (tp + 2) * 16 > N;
    const bf16x8_t kA = *reinterpret_cast<const bf16x8_t*>(Ks + (16 * tp + fr) * kKLD + g4 * 8);
    bf16x8_t kB;
    if (hasB) kB = *reinterpret_cast<const bf16x8_t*>(Ks + (16 * tp + 16 + fr) * kKLD + g4 * 8);
    else kB = bf16x8_t{};
    const int gA = kaddr[4 * tp + g4];
    const int gB = hasB ? kaddr[4 * tp + 4 + g4] : 0;
    int lA = 0, lB = 0;
    if (sel) {
      lA = klab[4 * tp + g4];
      lB = hasB ? klab[4 * tp + 4 + g4] : kDummyLab;
    }
    bf16x8_t vA0, vA1;
    if (MODE != 1) {
      const u32x2_t* p0 = reinterpret_cast<const u32x2_t*>(Vt + fr * VST + 16 * tp + 4 * g4);
      const u32x2_t* p1 = reinterpret_cast<const u32x2_t*>(Vt + (fr + 16) * VST + 16 * tp + 4 * g4);
      u32x4_t t0, t1;
      const u32x2_t a0 = p0[0], b0 = p0[4], a1 = p1[0], b1 = p1[4];   // +16 slots = +32 bytes
      t0[0] = a0[0]; t0[1] = a0[1]; t0[2] = b0[0]; t0[3] = b0[1];
      t1[0] = a1[0]; t1[1] = a1[1]; t1[2] = b1[0]; t1[3] = b1[1];
      vA0 = __builtin_bit_cast(bf16x8_t, t0);
      vA1 = __builtin_bit_cast(bf16x8_t, t1);
    }
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
      if (!vq[u]) continue;
      const f32x4_t sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, qreg[u], zero4, 0, 0, 0);
      f32x4_t sB = zero4;
      if (hasB) sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kB, qreg[u], zero4, 0, 0, 0);
      int adA = qaddr[u] + gA, adB = qaddr[u] + gB;
      if (sel) {
        adA = (lA == qlab[u]) ? adA : zone;
        adB = (lB == qlab[u]) ? adB : zone;
      }
      float xA[4], xB[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bA = (float)*reinterpret_cast<const _Float16*>(tabb + adA + i * R2);
        const float bB = (float)*reinterpret_cast<const _Float16*>(tabb + adB + i * R2);
        xA[i] = __builtin_fmaf(sA[i], alpha, bA);
        xB[i] = __builtin_fmaf(sB[i], alpha, bB);
      }
      if (MODE == 1) {
        float m = mrow[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(xA[i], xB[i]));
        mrow[u] = m;
      } else {
        float pA[4], pB[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (MODE == 2) {
            pA[i] = __builtin_amdgcn_exp2f(xA[i] - mrow[u]);
            pB[i] = __builtin_amdgcn_exp2f(xB[i] - mrow[u]);
          } else {
            pA[i] = __builtin_amdgcn_exp2f(xA[i]);
            pB[i] = __builtin_amdgcn_exp2f(xB[i]);
          }
        }
        u32x4_t pk;
        pk[0] = pack_bf16x2(pA[0], pA[1]);
        pk[1] = pack_bf16x2(pA[2], pA[3]);
        pk[2] = pack_bf16x2(pB[0], pB[1]);
        pk[3] = pack_bf16x2(pB[2], pB[3]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
        acc0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA0, pb, acc0[u], 0, 0, 0);
        acc1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA1, pb, acc1[u], 0, 0, 0);
        accs[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, accs[u], 0, 0, 0);
      }
    }
  }
}

__global__ void __launch_bounds__(256) attn_mfma_kernel(const AttnArgs a, const MfmaLaunch L, const float alpha) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem);
  bf16_t* Vt = reinterpret_cast<bf16_t*>(smem + L.off_vt);
  _Float16* tab = reinterpret_cast<_Float16*>(smem + L.off_tab);
  int* kaddr = reinterpret_cast<int*>(smem + L.off_kaddr);
  int* klab = reinterpret_cast<int*>(smem + L.off_klab);
  int* red = reinterpret_cast<int*>(smem + L.off_red);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int fr = lane & 15, g4 = lane >> 4;
  // XCD-aware order: consecutive logical blocks (the query splits of one
  // window-head, then neighbouring heads) land on the same XCD and L2.
  const int64_t nblk = gridDim.x;
  int64_t bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int64_t item = bid / L.qsplit;
  const int split = (int)(bid - item * L.qsplit);
  const int64_t w = item / a.heads;
  const int h = (int)(item - w * a.heads);
  const WinGeo& g = a.geo;
  const int N = a.N;
  const int mhw = g.Mh * g.Mw;
  const int wr = (int)(w % g.nws);
  const int wpl = g.nwh * g.nww;
  const int wt = wr / wpl, rem = wr - wt * wpl, wh = rem / g.nww, ww = rem - (rem / g.nww) * g.nww;
  const int rt0 = wt * g.P, rh0 = wh * g.Mh, rw0 = ww * g.Mw;
  const bf16_t* Qg = reinterpret_cast<const bf16_t*>(a.q) + item * N * 32;
  const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + item * N * 32;
  const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + item * N * 32;
  const bf16_t* Tg = reinterpret_cast<const bf16_t*>(a.table);
  const int rows = a.rel.rows, R = a.rel.R, Rw = a.rel.Rw;

  if (tid < 4) red[tid] = 0;
  __syncthreads();

  // ---- stage the head's table: reversed, * log2(e), fp16; then -inf zone
  float tmax = 0.f;
  for (int x = tid; x < L.tab_n; x += 256) {
    if (x < rows) {
      const float t = bf2f(Tg[(int64_t)(rows - 1 - x) * a.heads + h]);
      tmax = fmaxf(tmax, fabsf(t));
      tab[x] = (_Float16)(t * kLog2e);
    } else {
      tab[x] = (_Float16)(-INFINITY);
    }
  }
  // ---- K rows in slot order (slot k = 4m + i -> token (kt = 4a+i, kh, kw))
  float kmax2 = 0.f;
  for (int c = tid; c < L.NT * 64; c += 256) {
    const int kap = c >> 2, ch = c & 3;
    u32x4_t val = {0u, 0u, 0u, 0u};
    float sq = 0.f;
    if (kap < N) {
      const int m = kap >> 2, i = kap & 3;
      const int aa = m / mhw, r2 = m - aa * mhw, kh = r2 / g.Mw, kw = r2 - kh * g.Mw;
      const int n = ((4 * aa + i) * g.Mh + kh) * g.Mw + kw;
      val = *reinterpret_cast<const u32x4_t*>(Kg + n * 32 + ch * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bflo(val[e]), hi = bfhi(val[e]);
        sq += lo * lo + hi * hi;
      }
    }
    *reinterpret_cast<u32x4_t*>(Ks + kap * kKLD + ch * 8) = val;
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    kmax2 = fmaxf(kmax2, sq);
  }
  // ---- V^T in slot order, zero beyond N
  const int nslot_v = ((L.NT + 1) & ~1) * 16;
  for (int c = tid; c < nslot_v * 4; c += 256) {
    const int kap = c >> 2, ch = c & 3;
    u32x4_t val = {0u, 0u, 0u, 0u};
    if (kap < N) {
      const int m = kap >> 2, i = kap & 3;
      const int aa = m / mhw, r2 = m - aa * mhw, kh = r2 / g.Mw, kw = r2 - kh * g.Mw;
      const int n = ((4 * aa + i) * g.Mh + kh) * g.Mw + kw;
      val = *reinterpret_cast<const u32x4_t*>(Vg + n * 32 + ch * 8);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Vt[(ch * 8 + 2 * e) * L.VST + kap] = (bf16_t)(val[e] & 0xffffu);
      Vt[(ch * 8 + 2 * e + 1) * L.VST + kap] = (bf16_t)(val[e] >> 16);
    }
  }
  // ---- key groups: table byte offset of the group's first key, region label
  const int lab0 = slot_label_at(g, rt0, rh0, rw0);
  int anymask = 0;
  for (int m = tid; m < L.NT * 4; m += 256) {
    if (m < N / 4) {
      const int aa = m / mhw, r2 = m - aa * mhw, kh = r2 / g.Mw, kw = r2 - kh * g.Mw;
      kaddr[m] = 2 * (4 * aa * R + kh * Rw + kw);
      const int lab = slot_label_at(g, rt0 + 4 * aa, rh0 + kh, rw0 + kw);
      klab[m] = lab;
      anymask |= (lab != lab0);
    } else {
      kaddr[m] = 0;
      klab[m] = kDummyLab;
    }
  }
  atomicMax(&red[0], __float_as_int(kmax2));
  atomicMax(&red[1], __float_as_int(tmax));
  if (anymask) atomicOr(&red[2], 1);
  __syncthreads();
  const float kmax = sqrtf(__int_as_float(red[0]));
  const float tmx = __int_as_float(red[1]);
  const bool wmasked = a.use_mask && red[2] != 0;

  // ---- this wave's query tiles
  const int j0 = split * L.tps;
  const int j1 = min(L.QTT, j0 + L.tps);
  bool vq[kQT];
  bf16x8_t qreg[kQT];
  int qaddr[kQT], qlab[kQT];
  float mrow[kQT];
  f32x4_t acc0[kQT], acc1[kQT], accs[kQT];
  bool need_max = false;
  const int zone = 2 * rows;
  const int cq = rows - 1 - a.rel.centre;
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const int j = j0 + wv + kWaves * u;
    vq[u] = j < j1;
    const int qn = 16 * j + fr;
    const bool valid = vq[u] && qn < N;
    u32x4_t qv = {0u, 0u, 0u, 0u};
    int fq = 0;
    qlab[u] = kNoQueryLab;
    if (valid) {
      qv = *reinterpret_cast<const u32x4_t*>(Qg + qn * 32 + g4 * 8);
      const int pt = qn / mhw, r2 = qn - pt * mhw, ph = r2 / g.Mw, pw = r2 - ph * g.Mw;
      fq = pt * R + ph * Rw + pw;
      qlab[u] = slot_label_at(g, rt0 + pt, rh0 + ph, rw0 + pw);
    }
    qreg[u] = __builtin_bit_cast(bf16x8_t, qv);
    qaddr[u] = 2 * (cq - fq);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bflo(qv[e]), hi = bfhi(qv[e]);
      sq += lo * lo + hi * hi;
    }
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    const float bound = alpha * sqrtf(sq) * kmax + kLog2e * tmx;
    need_max |= valid && !(bound <= 90.f);
    mrow[u] = -INFINITY;
    acc0[u] = acc1[u] = accs[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bool wave_max = a.force_max || __ballot(need_max) != 0;
  const unsigned char* tabb = reinterpret_cast<const unsigned char*>(tab);
  const int R2 = 2 * R;
  if (!wave_max) {
    attn_pass<0>(Ks, Vt, tabb, kaddr, klab, L.NT, N, L.VST, R2, zone, wmasked, alpha, vq, qreg, qaddr, qlab,
                 mrow, acc0, acc1, accs);
  } else {
    attn_pass<1>(Ks, Vt, tabb, kaddr, klab, L.NT, N, L.VST, R2, zone, wmasked, alpha, vq, qreg, qaddr, qlab,
                 mrow, acc0, acc1, accs);
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
      float m = mrow[u];
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      mrow[u] = (m == -INFINITY) ? 0.f : m;
    }
    attn_pass<2>(Ks, Vt, tabb, kaddr, klab, L.NT, N, L.VST, R2, zone, wmasked, alpha, vq, qreg, qaddr, qlab,
                 mrow, acc0, acc1, accs);
  }

  // ---- normalise and write O (window order, head h at columns h*32)
  bf16_t* Og = reinterpret_cast<bf16_t*>(a.o);
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    if (!vq[u]) continue;
    const int qn = 16 * (j0 + wv + kWaves * u) + fr;
    if (qn >= N) continue;
    const float inv = 1.0f / accs[u][0];
    float o0[4], o1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { o0[i] = acc0[u][i] * inv; o1[i] = acc1[u][i] * inv; }
    const int64_t base = (w * N + qn) * (int64_t)a.C + h * 32;
    store4(Og, base + 4 * g4, o0);
    store4(Og, base + 16 + 4 * g4, o1);
  }
}

hipError_t attention_mfma(const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  const MfmaLaunch L = mfma_launch(a);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_mfma_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  const float alpha = kLog2e / sqrtf((float)a.d);
  AttnArgs ak = a;
  // VSWIN_ATTN_MAXPASS=1 makes every wave take the exact row-max pass (test
  // hook for the path that otherwise runs only for very large logits).
  if (const char* f = getenv("VSWIN_ATTN_MAXPASS")) ak.force_max = atoi(f) != 0;
  hipLaunchKernelGGL(attn_mfma_kernel, dim3((unsigned)(items * L.qsplit)), dim3(256), L.lds, st, ak, L, alpha);
  return hipGetLastError();
}

}  // namespace vswin
