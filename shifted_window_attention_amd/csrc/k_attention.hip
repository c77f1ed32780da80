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
constexpr int kQT = 4;            // query tiles of 16 a wave carries at once
constexpr int kWaves = 4;
constexpr int kKLD = 40;          // K row pitch in LDS (elements): 80 bytes
constexpr int kDummyLab = 0x7fff0000;
constexpr int kNoQueryLab = 0x7ffe0000;

int attention_table_stride(const RelTab& rel) { return (rel.rows + 3 * rel.R + 8 + 7) & ~7; }

size_t attention_workspace_bytes(const RelTab& rel, int heads) {
  return ((size_t)heads * attention_table_stride(rel) * 2 + 255) / 256 * 256 + ((size_t)heads * 4 + 255) / 256 * 256;
}

// Per head: fp16 table reversed and scaled by log2(e), followed by a -inf zone
// of 3R + 8 entries; tmax[h] = log2(e) * max |T|.
__global__ void __launch_bounds__(256) attn_prep_kernel(const bf16_t* __restrict__ table, _Float16* __restrict__ tab16,
                                                        float* __restrict__ tmax, int rows, int heads, int stride) {
  __shared__ float red[4];
  const int h = blockIdx.x;
  float m = 0.f;
  for (int x = threadIdx.x; x < stride; x += 256) {
    if (x < rows) {
      const float t = bf2f(table[(int64_t)(rows - 1 - x) * heads + h]);
      m = fmaxf(m, fabsf(t));
      tab16[(int64_t)h * stride + x] = (_Float16)(t * kLog2e);
    } else {
      tab16[(int64_t)h * stride + x] = (_Float16)(-INFINITY);
    }
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) tmax[h] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) * kLog2e;
}

struct MfmaLaunch {
  int NT;         // key tiles of 16 (slots padded to NT*16)
  int NVS;        // V^T columns staged (NT rounded up to even, *16)
  int VST;        // V^T row pitch in LDS (elements): (VST/2) mod 32 = 2*odd
  int QTT;        // query tiles of 16
  int tstride;    // fp16 table entries per head
  size_t lds, off_vt, off_tab, off_kaddr, off_klab, off_red;
};

static MfmaLaunch mfma_launch(const AttnArgs& a) {
  MfmaLaunch L{};
  L.NT = (a.N + 15) / 16;
  L.NVS = ((L.NT + 1) & ~1) * 16;
  L.VST = L.NVS + 4;
  L.QTT = L.NT;
  L.tstride = attention_table_stride(a.rel);
  size_t off = (size_t)L.NT * 16 * kKLD * 2;
  L.off_vt = off;
  off += (size_t)32 * L.VST * 2;
  off = (off + 15) & ~(size_t)15;
  L.off_tab = off;
  off += (size_t)L.tstride * 2;
  L.off_kaddr = off;
  off += (size_t)(L.NT * 4 + 4) * 4;
  L.off_klab = off;
  off += (size_t)(L.NT * 4 + 4) * 4;
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

template <int QT>
struct QState {
  bf16x8_t q[QT];       // B operand: 8 head-dim values of this lane's query
  int qaddr[QT];        // byte offset of the query's reversed-table base
  int qlab[QT];         // region label of the query
  float mrow[QT];       // row max (two-pass mode)
  f32x4_t o0[QT], o1[QT], os[QT];   // O^T (d 0-15, d 16-31) and row sums
};

// One pair of key tiles (32 slots) for the QT query tiles of the wave, all in
// one basic block so the tiles' MFMA, LDS and VALU work interleave.
//   MODE 0: P = exp2(x); 1: track the row max of x; 2: P = exp2(x - max).
//   SEL: per key group, point masked / dummy groups at the -inf zone.
//   TAIL: the pair may end in dummy slots or lack its second tile.
//   R2C: byte stride of one temporal offset in the table (0 = runtime R2).
template <int MODE, bool SEL, bool TAIL, int QT, int R2C>
__device__ __forceinline__ void attn_pair(int tp, int NT, const bf16_t* __restrict__ Ks,
                                          const bf16_t* __restrict__ Vt, int VST,
                                          const unsigned char* __restrict__ tabb, const int* __restrict__ kaddr,
                                          const int* __restrict__ klab, int R2r, int zone, float alpha,
                                          const bf16x8_t& ones, QState<QT>& st) {
  const int R2 = R2C ? R2C : R2r;
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const bool hasB = !TAIL || tp + 1 < NT;
  const bf16x8_t kA = *reinterpret_cast<const bf16x8_t*>(Ks + (16 * tp + fr) * kKLD + g4 * 8);
  bf16x8_t kB = bf16x8_t{};
  if (hasB) kB = *reinterpret_cast<const bf16x8_t*>(Ks + (16 * tp + 16 + fr) * kKLD + g4 * 8);
  const int gA = kaddr[4 * tp + g4];
  const int gB = kaddr[4 * tp + 4 + g4];
  int lA = 0, lB = 0;
  if (SEL) {
    lA = klab[4 * tp + g4];
    lB = hasB ? klab[4 * tp + 4 + g4] : kDummyLab;
  }
  bf16x8_t vA0 = bf16x8_t{}, vA1 = bf16x8_t{};
  if (MODE != 1) {
    const u32x2_t* p0 = reinterpret_cast<const u32x2_t*>(Vt + fr * VST + 16 * tp + 4 * g4);
    const u32x2_t* p1 = reinterpret_cast<const u32x2_t*>(Vt + (fr + 16) * VST + 16 * tp + 4 * g4);
    const u32x2_t a0 = p0[0], b0 = p0[4], a1 = p1[0], b1 = p1[4];   // +16 slots = +32 bytes
    u32x4_t t0, t1;
    t0[0] = a0[0]; t0[1] = a0[1]; t0[2] = b0[0]; t0[3] = b0[1];
    t1[0] = a1[0]; t1[1] = a1[1]; t1[2] = b1[0]; t1[3] = b1[1];
    vA0 = __builtin_bit_cast(bf16x8_t, t0);
    vA1 = __builtin_bit_cast(bf16x8_t, t1);
  }
  f32x4_t sA[QT], sB[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    sA[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, st.q[u], zero4, 0, 0, 0);
    sB[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kB, st.q[u], zero4, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    int adA = st.qaddr[u] + gA, adB = st.qaddr[u] + gB;
    if (SEL) {
      adA = (lA == st.qlab[u]) ? adA : zone;
      adB = (lB == st.qlab[u]) ? adB : zone;
    }
    float xA[4], xB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xA[i] = __builtin_fmaf(sA[u][i], alpha, (float)*reinterpret_cast<const _Float16*>(tabb + adA + i * R2));
      xB[i] = __builtin_fmaf(sB[u][i], alpha, (float)*reinterpret_cast<const _Float16*>(tabb + adB + i * R2));
    }
    if (MODE == 1) {
      float m = st.mrow[u];
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(xA[i], xB[i]));
      st.mrow[u] = m;
    } else {
      float pA[4], pB[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pA[i] = __builtin_amdgcn_exp2f(MODE == 2 ? xA[i] - st.mrow[u] : xA[i]);
        pB[i] = __builtin_amdgcn_exp2f(MODE == 2 ? xB[i] - st.mrow[u] : xB[i]);
      }
      u32x4_t pk;
      pk[0] = pack_bf16x2(pA[0], pA[1]);
      pk[1] = pack_bf16x2(pA[2], pA[3]);
      pk[2] = pack_bf16x2(pB[0], pB[1]);
      pk[3] = pack_bf16x2(pB[2], pB[3]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
      st.o0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA0, pb, st.o0[u], 0, 0, 0);
      st.o1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA1, pb, st.o1[u], 0, 0, 0);
      st.os[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, st.os[u], 0, 0, 0);
    }
  }
}

struct AttnCtx {
  const bf16_t* Ks;
  const bf16_t* Vt;
  const unsigned char* tabb;
  const int* kaddr;
  const int* klab;
  int N, NT, VST, R2, zone;
  float alpha;
};

template <int MODE, bool MASKED, int QT, int R2C>
__device__ __forceinline__ void attn_pass(const AttnCtx& c, const bf16x8_t& ones, QState<QT>& st) {
  const int nclean = c.N / 32;   // pairs whose 32 slots are all real keys
  for (int pi = 0; pi < nclean; ++pi)
    attn_pair<MODE, MASKED, false, QT, R2C>(2 * pi, c.NT, c.Ks, c.Vt, c.VST, c.tabb, c.kaddr, c.klab, c.R2,
                                            c.zone, c.alpha, ones, st);
  if (2 * nclean < c.NT)
    attn_pair<MODE, true, true, QT, R2C>(2 * nclean, c.NT, c.Ks, c.Vt, c.VST, c.tabb, c.kaddr, c.klab, c.R2,
                                         c.zone, c.alpha, ones, st);
}

// Process query tiles j0, j0 + step, ... (QT of them) of one wave.
template <int QT, int R2C>
__device__ __forceinline__ void attn_tiles(const AttnArgs& a, const AttnCtx& c, int j0, int step, int64_t w, int h,
                                           int rt0, int rh0, int rw0, float kmax, float tmx, bool wmasked,
                                           const bf16_t* Qg, bf16_t* Og) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const WinGeo& g = a.geo;
  const int mhw = g.Mh * g.Mw;
  const int R = a.rel.R, Rw = a.rel.Rw;
  const int cq = a.rel.rows - 1 - a.rel.centre;
  QState<QT> st;
  bool need_max = false;
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qs = 16 * (j0 + step * u) + fr;
    const bool valid = qs < c.N;
    u32x4_t qv = {0u, 0u, 0u, 0u};
    int fq = 0;
    st.qlab[u] = kNoQueryLab;
    if (valid) {
      qv = *reinterpret_cast<const u32x4_t*>(Qg + qs * 32 + g4 * 8);
      const int m = qs >> 2, i = qs & 3;
      const int aa = m / mhw, r2 = m - aa * mhw, kh = r2 / g.Mw, kw = r2 - kh * g.Mw;
      fq = (4 * aa + i) * R + kh * Rw + kw;
      st.qlab[u] = slot_label_at(g, rt0 + 4 * aa + i, rh0 + kh, rw0 + kw);
    }
    st.q[u] = __builtin_bit_cast(bf16x8_t, qv);
    st.qaddr[u] = 2 * (cq - fq);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bflo(qv[e]), hi = bfhi(qv[e]);
      sq += lo * lo + hi * hi;
    }
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    need_max |= valid && !(c.alpha * sqrtf(sq) * kmax + tmx <= 90.f);
    st.mrow[u] = -INFINITY;
    st.o0[u] = st.o1[u] = st.os[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  const bool wave_max = a.force_max || __ballot(need_max) != 0;
  if (wave_max) {
    if (wmasked) attn_pass<1, true, QT, R2C>(c, ones, st);
    else attn_pass<1, false, QT, R2C>(c, ones, st);
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      float m = st.mrow[u];
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      st.mrow[u] = (m == -INFINITY) ? 0.f : m;
    }
    if (wmasked) attn_pass<2, true, QT, R2C>(c, ones, st);
    else attn_pass<2, false, QT, R2C>(c, ones, st);
  } else {
    if (wmasked) attn_pass<0, true, QT, R2C>(c, ones, st);
    else attn_pass<0, false, QT, R2C>(c, ones, st);
  }
  // normalise and write O^T fragments (rows in slot order)
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qs = 16 * (j0 + step * u) + fr;
    if (qs >= c.N) continue;
    const float inv = 1.0f / st.os[u][0];
    float o0[4], o1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { o0[i] = st.o0[u][i] * inv; o1[i] = st.o1[u][i] * inv; }
    const int64_t base = (w * c.N + qs) * (int64_t)a.C + h * 32;
    store4(Og, base + 4 * g4, o0);
    store4(Og, base + 16 + 4 * g4, o1);
  }
}

// One workgroup per (window, head).  Inputs (slot order, see slot_to_natural):
// q, k (item, N, 32); v transposed (item, 32, N); tab16 / tmax from the prep
// kernel.  Output rows of o in slot order.  R2C: compile-time table stride.
template <int R2C>
__global__ void __launch_bounds__(256) attn_mfma_kernel(const AttnArgs a, const MfmaLaunch L, const float alpha) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem);
  bf16_t* Vt = reinterpret_cast<bf16_t*>(smem + L.off_vt);
  _Float16* tab = reinterpret_cast<_Float16*>(smem + L.off_tab);
  int* kaddr = reinterpret_cast<int*>(smem + L.off_kaddr);
  int* klab = reinterpret_cast<int*>(smem + L.off_klab);
  int* red = reinterpret_cast<int*>(smem + L.off_red);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: consecutive logical blocks (neighbouring heads of one
  // window, then neighbouring windows) land on the same XCD.
  const int64_t nblk = gridDim.x;
  int64_t item = blockIdx.x;
  if ((nblk & 7) == 0) item = (item & 7) * (nblk >> 3) + (item >> 3);
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
  const _Float16* Tg = reinterpret_cast<const _Float16*>(a.tab16) + (int64_t)h * L.tstride;
  const int R = a.rel.R, Rw = a.rel.Rw;

  if (tid < 4) red[tid] = 0;
  __syncthreads();

  // ---- stage: table (16-byte copies), K rows, V^T rows, key-group info.
  // Loads are issued in batches before their LDS stores so that each thread
  // has several global requests in flight.
  for (int c0 = 0; c0 < L.tstride / 8; c0 += 256 * 4) {
    u32x4_t buf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + tid + 256 * i;
      if (c < L.tstride / 8) buf[i] = reinterpret_cast<const u32x4_t*>(Tg)[c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + tid + 256 * i;
      if (c < L.tstride / 8) reinterpret_cast<u32x4_t*>(tab)[c] = buf[i];
    }
  }
  float kmax2 = 0.f;
  for (int c0 = 0; c0 < L.NT * 64; c0 += 256 * 8) {
    u32x4_t buf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + tid + 256 * i;
      buf[i] = u32x4_t{0u, 0u, 0u, 0u};
      if ((c >> 2) < N) buf[i] = *reinterpret_cast<const u32x4_t*>(Kg + (c >> 2) * 32 + (c & 3) * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = c0 + tid + 256 * i;
      if (c0 + 256 * i >= L.NT * 64) break;      // depends on the batch index only: wave uniform
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bflo(buf[i][e]), hi = bfhi(buf[i][e]);
        sq += lo * lo + hi * hi;
      }
      if (c < L.NT * 64) *reinterpret_cast<u32x4_t*>(Ks + (c >> 2) * kKLD + (c & 3) * 8) = buf[i];
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
      kmax2 = fmaxf(kmax2, sq);
    }
  }
  const int c4 = L.NVS / 4;
  for (int c0 = 0; c0 < 32 * c4; c0 += 256 * 16) {
    u32x2_t buf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = c0 + tid + 256 * i;
      const int d = c / c4, k4 = (c - d * c4) * 4;
      buf[i] = u32x2_t{0u, 0u};
      if (c < 32 * c4 && k4 < N) buf[i] = *reinterpret_cast<const u32x2_t*>(Vg + d * N + k4);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = c0 + tid + 256 * i;
      const int d = c / c4, k4 = (c - d * c4) * 4;
      if (c < 32 * c4) *reinterpret_cast<u32x2_t*>(Vt + d * L.VST + k4) = buf[i];
    }
  }
  int anymask = 0;
  const int lab0 = slot_label_at(g, rt0, rh0, rw0);
  for (int m = tid; m < L.NT * 4 + 4; m += 256) {
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
  if (anymask) atomicOr(&red[1], 1);
  __syncthreads();
  const float kmax = sqrtf(__int_as_float(red[0]));
  const float tmx = a.tmax[h];
  const bool wmasked = a.use_mask && red[1] != 0;
  AttnCtx c;
  c.Ks = Ks; c.Vt = Vt; c.tabb = reinterpret_cast<const unsigned char*>(tab);
  c.kaddr = kaddr; c.klab = klab;
  c.N = N; c.NT = L.NT; c.VST = L.VST; c.R2 = 2 * R; c.zone = 2 * a.rel.rows; c.alpha = alpha;
  bf16_t* Og = reinterpret_cast<bf16_t*>(a.o);

  // ---- query tiles wv, wv + 4, wv + 8, ... in chunks of at most 4
  const int mine = (L.QTT - wv + kWaves - 1) / kWaves;
  for (int u0 = 0; u0 < mine; u0 += kQT) {
    const int n = min(kQT, mine - u0);
    const int j0 = wv + kWaves * u0;
    switch (n) {
      case 4: attn_tiles<4, R2C>(a, c, j0, kWaves, w, h, rt0, rh0, rw0, kmax, tmx, wmasked, Qg, Og); break;
      case 3: attn_tiles<3, R2C>(a, c, j0, kWaves, w, h, rt0, rh0, rw0, kmax, tmx, wmasked, Qg, Og); break;
      case 2: attn_tiles<2, R2C>(a, c, j0, kWaves, w, h, rt0, rh0, rw0, kmax, tmx, wmasked, Qg, Og); break;
      default: attn_tiles<1, R2C>(a, c, j0, kWaves, w, h, rt0, rh0, rw0, kmax, tmx, wmasked, Qg, Og); break;
    }
  }
}

hipError_t attention_mfma(const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  const MfmaLaunch L = mfma_launch(a);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_mfma_kernel<338>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    hipFuncSetAttribute((const void*)attn_mfma_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL(attn_prep_kernel, dim3(a.heads), dim3(256), 0, st, (const bf16_t*)a.table,
                     (_Float16*)a.tab16, (float*)a.tmax, a.rel.rows, a.heads, L.tstride);
  const float alpha = kLog2e / sqrtf((float)a.d);
  AttnArgs ak = a;
  // VSWIN_ATTN_MAXPASS=1 makes every wave take the exact row-max pass (test
  // hook for the path that otherwise runs only for very large logits).
  if (const char* f = getenv("VSWIN_ATTN_MAXPASS")) ak.force_max = atoi(f) != 0;
  // the (8,7,7) window's table (R = 13 * 13) gets compile-time read offsets
  if (2 * a.rel.R == 338)
    hipLaunchKernelGGL(attn_mfma_kernel<338>, dim3((unsigned)items), dim3(256), L.lds, st, ak, L, alpha);
  else
    hipLaunchKernelGGL(attn_mfma_kernel<0>, dim3((unsigned)items), dim3(256), L.lds, st, ak, L, alpha);
  return hipGetLastError();
}

}  // namespace vswin
