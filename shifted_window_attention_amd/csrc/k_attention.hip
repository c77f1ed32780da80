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
constexpr int kWaves = 4;         // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kQSplit = 2;        // workgroups per (window, head): query tiles split in halves
constexpr int kKLD = 40;          // K row pitch in the LDS ring (elements): 80 bytes
constexpr int kVLD = 36;          // V^T row pitch in the LDS ring (elements): 72 bytes
constexpr int kRing = 32 * kKLD + 32 * kVLD;   // one 32-key step: K rows + V^T columns
constexpr int kTabPer = 12;       // table entries staged per thread
constexpr int kKNorm = 8;         // 16-byte K chunks per thread for the key norms (N <= 512)
constexpr int kDummyLab = 0x7fff0000;
constexpr int kNoQueryLab = 0x7ffe0000;

int attention_table_stride(const RelTab& rel) { return (rel.rows + 3 * rel.R + 8 + 7) & ~7; }

size_t attention_workspace_bytes(const RelTab&, int) { return 0; }

struct MfmaLaunch {
  int NT;         // key tiles of 16
  int NP;         // 32-key steps (pairs of tiles), padded with dummy slots
  int QTT;        // query tiles of 16
  int tstride;    // fp16 table entries per head (table + -inf zone)
  size_t lds, off_ring, off_kaddr, off_klab, off_red;
};

static MfmaLaunch mfma_launch(const AttnArgs& a) {
  MfmaLaunch L{};
  L.NT = (a.N + 15) / 16;
  L.NP = (L.NT + 1) / 2;
  L.QTT = L.NT;
  L.tstride = attention_table_stride(a.rel);
  size_t off = ((size_t)L.tstride * 2 + 15) & ~(size_t)15;
  L.off_ring = off;
  off += (size_t)2 * kRing * 2;
  L.off_kaddr = off;
  off += (size_t)(L.NP * 8) * 4;
  L.off_klab = off;
  off += (size_t)(L.NP * 8) * 4;
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
  if (attention_table_stride(a.rel) > kTabPer * kThreads) return false;
  return mfma_launch(a).lds <= 64 * 1024;
}

template <int QT>
struct QState {
  bf16x8_t q[QT];       // B operand: 8 head-dim values of this lane's query
  int qaddr[QT];        // byte offset of the query's reversed-table base
  int qlab[QT];         // region label of the query
  float mrow[QT];       // row max (two-pass mode)
  f32x4_t o0[QT], o1[QT], os[QT];   // O^T (d 0-15, d 16-31) and row sums
};

// One 32-key step from ring buffer `rb` for the QT query tiles of the wave,
// in one basic block so the tiles' MFMA, LDS and VALU work interleave.
//   MODE 0: P = exp2(x); 1: track the row max of x; 2: P = exp2(x - max).
//   SEL: per key group, point masked / dummy groups at the -inf zone.
//   R2C: byte stride of one temporal offset in the table (0 = runtime R2).
template <int MODE, bool SEL, int QT, int R2C>
__device__ __forceinline__ void attn_step(int p, const bf16_t* __restrict__ rb,
                                          const unsigned char* __restrict__ tabb, const int* __restrict__ kaddr,
                                          const int* __restrict__ klab, int R2r, int zone, float alpha,
                                          const bf16x8_t& ones, QState<QT>& st) {
  const int R2 = R2C ? R2C : R2r;
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const bf16_t* Kb = rb;
  const bf16_t* Vb = rb + 32 * kKLD;
  const bf16x8_t kA = *reinterpret_cast<const bf16x8_t*>(Kb + fr * kKLD + g4 * 8);
  const bf16x8_t kB = *reinterpret_cast<const bf16x8_t*>(Kb + (16 + fr) * kKLD + g4 * 8);
  const int gA = kaddr[8 * p + g4];
  const int gB = kaddr[8 * p + 4 + g4];
  int lA = 0, lB = 0;
  if (SEL) {
    lA = klab[8 * p + g4];
    lB = klab[8 * p + 4 + g4];
  }
  bf16x8_t vA0 = bf16x8_t{}, vA1 = bf16x8_t{};
  if (MODE != 1) {
    const u32x2_t* p0 = reinterpret_cast<const u32x2_t*>(Vb + fr * kVLD + 4 * g4);
    const u32x2_t* p1 = reinterpret_cast<const u32x2_t*>(Vb + (fr + 16) * kVLD + 4 * g4);
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

// Per-thread share of one 32-key step: threads 0-127 one 16-byte chunk of the
// K rows, threads 128-255 one of the V^T columns (two 8-byte halves).
struct StepChunk {
  u32x4_t v;
};

struct StreamCtx {
  const bf16_t* Kg;     // (N, 32) slot order
  const bf16_t* Vg;     // (32, N) slot order
  bf16_t* ring;         // 2 x kRing elements
  const unsigned char* tabb;
  const int* kaddr;
  const int* klab;
  int N, NP, R2, zone;
  float alpha;
};

__device__ __forceinline__ StepChunk load_step(const StreamCtx& c, int p) {
  const int t = threadIdx.x;
  StepChunk r;
  r.v = u32x4_t{0u, 0u, 0u, 0u};
  if (p >= c.NP) return r;
  if (t < 128) {
    const int row = 32 * p + (t >> 2);
    if (row < c.N) r.v = *reinterpret_cast<const u32x4_t*>(c.Kg + row * 32 + (t & 3) * 8);
  } else {
    const int d = (t - 128) >> 2, k0 = 32 * p + ((t - 128) & 3) * 8;
    const bf16_t* src = c.Vg + d * c.N + k0;
    if (k0 < c.N) {
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src);
      r.v[0] = lo[0]; r.v[1] = lo[1];
    }
    if (k0 + 4 < c.N) {
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(src + 4);
      r.v[2] = hi[0]; r.v[3] = hi[1];
    }
  }
  return r;
}

__device__ __forceinline__ void store_step(const StreamCtx& c, int buf, const StepChunk& r) {
  const int t = threadIdx.x;
  bf16_t* rb = c.ring + buf * kRing;
  if (t < 128) {
    *reinterpret_cast<u32x4_t*>(rb + (t >> 2) * kKLD + (t & 3) * 8) = r.v;
  } else {
    const int d = (t - 128) >> 2, k0 = ((t - 128) & 3) * 8;
    u32x2_t lo, hi;
    lo[0] = r.v[0]; lo[1] = r.v[1]; hi[0] = r.v[2]; hi[1] = r.v[3];
    *reinterpret_cast<u32x2_t*>(rb + 32 * kKLD + d * kVLD + k0) = lo;
    *reinterpret_cast<u32x2_t*>(rb + 32 * kKLD + d * kVLD + k0 + 4) = hi;
  }
}

// One pass over all keys.  Step p computes from ring buffer p % 2 while the
// chunk of step p + 1 waits in registers and step p + 2 is being fetched.
// Entry: step 0 in ring buffer 0 (visible to all waves), step 1 in `next`.
template <int MODE, bool MASKED, int QT, int R2C>
__device__ __forceinline__ void attn_stream(const StreamCtx& c, StepChunk next, const bf16x8_t& ones,
                                            QState<QT>& st) {
  const int nclean = c.N / 32;   // steps whose 32 slots are all real keys
  for (int p = 0; p < c.NP; ++p) {
    const StepChunk fut = load_step(c, p + 2);
    const bf16_t* rb = c.ring + (p & 1) * kRing;
    if (p < nclean)
      attn_step<MODE, MASKED, QT, R2C>(p, rb, c.tabb, c.kaddr, c.klab, c.R2, c.zone, c.alpha, ones, st);
    else
      attn_step<MODE, true, QT, R2C>(p, rb, c.tabb, c.kaddr, c.klab, c.R2, c.zone, c.alpha, ones, st);
    if (p + 1 < c.NP) store_step(c, (p + 1) & 1, next);
    next = fut;
    __syncthreads();
  }
}

// One workgroup per (window, head, query half).  Inputs (slot order, see
// slot_to_natural): q, k (item, N, 32); v transposed (item, 32, N); table
// (rows, heads) bf16.  Output rows of o in slot order.  R2C: compile-time
// table stride (0 = runtime).
template <int R2C>
__global__ void __launch_bounds__(kThreads)
attn_mfma_kernel(const AttnArgs a, const MfmaLaunch L, const float alpha) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* tab = reinterpret_cast<_Float16*>(smem);
  bf16_t* ring = reinterpret_cast<bf16_t*>(smem + L.off_ring);
  int* kaddr = reinterpret_cast<int*>(smem + L.off_kaddr);
  int* klab = reinterpret_cast<int*>(smem + L.off_klab);
  int* red = reinterpret_cast<int*>(smem + L.off_red);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, g4 = lane >> 4;
  // XCD-aware order: consecutive logical blocks (the halves of one window-head,
  // then neighbouring heads and windows) land on the same XCD and its L2.
  const int64_t nblk = gridDim.x;
  int64_t bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int item = (int)(bid / kQSplit);
  const int split = (int)(bid - (int64_t)item * kQSplit);
  const int w = item / a.heads;
  const int h = item - w * a.heads;
  const WinGeo& g = a.geo;
  const int N = a.N;
  const int mhw = g.Mh * g.Mw;
  const int wr = w % g.nws;
  const int wpl = g.nwh * g.nww;
  const int wt = wr / wpl, rem = wr - wt * wpl, wh = rem / g.nww, ww = rem - (rem / g.nww) * g.nww;
  const int rt0 = wt * g.P, rh0 = wh * g.Mh, rw0 = ww * g.Mw;
  const bf16_t* Qg = reinterpret_cast<const bf16_t*>(a.q) + (int64_t)item * N * 32;
  const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + (int64_t)item * N * 32;
  const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + (int64_t)item * N * 32;
  const bf16_t* Tg = reinterpret_cast<const bf16_t*>(a.table);
  const int R = a.rel.R, Rw = a.rel.Rw;

  StreamCtx c;
  c.Kg = Kg; c.Vg = Vg; c.ring = ring;
  c.tabb = reinterpret_cast<const unsigned char*>(tab);
  c.kaddr = kaddr; c.klab = klab;
  c.N = N; c.NP = L.NP; c.R2 = 2 * R; c.zone = 2 * a.rel.rows; c.alpha = alpha;

  if (tid < 4) red[tid] = 0;

  // ---- one batch of global loads: table column, K rows (norms), the first
  // two key steps and this wave's query tiles
  uint16_t tv[kTabPer];
#pragma unroll
  for (int i = 0; i < kTabPer; ++i) {
    const int x = tid + kThreads * i;
    tv[i] = 0;
    if (x < a.rel.rows) tv[i] = Tg[(int64_t)(a.rel.rows - 1 - x) * a.heads + h];
  }
  float kmax2 = 0.f;
  {
    u32x4_t kv[kKNorm];
#pragma unroll
    for (int i = 0; i < kKNorm; ++i) {
      const int cc = tid + kThreads * i;
      kv[i] = u32x4_t{0u, 0u, 0u, 0u};
      if ((cc >> 2) < N) kv[i] = *reinterpret_cast<const u32x4_t*>(Kg + (cc >> 2) * 32 + (cc & 3) * 8);
    }
#pragma unroll
    for (int i = 0; i < kKNorm; ++i) {
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bflo(kv[i][e]), hi = bfhi(kv[i][e]);
        sq += lo * lo + hi * hi;
      }
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
      kmax2 = fmaxf(kmax2, sq);
    }
  }
  const StepChunk s0 = load_step(c, 0);
  const StepChunk s1 = load_step(c, 1);
  const int tps = (L.QTT + kQSplit - 1) / kQSplit;
  const int jb = split * tps;                          // first query tile of this workgroup
  const int jn = min(L.QTT, jb + tps) - jb;            // query tiles of this workgroup
  const int mine = max(0, (jn - wv + kWaves - 1) / kWaves);   // <= kQT for N <= 512

  // ---- geometry of the key groups (no memory traffic)
  int anymask = 0;
  const int lab0 = slot_label_at(g, rt0, rh0, rw0);
  for (int m = tid; m < L.NP * 8; m += kThreads) {
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
  // ---- LDS stores: table reversed and scaled by log2(e) (fp16), -inf zone
  float tmaxl = 0.f;
#pragma unroll
  for (int i = 0; i < kTabPer; ++i) {
    const int x = tid + kThreads * i;
    if (x < L.tstride) {
      const bool real = x < a.rel.rows;
      const float t = bf2f(tv[i]);
      tmaxl = real ? fmaxf(tmaxl, fabsf(t)) : tmaxl;
      tab[x] = real ? (_Float16)(t * kLog2e) : (_Float16)(-INFINITY);
    }
  }
  store_step(c, 0, s0);
  __syncthreads();      // red[] cleared before the atomics below
  atomicMax(&red[0], __float_as_int(kmax2));
  atomicMax(&red[2], __float_as_int(tmaxl * kLog2e));
  if (anymask) atomicOr(&red[1], 1);
  __syncthreads();
  const float kmax = sqrtf(__int_as_float(red[0]));
  const float tmx = __int_as_float(red[2]);
  const bool wmasked = a.use_mask && red[1] != 0;

  // ---- this wave's query tiles jb + wv, jb + wv + 4, ... (at most kQT)
  QState<kQT> st;
  bool need_max = false;
  const int cq = a.rel.rows - 1 - a.rel.centre;
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const int qs = 16 * (jb + wv + kWaves * u) + fr;
    const bool valid = u < mine && qs < N;
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
    need_max |= valid && !(alpha * sqrtf(sq) * kmax + tmx <= 90.f);
    st.mrow[u] = -INFINITY;
    st.o0[u] = st.o1[u] = st.os[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  // the whole workgroup takes the same passes (they share the ring barriers)
  const bool wg_max = a.force_max || __syncthreads_or(need_max ? 1 : 0);
  if (!wg_max) {
    if (wmasked) attn_stream<0, true, kQT, R2C>(c, s1, ones, st);
    else attn_stream<0, false, kQT, R2C>(c, s1, ones, st);
  } else {
    if (wmasked) attn_stream<1, true, kQT, R2C>(c, s1, ones, st);
    else attn_stream<1, false, kQT, R2C>(c, s1, ones, st);
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
      float m = st.mrow[u];
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      st.mrow[u] = (m == -INFINITY) ? 0.f : m;
    }
    const StepChunk t0 = load_step(c, 0);
    const StepChunk t1 = load_step(c, 1);
    store_step(c, 0, t0);
    __syncthreads();
    if (wmasked) attn_stream<2, true, kQT, R2C>(c, t1, ones, st);
    else attn_stream<2, false, kQT, R2C>(c, t1, ones, st);
  }

  // ---- normalise and write O^T fragments (rows in slot order)
  bf16_t* Og = reinterpret_cast<bf16_t*>(a.o);
#pragma unroll
  for (int u = 0; u < kQT; ++u) {
    const int qs = 16 * (jb + wv + kWaves * u) + fr;
    if (u >= mine || qs >= N) continue;
    const float inv = 1.0f / st.os[u][0];
    float o0[4], o1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { o0[i] = st.o0[u][i] * inv; o1[i] = st.o1[u][i] * inv; }
    const int64_t base = ((int64_t)w * N + qs) * a.C + h * 32;
    store4(Og, base + 4 * g4, o0);
    store4(Og, base + 16 + 4 * g4, o1);
  }
}

hipError_t attention_mfma(const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  const MfmaLaunch L = mfma_launch(a);
  const float alpha = kLog2e / sqrtf((float)a.d);
  AttnArgs ak = a;
  // VSWIN_ATTN_MAXPASS=1 makes every workgroup take the exact row-max pass
  // (test hook for the path that otherwise runs only for very large logits).
  if (const char* f = getenv("VSWIN_ATTN_MAXPASS")) ak.force_max = atoi(f) != 0;
  const dim3 grid((unsigned)(items * kQSplit));
  // the (8,7,7) window's table (R = 13 * 13) gets compile-time read offsets
  if (2 * a.rel.R == 338)
    hipLaunchKernelGGL(attn_mfma_kernel<338>, grid, dim3(kThreads), L.lds, st, ak, L, alpha);
  else
    hipLaunchKernelGGL(attn_mfma_kernel<0>, grid, dim3(kThreads), L.lds, st, ak, L, alpha);
  return hipGetLastError();
}

}  // namespace vswin
