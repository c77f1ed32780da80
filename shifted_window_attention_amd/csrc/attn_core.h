// Device core of the MFMA window attention (bf16, head_dim 32), shared by the
// attention kernel on prepared q, k, V^T (k_attn_mfma.hip) and the kernel
// that also computes them from the tokens (k_attn_fused.hip): the launch
// geometry (A5), the per-window label and offset tables, and the 32-key step
// and pass of a wave's query tiles.  The layouts are described at the top of
// k_attn_mfma.hip.
#pragma once

#include "vswin_kernels.h"

#include <math.h>

#include <type_traits>

namespace vswin {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxWaves = 16;
constexpr int kMaxTab = 4096;     // table 4-tuples held in LDS at most
constexpr int kDummyLab = 0x7fff0000;
// per-key labels: one byte per key of the group (region labels are < 27, pads
// 255), dummy keys 0xfe, which no query carries
constexpr uint32_t kDummyLab4 = 0xfefefefeu;
constexpr size_t kLdsMax = 160 * 1024;

// Temporal stride of the scalar bias table for the 7 x 7 spatial window
// (R = 169): a compile-time constant, so a 4-tuple is two ds_read2_b32.
constexpr int kBigRp = 180;

// W waves per workgroup; a wave carries at most QTM query tiles of a window,
// in groups of at most 4.  BIG: windows of more than kMfmaMaxN tokens, with
// the scalar bias table and one K / V^T buffer.  M100: pairs of different
// regions get -100 added to their logit instead of being excluded.  PERKEY:
// the 4 keys of a key group may lie in different regions (a temporal region
// boundary inside a group, e.g. window 4 with temporal shift 2); their labels
// are compared one by one and masked keys get P = 0.
template <int W, int QTM, bool BIG = false, bool M100 = false, bool PERKEY = false>
struct Cfg {
  static constexpr int kWaves = W;
  static constexpr int kQTM = QTM;
  static constexpr bool kBig = BIG;
  static constexpr bool kM100 = M100;
  static constexpr bool kPerKey = PERKEY;
  static_assert(!(M100 && PERKEY), "the -100 mask needs group-uniform labels");
  static constexpr int kTabEs = BIG ? 4 : 16;   // bytes per table index step
  static constexpr int kThreads = 64 * W;
  static_assert(((BIG ? kMfmaBigN : kMfmaMaxN) / 16 + W - 1) / W <= QTM, "a wave's tiles of one window exceed QTM");
  static_assert(QTM <= 4 || QTM == 8, "tile groups of 4");
  static_assert(W <= kMaxWaves, "too many waves");
};

struct A5 {
  int N, NPAD, NP, QTT, NB;
  int pitch_v;                // V^T row pitch (16-byte chunks)
  int Rp, Rw, R, TD, TH, A;   // table: temporal stride R', row stride, true R, extents, query base
  int TS4;                    // 16-byte table entries per head
  int zone;                   // LDS byte address of the -inf 4-tuple
  int nW, heads;
  FastDiv fdRp, fdRw, fdKC, fdH, fdNW, fdQTT;
  Tab4Geo tg;                 // the prepared table (same extents as above)
  float qscale;               // multiplier applied to q on load (1 when pre-scaled)
  int force_max;
  int run_q, run_r;           // the tile list split over the grid G: total = run_q G + run_r
  FastDiv fdG;
  uint32_t off_kp, off_tab, off_buf, buf_bytes, off_v, off_lp, off_red;
};

template <int QT>
struct QState {
  bf16x8_t q[QT];
  int qaddr[QT];      // byte offset of the query's table base
  int qlab[QT];       // (PERKEY: the query's label byte in all 4 bytes)
  float mrow[QT];
  f32x4_t o0[QT], o1[QT], os[QT];
};

struct Win {          // one (head, window) item
  int h, w, mem;      // head, window, item index in q/k/v (w * heads + h)
  int rt0, rh0, rw0;  // rolled origin of the window
};

// item it of the head-major work list: head it / nW, window it % nW
__device__ __forceinline__ Win window_of(const AttnArgs& a, const A5& L, int it) {
  const WinGeo& g = a.geo;
  Win r;
  r.h = (int)fdiv((uint32_t)it, L.fdNW);
  const int w = it - r.h * L.nW;
  r.w = w;
  r.mem = w * L.heads + r.h;
  const int wr = w - (int)fdiv((uint32_t)w, g.fnws) * g.nws;
  const int wt = (int)fdiv((uint32_t)wr, g.fwpl);
  const int rem = wr - wt * g.nwh * g.nww;
  const int wh = (int)fdiv((uint32_t)rem, g.fnww);
  r.rt0 = wt * g.P;
  r.rh0 = wh * g.Mh;
  r.rw0 = (rem - wh * g.nww) * g.Mw;
  return r;
}

// threadIdx.x behind an empty asm: keeps the compiler from hoisting the
// per-lane address math of the staging helpers out of the window loop (it
// would hold those values in registers across the compute)
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}

// index of key group m's entry in the (step, lane group) pair layout
__device__ __forceinline__ int pair_slot(int m) { return 2 * (4 * (m >> 3) + (m & 3)) + ((m >> 2) & 1); }

// LDS address space pointer for the global-to-LDS loads
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// region labels of the window's key groups and whether they differ
template <class CF>
__device__ __forceinline__ void stage_labels(const AttnArgs& a, const A5& L, const Win& wi, unsigned char* B) {
  const WinGeo& g = a.geo;
  const int tid = opaque_tid();
  const int mhw = g.Mh * g.Mw;
  const int lab0 = slot_label_at(g, wi.rt0, wi.rh0, wi.rw0);
  int* lp = reinterpret_cast<int*>(B + L.off_lp);
  bool differs = false;
  for (int m = tid; m < L.NP * 8; m += CF::kThreads) {
    int lab = CF::kPerKey ? (int)kDummyLab4 : kDummyLab;
    if (m < L.N / 4) {
      const int aa = (int)fdiv((uint32_t)m, g.fmhw), r2 = m - aa * mhw;
      const int kh = (int)fdiv((uint32_t)r2, g.fMw), kw = r2 - kh * g.Mw;
      if constexpr (CF::kPerKey) {
        uint32_t w4 = 0;
        for (int i = 0; i < 4; ++i) {
          const int li = slot_label_at(g, wi.rt0 + 4 * aa + i, wi.rh0 + kh, wi.rw0 + kw);
          differs |= li != lab0;
          w4 |= (uint32_t)li << (8 * i);
        }
        lab = (int)w4;
      } else {
        lab = slot_label_at(g, wi.rt0 + 4 * aa, wi.rh0 + kh, wi.rw0 + kw);
        differs |= lab != lab0;
      }
    }
    lp[pair_slot(m)] = lab;
  }
  const uint64_t any = __builtin_amdgcn_ballot_w64(differs);
  if ((tid & 63) == 0) reinterpret_cast<int*>(B + L.off_red)[tid >> 6] = any != 0;
}

// key-group table offsets (bytes; the same for every window)
template <class CF>
__device__ __forceinline__ void stage_offsets(const AttnArgs& a, const A5& L, int* kp) {
  constexpr int ES = CF::kTabEs;
  const WinGeo& g = a.geo;
  const int mhw = g.Mh * g.Mw;
  for (int m = (int)threadIdx.x; m < L.NP * 8; m += CF::kThreads) {
    int off = 0;
    if (m < L.N / 4) {
      const int aa = (int)fdiv((uint32_t)m, g.fmhw), r2 = m - aa * mhw;
      const int kh = (int)fdiv((uint32_t)r2, g.fMw), kw = r2 - kh * g.Mw;
      off = ES * (4 * aa * L.Rp + kh * L.Rw + kw);
    }
    kp[pair_slot(m)] = off;
  }
}

// PERKEY masks of one key group against a query: x = label word ^ query
// label in every byte; bit 7 of byte i of z is set iff key i's label equals
// the query's; m01 / m23 hold 0xffff in the 16-bit half of each kept key of
// the bf16 pairs (keys 0, 1) / (keys 2, 3) (v_perm_b32 selectors 8..11
// replicate the sign bits of bytes 1, 3 of the second and first operand).
__device__ __forceinline__ uint32_t key_match(uint32_t lw, uint32_t q4) {
  const uint32_t x = lw ^ q4;
  return ~(((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) & 0x80808080u;
}
__device__ __forceinline__ void key_masks(uint32_t z, uint32_t& m01, uint32_t& m23) {
  const uint32_t zs = z << 8;
  m01 = __builtin_amdgcn_perm(zs, z, 0x08080a0au);
  m23 = __builtin_amdgcn_perm(zs, z, 0x09090b0bu);
}

// ---- one 32-key step for the wave's QT tiles --------------------------------
//   MODE 0: P = exp2(x); 1: row max of x only; 2: P = exp2(x - max).
//   SEL: per key group, masked / dummy groups read the -inf 4-tuple.
//   gk / lk: this step's key-group offsets / labels for lane group g4.
//   HALF: keys 32p + 16 .. + 31 are all padding; that half is skipped (P = 0).
//   CF::kBig: scalar bias table (a 4-tuple is 4 floats kBigRp apart).
//   CF::kM100 (with SEL): a key group of another region keeps its bias and
//   gets -100 log2(e) added; only dummy key groups read the -inf 4-tuple.
//   CF::kPerKey (with SEL): every group reads its own bias; keys whose label
//   differs from the query's get P = 0 (and are left out of the row max).
template <int MODE, bool SEL, int QT, bool HALF, class CF>
__device__ __forceinline__ void attn_step(int p, const unsigned char* __restrict__ B, const A5& L,
                                          const unsigned char* __restrict__ tabb, int2 gk, int2 lk, int zone,
                                          const bf16x8_t& ones, QState<QT>& st) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const int sw = (fr >> 2) & 3;
  const bf16x8_t kA = *reinterpret_cast<const bf16x8_t*>(B + (32 * p + fr) * 64 + ((g4 ^ sw) << 4));
  bf16x8_t kB = bf16x8_t{};
  if (!HALF) kB = *reinterpret_cast<const bf16x8_t*>(B + (32 * p + 16 + fr) * 64 + ((g4 ^ sw) << 4));
  bf16x8_t vA0 = bf16x8_t{}, vA1 = bf16x8_t{};
  if (MODE != 1) {
    const int d0 = 8 * (fr >> 2) + (fr & 3);
    const unsigned char* vb = B + L.off_v + p * 64 + ((g4 ^ sw) << 4);
    vA0 = *reinterpret_cast<const bf16x8_t*>(vb + d0 * L.pitch_v * 16);
    vA1 = *reinterpret_cast<const bf16x8_t*>(vb + (d0 + 4) * L.pitch_v * 16);
  }
  constexpr bool BIG = CF::kBig;
  // tiles U0 .. U0 + NU - 1: their table reads, then their products
  auto part = [&](auto u0c, auto nuc) {
    constexpr int U0 = decltype(u0c)::value, NU = decltype(nuc)::value;
    f32x4_t tA[NU], tB[NU];
    float mA[NU], mB[NU];
#pragma unroll
    for (int v = 0; v < NU; ++v) {
      const int u = U0 + v;
      // pointers selected rather than offsets, so that the LDS base is not
      // added again after each select
      const unsigned char* pA = tabb + (st.qaddr[u] + gk.x);
      const unsigned char* pB = tabb + (st.qaddr[u] + gk.y);
      const unsigned char* pz = tabb + zone;
      if (SEL && CF::kM100) {
        constexpr float kM = -100.0f * kLog2e;
        mA[v] = (lk.x == st.qlab[u] || lk.x == kDummyLab) ? 0.f : kM;
        mB[v] = (lk.y == st.qlab[u] || lk.y == kDummyLab) ? 0.f : kM;
        pA = lk.x == kDummyLab ? pz : pA;
        pB = lk.y == kDummyLab ? pz : pB;
      } else if (SEL && !CF::kPerKey) {
        pA = (lk.x == st.qlab[u]) ? pA : pz;
        pB = (lk.y == st.qlab[u]) ? pB : pz;
      }
      if constexpr (BIG) {
        const float* sa = reinterpret_cast<const float*>(pA);
        tA[v] = f32x4_t{sa[0], sa[kBigRp], sa[2 * kBigRp], sa[3 * kBigRp]};
        if (!HALF) {
          const float* sb = reinterpret_cast<const float*>(pB);
          tB[v] = f32x4_t{sb[0], sb[kBigRp], sb[2 * kBigRp], sb[3 * kBigRp]};
        }
      } else {
        tA[v] = *reinterpret_cast<const f32x4_t*>(pA);
        if (!HALF) tB[v] = *reinterpret_cast<const f32x4_t*>(pB);
      }
    }
    // every LDS read of the part is in flight before the first MFMA waits on one
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SEL && CF::kM100) {
#pragma unroll
      for (int v = 0; v < NU; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tA[v][i] += mA[v];
          if (!HALF) tB[v][i] += mB[v];
        }
    }
    if constexpr (MODE != 1 && !CF::kPerKey) {
      // software-pipelined issue order: the score products run two tiles
      // ahead of the exponentials, and each group of VALU work (4 exp2 and 2
      // packs of one half of a tile's scores) is issued behind one to three
      // products (scores of tile v + 2, P V of tile v - 1), so that the
      // matrix core and the VALU are busy at the same time.  sched_barrier
      // keeps the groups in this order.
      f32x4_t sA[NU], sB[NU];
      u32x4_t pk[NU];
      auto score = [&](int v, int hb) {
        if (hb == 0) sA[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, st.q[U0 + v], tA[v], 0, 0, 0);
        else if (!HALF) sB[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kB, st.q[U0 + v], tB[v], 0, 0, 0);
      };
      auto expo = [&](int v, int hb) {
        if (hb == 1 && HALF) {
          pk[v][2] = pk[v][3] = 0u;
          return;
        }
        const f32x4_t x = hb ? sB[v] : sA[v];
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(MODE == 2 ? x[i] - st.mrow[U0 + v] : x[i]);
        pk[v][2 * hb] = pack_bf16x2(e[0], e[1]);
        pk[v][2 * hb + 1] = pack_bf16x2(e[2], e[3]);
      };
      auto pv = [&](int v, int which) {
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk[v]);
        const int u = U0 + v;
        if (which == 0) st.o0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA0, pb, st.o0[u], 0, 0, 0);
        else if (which == 1) st.o1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA1, pb, st.o1[u], 0, 0, 0);
        else st.os[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, st.os[u], 0, 0, 0);
      };
#pragma unroll
      for (int v = 0; v < (NU < 2 ? NU : 2); ++v) {
        score(v, 0);
        score(v, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < NU; ++v) {
        if (v + 2 < NU) score(v + 2, 0);
        if (v >= 1) pv(v - 1, 0);
        expo(v, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (v + 2 < NU) score(v + 2, 1);
        if (v >= 1) {
          pv(v - 1, 1);
          pv(v - 1, 2);
        }
        expo(v, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      pv(NU - 1, 0);
      pv(NU - 1, 1);
      pv(NU - 1, 2);
      return;
    }
#pragma unroll
    for (int v = 0; v < NU; ++v) {
      const int u = U0 + v;
      const f32x4_t sA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kA, st.q[u], tA[v], 0, 0, 0);
      f32x4_t sB = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (!HALF) sB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kB, st.q[u], tB[v], 0, 0, 0);
      if (MODE == 1) {
        f32x4_t xA = sA, xB = sB;
        if constexpr (SEL && CF::kPerKey) {
          const uint32_t zA = key_match((uint32_t)lk.x, (uint32_t)st.qlab[u]);
          const uint32_t zB = key_match((uint32_t)lk.y, (uint32_t)st.qlab[u]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!((zA >> (8 * i + 7)) & 1u)) xA[i] = -INFINITY;
            if (!((zB >> (8 * i + 7)) & 1u)) xB[i] = -INFINITY;
          }
        }
        float m = st.mrow[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, HALF ? xA[i] : fmaxf(xA[i], xB[i]));
        st.mrow[u] = m;
      } else {
        float pA[4], pB[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pA[i] = __builtin_amdgcn_exp2f(MODE == 2 ? sA[i] - st.mrow[u] : sA[i]);
          pB[i] = HALF ? 0.f : __builtin_amdgcn_exp2f(MODE == 2 ? sB[i] - st.mrow[u] : sB[i]);
        }
        u32x4_t pk;
        pk[0] = pack_bf16x2(pA[0], pA[1]);
        pk[1] = pack_bf16x2(pA[2], pA[3]);
        pk[2] = pack_bf16x2(pB[0], pB[1]);
        pk[3] = pack_bf16x2(pB[2], pB[3]);
        if constexpr (SEL && CF::kPerKey) {
          uint32_t m01, m23;
          key_masks(key_match((uint32_t)lk.x, (uint32_t)st.qlab[u]), m01, m23);
          pk[0] &= m01;
          pk[1] &= m23;
          if (!HALF) {
            key_masks(key_match((uint32_t)lk.y, (uint32_t)st.qlab[u]), m01, m23);
            pk[2] &= m01;
            pk[3] &= m23;
          }
        }
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
        st.o0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA0, pb, st.o0[u], 0, 0, 0);
        st.o1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA1, pb, st.o1[u], 0, 0, 0);
        st.os[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, st.os[u], 0, 0, 0);
      }
    }
  };
  // up to 4 tiles in one part; 5 as 3 + 2 (the second part's table reads
  // after the first part's products: fewer registers live at once)
  if constexpr (QT <= 4) {
    part(std::integral_constant<int, 0>{}, std::integral_constant<int, QT>{});
  } else {
    part(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
    part(std::integral_constant<int, 3>{}, std::integral_constant<int, QT - 3>{});
  }
}

// One pass over the keys; the next step's offsets and labels are read a step ahead.
template <int MODE, bool MASKED, int QT, class CF>
__device__ __forceinline__ void attn_pass(const unsigned char* B, const A5& L, const unsigned char* tabb,
                                          const int2* kp2, int zone, const bf16x8_t& ones, QState<QT>& st) {
  const int g4 = (threadIdx.x & 63) >> 4;
  const int2* lp2 = reinterpret_cast<const int2*>(B + L.off_lp);
  const int nclean = L.N >> 5;   // steps whose 32 keys are all real
  int2 gk = kp2[g4];
  int2 lk = lp2[g4];
  // the last step's second 16 keys are all padding when N mod 32 is in 1..16
  const bool half = L.N - 32 * (L.NP - 1) <= 16;
  const int full = half ? L.NP - 1 : L.NP;
  // the steps without labels, then those with: two loops, each with one body
  // (a branch per step would merge two register assignments of the
  // accumulators at every back edge)
  int p = 0;
  if (!MASKED) {
    const int e = nclean < full ? nclean : full;
    for (; p < e; ++p) {
      const int pn = p + 1 < L.NP ? p + 1 : p;
      const int2 gkn = kp2[4 * pn + g4];
      const int2 lkn = lp2[4 * pn + g4];
      attn_step<MODE, false, QT, false, CF>(p, B, L, tabb, gk, lk, zone, ones, st);
      gk = gkn;
      lk = lkn;
    }
  }
  for (; p < full; ++p) {
    const int pn = p + 1 < L.NP ? p + 1 : p;
    const int2 gkn = kp2[4 * pn + g4];
    const int2 lkn = lp2[4 * pn + g4];
    attn_step<MODE, true, QT, false, CF>(p, B, L, tabb, gk, lk, zone, ones, st);
    gk = gkn;
    lk = lkn;
  }
  if (half) attn_step<MODE, true, QT, true, CF>(L.NP - 1, B, L, tabb, gk, lk, zone, ones, st);
}

inline size_t a5_lds(const A5& L) { return (size_t)L.off_buf + (size_t)L.NB * L.buf_bytes; }

// the split of `total` tiles into G contiguous runs that run_bounds reads;
// false when the tile count does not fit the device's 32-bit tile indices
inline bool set_runs(A5& L, int64_t total, int64_t G) {
  if (total <= 0 || total > 0x7fffffff || G <= 0 || G > 4096) return false;
  L.run_q = (int)(total / G);
  L.run_r = (int)(total % G);
  L.fdG = make_fastdiv((uint32_t)G);
  return true;
}

// run b of the grid: tiles [floor(b total / G), floor((b + 1) total / G)) of
// the head-major list, in 32-bit arithmetic (b total / G = b q + b r / G).
// The remainder is spread over the runs, so that at Swin-T stage 1 (37.5
// tiles per run) every run spans exactly two windows.
__device__ __forceinline__ void run_bounds(const A5& L, int b, int& t0, int& t1) {
  t0 = b * L.run_q + (int)fdiv((uint32_t)(b * L.run_r), L.fdG);
  t1 = (b + 1) * L.run_q + (int)fdiv((uint32_t)((b + 1) * L.run_r), L.fdG);
}

// temporal stride R' of the 4-tuple table: >= R and 4 mod 16 (conflict-free reads)
inline int tab_rp(int R) { return R + ((4 - R) % 16 + 16) % 16; }

inline bool plan_a5(const AttnArgs& a, A5& L) {
  L = A5{};
  L.N = a.N;
  L.NP = (a.N + 31) / 32;
  L.NPAD = 32 * L.NP;
  L.QTT = (a.N + 15) / 16;
  const int kc = L.NPAD / 8;                 // V^T chunks per row
  L.pitch_v = kc + ((4 - kc) % 16 + 16) % 16;
  L.R = a.rel.R;
  L.Rw = a.rel.Rw;
  L.TD = a.rel.rows / a.rel.R;               // 2 P0 - 1
  L.TH = a.rel.R / a.rel.Rw;                 // 2 Mh0 - 1
  L.Rp = tab_rp(L.R);
  L.A = (L.TD / 2) * L.Rp + (L.TH / 2) * L.Rw + L.Rw / 2;
  L.nW = (int)a.nW;
  L.heads = a.heads;
  L.fdRp = make_fastdiv((uint32_t)L.Rp);
  L.fdRw = make_fastdiv((uint32_t)L.Rw);
  L.fdKC = make_fastdiv((uint32_t)kc);
  L.fdH = make_fastdiv((uint32_t)a.heads);
  L.fdNW = make_fastdiv((uint32_t)L.nW);
  L.fdQTT = make_fastdiv((uint32_t)L.QTT);
  L.tg = tab4_geo(a.rel, a.heads, a.N);
  L.TS4 = L.tg.TS4;
  if (L.tg.scalar && L.Rp != kBigRp) return false;
  L.qscale = a.q_scaled ? 1.0f : kLog2e / sqrtf((float)a.d);
  L.force_max = a.force_max;
  if (L.TS4 > kMaxTab || a.heads > 256) return false;
  size_t off = 0;
  L.off_kp = (uint32_t)off;
  off += (size_t)L.NP * 8 * 4;
  off = (off + 15) & ~(size_t)15;
  L.off_tab = (uint32_t)off;
  L.zone = (int)L.off_tab + (L.tg.scalar ? 4 * L.TD * L.Rp : 16 * (L.TS4 - 1));
  off += (size_t)L.TS4 * 16;
  L.off_buf = (uint32_t)off;
  size_t bb = (size_t)L.NPAD * 64;
  L.off_v = (uint32_t)bb;
  bb += (size_t)32 * L.pitch_v * 16;
  L.off_lp = (uint32_t)bb;
  bb += (size_t)L.NP * 8 * 4;
  L.off_red = (uint32_t)bb;
  bb += 4 * kMaxWaves;
  L.buf_bytes = (uint32_t)((bb + 15) & ~(size_t)15);
  L.NB = off + 2 * (size_t)L.buf_bytes <= kLdsMax ? 2 : 1;
  return a5_lds(L) <= kLdsMax;
}

// whether every group of 4 temporal positions (kt = 4a .. 4a+3) of every
// window shares its temporal label and temporal pad status (else the kernel
// compares labels key by key)
inline bool groups_uniform(const AttnArgs& a) {
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
  return true;
}

}  // namespace

}  // namespace vswin
