// LN1 + pad/roll/partition gather + qkv projection + window attention in one
// kernel (bf16, head_dim 32, C in {96, 128}):
//   per (window, head) item: X = LN1(x) gathered through the slot -> token map
//   (eq. 1 first line; the mmaction2 walk-through's op order LN -> pad -> roll
//   -> partition), [q | k | v] = X Wqkv^T + b for the head's 32 features each,
//   S = q k^T / sqrt(d) + B[idx(i, j)], masked pairs excluded, O = softmax(S) v
//   (§3.2, eq. 2), heads concatenated as h * 32 + e in window slot order.
// q, k and v never reach global memory.
//
// Work split.  The query tiles (16 queries) of all items, head-major, form one
// list cut into equal contiguous runs, one per workgroup (8 waves, one per
// CU).  A run is processed in chunks of at most two consecutive items of one
// head (at Swin-T stage 1 every run is 1.5 items: one chunk, except the two
// runs that cross a head boundary).  Per chunk:
//   phase A  all waves compute K (keys x 32) and V^T (32 x keys) of every key
//            tile of the chunk's items into LDS, each from 16 gathered and
//            normalised token rows held in registers; a wave's own query
//            tiles (a contiguous share of the chunk's tiles) are among its
//            jobs, and q of those tiles comes out of the same rows straight
//            into the MFMA B-operand layout of the score product;
//   barrier
//   phase B  each wave runs the score / softmax / P v steps of its own tiles
//            (the 32-key step of the MFMA attention core) with no further
//            barrier: the waves' shares differ by at most one tile.
// The bias table of the chunk's head is built in LDS from the bf16 table (fp32
// 4-tuples times log2 e, the core's layout) when the head changes.
//
// Register layouts of phase A (lane = (fr, g), fr = lane & 15, g = lane >> 4):
// the lane holds channels 32j + 8g .. + 7 of token row fr (j < C/32), i.e.
// its k-chunks of an MFMA operand, so LayerNorm runs in registers (4 lanes
// per row) and the same registers are the B operand of K^T = Wk X^T and
// q^T = Wq X^T and the A operand of V = X Wv^T.  Wq and Wk rows are taken in
// pair order (MFMA block p, row 4g' + i = feature 8g' + 4p + i), so after the
// two blocks a lane holds features 8g .. 8g + 7 of its row: one 16-byte K
// row chunk, or exactly the q fragment of the score MFMA.  V comes out as 4
// consecutive keys of one feature: an 8-byte write into the V^T row.
#include "attn_core.h"

namespace vswin {

namespace {

using FCF = Cfg<8, 4>;            // 8 waves, 4-tuple table, group labels, exclusion mask
constexpr int kFWaves = FCF::kWaves;
constexpr int kFThreads = FCF::kThreads;
constexpr int kQOwn = 5;          // query tiles a wave owns in one chunk, at most


using FCFS = Cfg<8, 8, true>;      // the scalar-table form of the step (a chunk's second head)

// LDS layout of the fused kernel, beside the A5 geometry (whose off_kp,
// off_tab, zone, off_buf, buf_bytes, off_v, off_lp and off_red it sets):
//   [key-group offsets (4-tuple units) | key-group offsets (scalar units) |
//    4-tuple table | scalar table | buffer 0 | buffer 1 | LN1 gamma, beta,
//    qkv bias (bf16)]
// A buffer holds one item's K rows (16 QTT of them: every row a step reads),
// V^T rows, key-group labels and per-wave flags.  The scalar table (4x
// smaller) holds the second head of a chunk whose two items belong to
// different heads; without room for it (dual = 0) such items go to separate
// chunks.
struct FLay {
  uint32_t off_kps, off_tabs, off_par;
  int zone_s;      // LDS address of the scalar table's first -inf entry
  int TS4s;        // 16-byte entries of the scalar table
  int dual;
  uint32_t bytes;  // total LDS
};

inline bool fused_layout(const AttnArgs& a, A5& L, FLay& F) {
  if (!plan_a5(a, L) || L.tg.scalar) return false;
  F = FLay{};
  RelTab rel = a.rel;
  const Tab4Geo ts = tab4_geo(rel, a.heads, kMfmaMaxN + 1);   // the scalar form's extents
  if (ts.Rp != kBigRp) return false;
  size_t off = 0;
  L.off_kp = (uint32_t)off;
  off += (size_t)L.NP * 8 * 4;
  F.off_kps = (uint32_t)off;
  off += (size_t)L.NP * 8 * 4;
  off = (off + 15) & ~(size_t)15;
  L.off_tab = (uint32_t)off;
  L.zone = (int)L.off_tab + 16 * (L.TS4 - 1);
  off += (size_t)L.TS4 * 16;
  const size_t off_tabs = off;
  // a buffer: K rows, V^T, labels, flags
  size_t bb = (size_t)16 * L.QTT * 64;
  L.off_v = (uint32_t)bb;
  bb += (size_t)32 * L.pitch_v * 16;
  L.off_lp = (uint32_t)bb;
  bb += (size_t)L.NP * 8 * 4;
  L.off_red = (uint32_t)bb;
  bb += 4 * kMaxWaves;
  L.buf_bytes = (uint32_t)((bb + 15) & ~(size_t)15);
  L.NB = 2;
  const size_t par = 10 * (size_t)a.C;
  for (int dual = 1; dual >= 0; --dual) {
    size_t o = off_tabs;
    F.dual = dual;
    F.TS4s = dual ? ts.TS4 : 0;
    F.off_tabs = dual ? (uint32_t)o : 0;
    F.zone_s = dual ? (int)o + 4 * ts.TD * ts.Rp : 0;
    o += (size_t)F.TS4s * 16;
    L.off_buf = (uint32_t)o;
    o += 2 * (size_t)L.buf_bytes;
    F.off_par = (uint32_t)o;
    o += par;
    F.bytes = (uint32_t)o;
    if (o <= kLdsMax) return true;
  }
  return false;
}

__device__ __forceinline__ bf16x8_t ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Weight fragments of one head (registers, phase A): wq / wk rows in pair
// order, wv rows in natural order; [block p][k-chunk j].
template <int KS>
struct HeadW {
  bf16x8_t q[2][KS], k[2][KS], v[2][KS];
};

template <int C>
__device__ __forceinline__ void load_head_w(HeadW<C / 32>& w, const FusedArgs& f, int h) {
  constexpr int KS = C / 32;
  const int lane = threadIdx.x & 63, fr = lane & 15, g = lane >> 4;
  const bf16_t* W = reinterpret_cast<const bf16_t*>(f.w);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int pr = 8 * (fr >> 2) + 4 * p + (fr & 3);   // pair-order feature of MFMA row fr
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      w.q[p][j] = ld8(W + (size_t)(32 * h + pr) * C + 32 * j + 8 * g);
      w.k[p][j] = ld8(W + (size_t)(C + 32 * h + pr) * C + 32 * j + 8 * g);
      w.v[p][j] = ld8(W + (size_t)(2 * C + 32 * h + 16 * p + fr) * C + 32 * j + 8 * g);
    }
  }
}

// LayerNorm of 16 window rows held as raw bf16 chunks (lane: channels
// 32j + 8g .. + 7 of row fr), in registers (4 lanes per row); rows that are
// not live (pad slots, slots past N) become zero rows (the grid is padded
// after the norm).  With f.ln == 0 the rows pass through.
template <int C>
__device__ __forceinline__ void ln_rows(bf16x8_t af[C / 32], const u32x4_t (&xr)[C / 32], int live,
                                        const FusedArgs& f, const unsigned char* par) {
  constexpr int KS = C / 32;
  const int g = (threadIdx.x & 63) >> 4;
  if (!f.ln) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = live ? xr[j][e] : 0u;
      af[j] = __builtin_bit_cast(bf16x8_t, v);
    }
    return;
  }
  float xv[KS][8];
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[j][2 * e] = bflo(xr[j][e]);
      xv[j][2 * e + 1] = bfhi(xr[j][e]);
    }
  float sm = 0.f;
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) sm += xv[j][e];
  sm = row4_sum(sm);
  const float mean = sm * (1.0f / C);
  float sq = 0.f;
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dd = xv[j][e] - mean;
      sq += dd * dd;
    }
  sq = row4_sum(sq);
  const float rstd = 1.0f / sqrtf(sq * (1.0f / C) + f.eps);
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const u32x4_t gg = *reinterpret_cast<const u32x4_t*>(par + 2 * (32 * j + 8 * g));
    const u32x4_t bb = *reinterpret_cast<const u32x4_t*>(par + 2 * (C + 32 * j + 8 * g));
    u32x4_t pk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = live ? (xv[j][2 * e] - mean) * rstd * bflo(gg[e]) + bflo(bb[e]) : 0.f;
      const float hi = live ? (xv[j][2 * e + 1] - mean) * rstd * bfhi(gg[e]) + bfhi(bb[e]) : 0.f;
      pk[e] = pack_bf16x2(lo, hi);
    }
    af[j] = __builtin_bit_cast(bf16x8_t, pk);
  }
}

// K rows and V^T entries of key tile kt of the item in buffer B; with WQ
// also returns the q fragment of query tile kt (else zeros).
template <int C, bool WQ>
__device__ __forceinline__ bf16x8_t kv_tile(const bf16x8_t af[C / 32], const HeadW<C / 32>& w, const A5& L,
                                            unsigned char* B, int kt, float qscale, const unsigned char* bias_lds,
                                            int h) {
  bf16x8_t qf = bf16x8_t{};
  // the head's q / k / v biases of the lane's features (LDS copy of the
  // (3C) bias vector): q, k features 8g .. 8g + 7, v features fr, 16 + fr
  const bf16_t* bl = reinterpret_cast<const bf16_t*>(bias_lds);
  const u32x4_t bk4 = *reinterpret_cast<const u32x4_t*>(bl + C + 32 * h + 8 * ((threadIdx.x & 63) >> 4));
  const float bv0 = bf2f(bl[2 * C + 32 * h + (threadIdx.x & 15)]);
  const float bv1 = bf2f(bl[2 * C + 32 * h + 16 + (threadIdx.x & 15)]);
  constexpr int KS = C / 32;
  const int lane = threadIdx.x & 63, fr = lane & 15, g = lane >> 4;
  // K: features 8g .. 8g + 7 of key row 16 kt + fr
  f32x4_t k0 = {0.f, 0.f, 0.f, 0.f}, k1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    k0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.k[0][j], af[j], k0, 0, 0, 0);
    k1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.k[1][j], af[j], k1, 0, 0, 0);
  }
  // V: keys 16 kt + 4g .. + 3 of features fr (block 0) and 16 + fr (block 1)
  f32x4_t v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    v0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], w.v[0][j], v0, 0, 0, 0);
    v1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], w.v[1][j], v1, 0, 0, 0);
  }
  if constexpr (WQ) {
    f32x4_t q0 = {0.f, 0.f, 0.f, 0.f}, q1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      q0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.q[0][j], af[j], q0, 0, 0, 0);
      q1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.q[1][j], af[j], q1, 0, 0, 0);
    }
    const u32x4_t bq4 = *reinterpret_cast<const u32x4_t*>(bl + 32 * h + 8 * ((threadIdx.x & 63) >> 4));
    u32x4_t pk;
    pk[0] = pack_bf16x2((q0[0] + bflo(bq4[0])) * qscale, (q0[1] + bfhi(bq4[0])) * qscale);
    pk[1] = pack_bf16x2((q0[2] + bflo(bq4[1])) * qscale, (q0[3] + bfhi(bq4[1])) * qscale);
    pk[2] = pack_bf16x2((q1[0] + bflo(bq4[2])) * qscale, (q1[1] + bfhi(bq4[2])) * qscale);
    pk[3] = pack_bf16x2((q1[2] + bflo(bq4[3])) * qscale, (q1[3] + bfhi(bq4[3])) * qscale);
    qf = __builtin_bit_cast(bf16x8_t, pk);
  }
  {
    const int r = 16 * kt + fr;
    u32x4_t pk;
    pk[0] = pack_bf16x2(k0[0] + bflo(bk4[0]), k0[1] + bfhi(bk4[0]));
    pk[1] = pack_bf16x2(k0[2] + bflo(bk4[1]), k0[3] + bfhi(bk4[1]));
    pk[2] = pack_bf16x2(k1[0] + bflo(bk4[2]), k1[1] + bfhi(bk4[2]));
    pk[3] = pack_bf16x2(k1[2] + bflo(bk4[3]), k1[3] + bfhi(bk4[3]));
    *reinterpret_cast<u32x4_t*>(B + r * 64 + ((g ^ ((fr >> 2) & 3)) << 4)) = pk;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const f32x4_t& v = p ? v1 : v0;
    const float bv = p ? bv1 : bv0;
    const int d = 16 * p + fr;
    u32x2_t pk;
    pk[0] = pack_bf16x2(v[0] + bv, v[1] + bv);
    pk[1] = pack_bf16x2(v[2] + bv, v[3] + bv);
    const int chunk = (4 * (kt >> 1) + g) ^ ((d >> 3) & 3);
    *reinterpret_cast<u32x2_t*>(B + L.off_v + (d * L.pitch_v + chunk) * 16 + 8 * (kt & 1)) = pk;
  }
  return qf;
}

// n bytes (a multiple of 16) from global memory to LDS by direct
// global-to-LDS loads (16 bytes per lane; wave w0 upward, 1 KB per wave
// instruction); the caller waits for vmcnt and a barrier.
__device__ __forceinline__ void dma_to_lds(const void* src, unsigned char* dst, int n, int w0) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const unsigned char* S = reinterpret_cast<const unsigned char*>(src);
  const int nchunk = n / 16;
  for (int b = (wv + kFWaves - w0) % kFWaves; 64 * b < nchunk; b += kFWaves)
    if (64 * b + lane < nchunk)
      __builtin_amdgcn_global_load_lds(S + 16 * (64 * b + lane), (lds_ptr_t)(dst + 1024 * b), 16, 0, 0);
}

// The bf16 table (rows, heads) into LDS at `raw`: the whole 16-byte chunks
// by direct loads; the last partial chunk's 2-byte entries (fewer than 8) are
// loaded into the returned register by lanes of wave 4 and written by
// raw_table_tail once the caller has waited for its loads.
__device__ __forceinline__ uint32_t stage_raw_table(const FusedArgs& f, unsigned char* raw) {
  const int n = f.a.rel.rows * f.a.heads * 2;
  dma_to_lds(f.a.table, raw, n & ~15, 0);
  const int tail = (n & 15) / 2;
  uint32_t v = 0;
  if (tail && (threadIdx.x >> 6) == 4 && (int)(threadIdx.x & 63) < tail)
    v = reinterpret_cast<const bf16_t*>(f.a.table)[(n & ~15) / 2 + (threadIdx.x & 63)];
  return v;
}
__device__ __forceinline__ void raw_table_tail(const FusedArgs& f, unsigned char* raw, uint32_t v) {
  const int n = f.a.rel.rows * f.a.heads * 2;
  const int tail = (n & 15) / 2;
  if (tail && (threadIdx.x >> 6) == 4 && (int)(threadIdx.x & 63) < tail)
    reinterpret_cast<bf16_t*>(raw)[(n & ~15) / 2 + (threadIdx.x & 63)] = (bf16_t)v;
}

// head h's prepared 4-tuple table (the core's layout: fp32 * log2 e, offsets
// outside the table 0, the last entry all -inf) built in LDS from the staged
// bf16 table
__device__ __forceinline__ void build_table(const A5& L, int heads, int h, const unsigned char* raw,
                                            unsigned char* smem) {
  constexpr int PER = 6;
  const Tab4Geo& tg = L.tg;
  const bf16_t* T = reinterpret_cast<const bf16_t*>(raw);
  for (int x0 = (int)threadIdx.x; x0 < L.TS4; x0 += PER * kFThreads) {
    float v[PER][4];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = x0 + u * kFThreads;
      const int dtr = (int)fdiv((uint32_t)x, tg.fdRp);
      const int rem = x - dtr * tg.Rp;
      const int dhr = (int)fdiv((uint32_t)rem, tg.fdRw);
      const int dwr = rem - dhr * tg.Rw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dt = dtr + i;
        const bool ok = x < L.TS4 - 1 && rem < tg.R && dt < tg.TD;
        const int row = ok ? (tg.TD - 1 - dt) * tg.R + (tg.TH - 1 - dhr) * tg.Rw + (tg.Rw - 1 - dwr) : 0;
        const float t = bf2f(T[row * heads + h]);
        v[u][i] = x >= L.TS4 - 1 ? -INFINITY : (ok ? t * kLog2e : 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = x0 + u * kFThreads;
      if (x < L.TS4)
        *reinterpret_cast<f32x4_t*>(smem + L.off_tab + 16 * x) = f32x4_t{v[u][0], v[u][1], v[u][2], v[u][3]};
    }
  }
}

// head h's table in the scalar form (S[y] = B(y) * log2 e for y < TD Rp,
// offsets outside the table 0, then 3 Rp + 1 entries of -inf) at off_tabs
__device__ __forceinline__ void build_table_s(const A5& L, const FLay& F, int heads, int h,
                                              const unsigned char* raw, unsigned char* smem) {
  const Tab4Geo& tg = L.tg;
  const bf16_t* T = reinterpret_cast<const bf16_t*>(raw);
  const int n = 4 * F.TS4s;
  for (int y = (int)threadIdx.x; y < n; y += kFThreads) {
    float e = -INFINITY;
    if (y < tg.TD * tg.Rp) {
      const int dtr = (int)fdiv((uint32_t)y, tg.fdRp);
      const int rem = y - dtr * tg.Rp;
      const int dhr = (int)fdiv((uint32_t)rem, tg.fdRw);
      const int dwr = rem - dhr * tg.Rw;
      const bool ok = rem < tg.R;
      const int row = ok ? (tg.TD - 1 - dtr) * tg.R + (tg.TH - 1 - dhr) * tg.Rw + (tg.Rw - 1 - dwr) : 0;
      const float t = bf2f(T[row * heads + h]);
      e = ok ? t * kLog2e : 0.f;
    }
    reinterpret_cast<float*>(smem + F.off_tabs)[y] = e;
  }
}

// Phase B of QT consecutive query tiles jt .. jt + QT - 1 of item wi (head
// h), q fragments given (already scaled by log2(e) / sqrt(d)).
// CF: FCF (the 4-tuple table at off_tab, offsets kp) or FCFS (the scalar
// table; kp then holds the offsets in scalar units); zone: the table's -inf
// entry.
template <int QT, class CF>
__device__ __forceinline__ void fused_tiles(const FusedArgs& f, const A5& L, const Win& wi, int jt,
                                            const bf16x8_t (&qg)[5], const unsigned char* B,
                                            const unsigned char* smem, const int* kp, uint32_t off_tab, int zone) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const int N = L.N;
  const unsigned char* tabb = smem;
  constexpr int ES = CF::kTabEs;
  const int* lp = reinterpret_cast<const int*>(B + L.off_lp);
  int masked = 0;
#pragma unroll
  for (int i = 0; i < CF::kWaves; ++i) masked |= reinterpret_cast<const int*>(B + L.off_red)[i];

  QState<QT> st;
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qs = 16 * (jt + u) + fr;
    const int ps = pair_slot(qs >> 2);
    st.qaddr[u] = (int)off_tab + ES * L.A - kp[ps] - ES * (qs & 3) * L.Rp;
    st.qlab[u] = lp[ps];
    st.q[u] = qg[u];
  }
  bf16x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  // held in VGPRs across the steps (not rebuilt from scalars in every step)
  asm volatile("" : "+v"(ones));
  const int2* kp2 = reinterpret_cast<const int2*>(kp);
  auto clear = [&]() {
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      st.mrow[u] = -INFINITY;
      st.o0[u] = st.o1[u] = st.os[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  // P = exp2(x) with no max first (softmax is shift invariant); a row whose
  // sum leaves [2^-100, 2^100] or whose accumulators are not finite sends the
  // wave through the exact pass that subtracts the row max first
  bool exact = L.force_max != 0;
  if (!exact) {
    clear();
    if (masked) attn_pass<0, true, QT, CF>(B, L, tabb, kp2, zone, ones, st);
    else attn_pass<0, false, QT, CF>(B, L, tabb, kp2, zone, ones, st);
    bool bad = false;
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int qs = 16 * (jt + u) + fr;
      const float sum = st.os[u][0];
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) t += st.o0[u][i] + st.o1[u][i];
      bad |= qs < N && !(sum >= 0x1p-100f && sum <= 0x1p100f && t - t == 0.f);
    }
    exact = __builtin_amdgcn_ballot_w64(bad) != 0;
  }
  if (exact) {
    clear();
    if (masked) attn_pass<1, true, QT, CF>(B, L, tabb, kp2, zone, ones, st);
    else attn_pass<1, false, QT, CF>(B, L, tabb, kp2, zone, ones, st);
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      float m = st.mrow[u];
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      st.mrow[u] = (m == -INFINITY) ? 0.f : m;
    }
    if (masked) attn_pass<2, true, QT, CF>(B, L, tabb, kp2, zone, ones, st);
    else attn_pass<2, false, QT, CF>(B, L, tabb, kp2, zone, ones, st);
  }
  // lane: query fr, output features 8 g4 .. + 7 of head h
  bf16_t* Og = reinterpret_cast<bf16_t*>(f.a.o);
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qs = 16 * (jt + u) + fr;
    if (qs >= N) continue;
    const float inv = __builtin_amdgcn_rcpf(st.os[u][0]);
    u32x4_t pk;
    pk[0] = pack_bf16x2(st.o0[u][0] * inv, st.o0[u][1] * inv);
    pk[1] = pack_bf16x2(st.o0[u][2] * inv, st.o0[u][3] * inv);
    pk[2] = pack_bf16x2(st.o1[u][0] * inv, st.o1[u][1] * inv);
    pk[3] = pack_bf16x2(st.o1[u][2] * inv, st.o1[u][3] * inv);
    *reinterpret_cast<u32x4_t*>(Og + ((int64_t)wi.w * N + qs) * f.a.C + wi.h * 32 + 8 * g4) = pk;
  }
}

// cnt (1 .. 4) consecutive tiles
template <class CF>
__device__ __forceinline__ void fused_group(int cnt, const FusedArgs& f, const A5& L, const Win& wi, int jt,
                                            const bf16x8_t (&qg)[5], const unsigned char* B,
                                            const unsigned char* smem, const int* kp, uint32_t off_tab, int zone) {
  if (cnt == 4) fused_tiles<4, CF>(f, L, wi, jt, qg, B, smem, kp, off_tab, zone);
  else if (cnt == 3) fused_tiles<3, CF>(f, L, wi, jt, qg, B, smem, kp, off_tab, zone);
  else if (cnt == 2) fused_tiles<2, CF>(f, L, wi, jt, qg, B, smem, kp, off_tab, zone);
  else if (cnt == 1) fused_tiles<1, CF>(f, L, wi, jt, qg, B, smem, kp, off_tab, zone);
}

}  // namespace

template <int C>
__global__ void __launch_bounds__(kFThreads) wattn_fused_kernel(const FusedArgs f, const A5 L, const FLay F) {
  warm_args_grid(f, L, F);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const AttnArgs& a = f.a;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // XCD-aware order: consecutive runs go to workgroups on the same XCD
  int b = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  int t0, t1;
  run_bounds(L, b, t0, t1);
  if (t0 >= t1) return;
  const int QTT = L.QTT;
  auto item_of = [&](int tile) { return (int)fdiv((uint32_t)tile, L.fdQTT); };

  int* kp = reinterpret_cast<int*>(smem + L.off_kp);
  int* kps = reinterpret_cast<int*>(smem + F.off_kps);
  stage_offsets<FCF>(a, L, kp);
  if (F.dual) stage_offsets<FCFS>(a, L, kps);
  // LN1 gamma, beta and the qkv bias, staged by DMA with the first table
  const uint32_t off_par = F.off_par;
  if (!f.bias)
    for (int c = (int)threadIdx.x; c < 3 * C / 8; c += kFThreads)
      *reinterpret_cast<u32x4_t*>(smem + off_par + 4 * C + 16 * c) = u32x4_t{0u, 0u, 0u, 0u};
  // V^T entries of keys 16 QTT .. 32 NP - 1 (the second half of the last
  // 32-key block when QTT is odd): never written by a key tile, multiplied by
  // P = 0 in the last step, so they must hold finite values
  if (QTT & 1) {
    for (int x = (int)threadIdx.x; x < 2 * 32 * 4; x += kFThreads) {
      const int nb = x >> 7, d = (x >> 2) & 31, gg = x & 3;
      unsigned char* B = smem + L.off_buf + (size_t)nb * L.buf_bytes;
      const int chunk = (4 * (L.NP - 1) + gg) ^ ((d >> 3) & 3);
      *reinterpret_cast<u32x2_t*>(B + L.off_v + (d * L.pitch_v + chunk) * 16 + 8) = u32x2_t{0u, 0u};
    }
  }

  int tab_head = -1, tabs_head = -1;   // heads in the 4-tuple and the scalar table
  bool first = true;
  for (int t = t0; t < t1;) {
    // chunk: one or two consecutive items of one head, at most 8 kQOwn tiles
    // (a long run then recomputes K and V^T of an item cut there)
    const int i0 = item_of(t);
    const int h = (int)fdiv((uint32_t)i0, L.fdNW);
    int i1 = i0;
    if ((i0 + 1) * QTT < t1 && (F.dual || i0 + 1 < (h + 1) * L.nW)) i1 = i0 + 1;
    int c1 = t1 < (i1 + 1) * QTT ? t1 : (i1 + 1) * QTT;
    if (c1 - t > kFWaves * kQOwn) c1 = t + kFWaves * kQOwn;
    if (c1 <= (i0 + 1) * QTT) i1 = i0;   // the cut left only the first item
    const int n = c1 - t;
    const int nit = i1 - i0 + 1;
    const int hB = (int)fdiv((uint32_t)i1, L.fdNW);   // the second item's head (h, or the next head)
    const Win win0 = window_of(a, L, i0);
    const Win win1 = window_of(a, L, i1);
    const int own_lo = t + wv * n / kFWaves, own_hi = t + (wv + 1) * n / kFWaves;
    const int nown = own_hi - own_lo;
    // jobs of the wave: its own tiles first (with q), then the key tiles no
    // wave owns (before and after the chunk's range), round robin
    const int lo = i0 * QTT, hi = (i1 + 1) * QTT;
    const int before = t - lo;
    const int norph = (hi - lo) - n;
    const int nj = nown + (norph > wv ? (norph - wv + kFWaves - 1) / kFWaves : 0);
    // job order: the first item's jobs (own tiles, then unowned key tiles
    // before the chunk's range), then the second item's (own, then unowned
    // after the range), so that the head's weights change at most once
    const int endA = (i0 + 1) * QTT;
    const int nownA = (own_hi < endA ? own_hi : endA) - own_lo > 0 ? (own_hi < endA ? own_hi : endA) - own_lo : 0;
    const int nownB = nown - nownA;
    const int norphA = before > wv ? (before - wv + kFWaves - 1) / kFWaves : 0;
    const int njA = nownA + norphA;
    auto job_tile = [&](int j) {     // list index of job j's key tile
      if (j < nownA) return own_lo + j;
      j -= nownA;
      if (j < norphA) return lo + wv + kFWaves * j;
      j -= norphA;
      if (j < nownB) return own_lo + nownA + j;
      j -= nownB;
      const int o = wv + kFWaves * (norphA + j);
      return c1 + (o - before);
    };
    // the gathered rows of job j (slot 16 kt + fr of its window), loaded
    // without branches so that the compiler can count them in flight: rows
    // that are not live (pad slots, slots past N, jobs past the last) read
    // token 0 and are zeroed by ln_rows
    auto job_load = [&](int j, u32x4_t (&xr)[C / 32], int& live) {
      const int jj = j < nj ? j : 0;
      const int gt = job_tile(jj);
      const int it = item_of(gt);
      const int sl = 16 * (gt - it * QTT) + (threadIdx.x & 15);
      int lab;
      const int64_t src = slot_source(a.geo, it == i0 ? win0.w : win1.w, sl < L.N ? sl : 0, lab);
      live = (j < nj && sl < L.N && src >= 0) ? 1 : 0;
      const bf16_t* xp =
          reinterpret_cast<const bf16_t*>(f.x) + (live ? src : 0) * C + 8 * ((threadIdx.x & 63) >> 4);
#pragma unroll
      for (int q = 0; q < C / 32; ++q) xr[q] = *reinterpret_cast<const u32x4_t*>(xp + 32 * q);
    };
    HeadW<C / 32> hw;   // the weights of head h (the chunk's second head, if any, is loaded when reached)
    u32x4_t xa[C / 32], xb[C / 32];
    int la, lb;
    unsigned char* raw = smem + L.off_buf + L.buf_bytes;   // the bf16 table, staged in buffer 1
    if (first) {
      // every global load of the start in flight at once: the table and the
      // LN / bias vectors to LDS, the head's weights and the first two jobs'
      // rows to registers; the label work runs meanwhile
      const uint32_t tailv = stage_raw_table(f, raw);
      if (f.ln) {
        dma_to_lds(f.ln_g, smem + off_par, 2 * C, 5);
        dma_to_lds(f.ln_b, smem + off_par + 2 * C, 2 * C, 6);
      }
      if (f.bias) dma_to_lds(f.bias, smem + off_par + 4 * C, 6 * C, 7);
      asm volatile("" ::: "memory");
      load_head_w<C>(hw, f, h);
      job_load(0, xa, la);
      job_load(1, xb, lb);
      stage_labels<FCF>(a, L, win0, smem + L.off_buf);
      if (nit > 1) stage_labels<FCF>(a, L, win1, smem + L.off_buf + L.buf_bytes);
      // the direct-to-LDS loads were issued before the 6 KS register loads
      // of the weights and 2 KS of the rows
      constexpr int kLater = 8 * (C / 32);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLater) : "memory");
      raw_table_tail(f, raw, tailv);
      __syncthreads();
      build_table(L, a.heads, h, raw, smem);
      if (hB != h) build_table_s(L, F, a.heads, hB, raw, smem);
      __syncthreads();
      tab_head = h;
      if (hB != h) tabs_head = hB;
    } else {
      __syncthreads();   // the previous chunk's phase B has left the buffers and the table
      const bool need_s = hB != h && hB != tabs_head;
      if (h != tab_head || need_s) {
        const uint32_t tailv = stage_raw_table(f, raw);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        raw_table_tail(f, raw, tailv);
        __syncthreads();
        if (h != tab_head) build_table(L, a.heads, h, raw, smem);
        if (need_s) build_table_s(L, F, a.heads, hB, raw, smem);
        __syncthreads();
        tab_head = h;
        if (need_s) tabs_head = hB;
      }
      stage_labels<FCF>(a, L, win0, smem + L.off_buf);
      if (nit > 1) stage_labels<FCF>(a, L, win1, smem + L.off_buf + L.buf_bytes);
      load_head_w<C>(hw, f, h);
      job_load(0, xa, la);
      job_load(1, xb, lb);
    }
    first = false;

    // q fragments of the wave's own tiles: registers, written and read under
    // wave-uniform branches (no indexed register array)
    bf16x8_t q0 = bf16x8_t{}, q1 = q0, q2 = q0, q3 = q0, q4 = q0;
    auto do_job = [&](int j, const u32x4_t (&xr)[C / 32], int live) {
      const int gt = job_tile(j);
      const int it = item_of(gt);
      const int k = it - i0, kt = gt - it * QTT;
      const int hk = k ? hB : h;
      if (j == njA && hB != h) load_head_w<C>(hw, f, hB);   // the second item is of the next head
      bf16x8_t af[C / 32];
      ln_rows<C>(af, xr, live, f, smem + off_par);
      unsigned char* B = smem + L.off_buf + (size_t)k * L.buf_bytes;
      if (gt >= own_lo && gt < own_hi) {
        const bf16x8_t qf = kv_tile<C, true>(af, hw, L, B, kt, L.qscale, smem + off_par + 4 * C, hk);
        const int u = gt - own_lo;
        if (u == 0) q0 = qf;
        else if (u == 1) q1 = qf;
        else if (u == 2) q2 = qf;
        else if (u == 3) q3 = qf;
        else q4 = qf;
      } else {
        kv_tile<C, false>(af, hw, L, B, kt, 1.0f, smem + off_par + 4 * C, hk);
      }
    };
    // two jobs' rows in flight in fixed registers (the loop is unrolled by
    // two: no register copy touches a row that is still loading)
    for (int j = 0; j < nj; j += 2) {
      do_job(j, xa, la);
      job_load(j + 2, xa, la);
      if (j + 1 < nj) do_job(j + 1, xb, lb);
      job_load(j + 3, xb, lb);
    }
    __syncthreads();

    // ---- phase B: the wave's own tiles in groups of at most 4 consecutive
    // tiles of one item (5 tiles of an item as 3 + 2); one copy of the group
    // code, looped over
    if (nown > 0) {
      const int k0 = item_of(own_lo) - i0;
      const int endA = (i0 + k0 + 1) * QTT;
      const int nA = (own_hi < endA ? own_hi : endA) - own_lo;
      int u0 = 0;
      while (u0 < nown) {
        const bool inA = u0 < nA;
        const int left = inA ? nA - u0 : nown - u0;
        const int cnt = left == 5 ? 3 : (left < 4 ? left : 4);
        const int kk = inA ? k0 : k0 + 1;
        const int jt = own_lo + u0 - (i0 + kk) * QTT;
        // the group's q fragments, shifted down to positions 0 .. cnt - 1
        bf16x8_t qg[5];
        if (u0 == 0) { qg[0] = q0; qg[1] = q1; qg[2] = q2; qg[3] = q3; qg[4] = q4; }
        else if (u0 == 1) { qg[0] = q1; qg[1] = q2; qg[2] = q3; qg[3] = q4; qg[4] = q4; }
        else if (u0 == 2) { qg[0] = q2; qg[1] = q3; qg[2] = q4; qg[3] = q4; qg[4] = q4; }
        else if (u0 == 3) { qg[0] = q3; qg[1] = q4; qg[2] = q4; qg[3] = q4; qg[4] = q4; }
        else { qg[0] = q4; qg[1] = q4; qg[2] = q4; qg[3] = q4; qg[4] = q4; }
        const unsigned char* B = smem + L.off_buf + (size_t)kk * L.buf_bytes;
        if (kk == 0 || hB == h)
          fused_group<FCF>(cnt, f, L, kk ? win1 : win0, jt, qg, B, smem, kp, L.off_tab, L.zone);
        else   // the chunk's second head: the scalar table
          fused_group<FCFS>(cnt, f, L, win1, jt, qg, B, smem, kps, F.off_tabs, F.zone_s);
        u0 += cnt;
      }
    }
    t = c1;
  }
}

bool attention_fused_supported(vswin_dtype dt, const AttnArgs& a) {
  if (dt != VSWIN_BF16 || a.d != 32 || (a.C != 96 && a.C != 128) || a.heads * 32 != a.C) return false;
  if (a.mask_m100 || a.geo.P % 4 != 0 || a.N > kMfmaMaxN || !groups_uniform(a)) return false;
  A5 L;
  FLay F;
  return fused_layout(a, L, F);
}

hipError_t attention_fused(const FusedArgs& f, hipStream_t st) {
  const AttnArgs& a = f.a;
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  AttnArgs ak = a;
  if (const char* e = getenv("VSWIN_ATTN_MAXPASS")) ak.force_max = atoi(e) != 0;
  A5 L;
  FLay F;
  if (!fused_layout(ak, L, F) || !ak.table || !f.x || !f.w || !ak.o) return hipErrorInvalidValue;
  L.qscale = kLog2e / sqrtf(32.0f);
  const int64_t tiles = items * (int64_t)L.QTT;
  if (tiles >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  // one workgroup per CU (the LDS of one), each a contiguous run
  int64_t G = device_cu_count();
  if (G > tiles) G = tiles;
  if (!set_runs(L, tiles, G)) return hipErrorInvalidValue;
  const size_t lds = F.bytes;
  FusedArgs fk = f;
  fk.a = ak;
  if (a.C == 96) {
    hipError_t e = ensure_dynamic_lds((const void*)wattn_fused_kernel<96>, lds);
    if (e != hipSuccess) return e;
    wattn_fused_kernel<96><<<dim3((unsigned)G), dim3(kFThreads), lds, st>>>(fk, L, F);
  } else {
    hipError_t e = ensure_dynamic_lds((const void*)wattn_fused_kernel<128>, lds);
    if (e != hipSuccess) return e;
    wattn_fused_kernel<128><<<dim3((unsigned)G), dim3(kFThreads), lds, st>>>(fk, L, F);
  }
  return hipGetLastError();
}

}  // namespace vswin
