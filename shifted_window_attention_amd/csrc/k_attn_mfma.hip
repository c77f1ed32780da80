// Window attention on MFMA for bf16, head_dim 32 (§3.2, eq. 2):
//   per (window, head): S = q k^T / sqrt(d) + B[idx(i, j)], masked pairs
//   excluded, P = softmax_j(S), O = P v, heads concatenated as h*32 + e.
//
// Work split.  The query tiles (16 queries) of all (head, window) items,
// head-major, form one list; each workgroup (W waves, one per CU) takes an
// equal contiguous run of it and copies the run's head's prepared bias table
// (built once per call) to LDS, again only where the run crosses into the next
// head.  At Swin-T stage 1 every run is 1.5 windows and spans exactly two
// windows.  A window's K and V^T are staged once in LDS for all of the run's
// tiles of that window by direct global-to-LDS loads, and the next window's
// are in flight while the current one is computed (two LDS buffers when they
// fit, else one).  Waves own tiles, not steps: inside a window no barrier is
// needed.
//
// Scores.  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (k = head_dim): a lane
// holds 4 keys of one query, so all per-query state stays in the lane.
//   * Keys are in slot order (slot 4m + i holds temporal position 4a + i of
//     spatial cell m), so the 4 keys of a lane differ only in their temporal
//     offset.  The bias table is stored in LDS as fp32 4-tuples
//     (B[r], B[r + R'], B[r + 2R'], B[r + 3R']) * log2(e) indexed by the
//     query's and the key group's offsets, and enters as the MFMA's C operand:
//     the bias costs one 16-byte LDS read per 4 scores and no VALU.  Masked
//     and dummy key groups read a 4-tuple of -inf instead.
//   * q arrives multiplied by log2(e) / sqrt(d), so the MFMA result is the
//     exponent of 2 directly.  P = exp2(x) with no running max (softmax is
//     shift invariant); a row whose sum leaves [2^-100, 2^100] or whose
//     accumulators are not finite sends its wave through an exact pass that
//     subtracts the row max first.
//   * O^T = V^T P^T on MFMA with P^T already in B-operand layout; the row
//     sums come from a third MFMA against a ones operand.  V^T rows are read
//     in pair order (d = 8g + 4p + i), so a lane ends with 8 consecutive
//     output features and writes one 16-byte vector per query.
//   * A query slot's table offset and region label are those of its key
//     group (the same 4 temporal positions), read from the per-window tables.
//
// LDS layouts (bank-conflict free 16-byte fragment reads):
//   K      key rows of 64 bytes; chunk c of row r at chunk c ^ ((r >> 2) & 3).
//   V^T    32 rows of the padded key count; inside each 32-key block the keys
//          are permuted so lane group g's 8 keys {4g..4g+3, 16+4g..16+4g+3}
//          are one 16-byte chunk; chunk c of row d at c ^ ((d >> 3) & 3); the
//          row pitch is 4 mod 16 chunks.
//   table  4-tuples with a temporal stride R' = 4 mod 16 entries (R' >= R).
#include "attn_core.h"

#include <stdlib.h>

namespace vswin {

namespace {

// ---- staging -------------------------------------------------------------
// One window's K and V^T go from global memory straight into LDS
// (global_load_lds: a wave instruction fills 1 KB, or 256 B for 4-byte
// elements, at a uniform LDS address, from per-lane global addresses), so no
// registers or VALU work carry them.  Lanes whose key is past N stay off; their
// LDS slots hold the zeros written once by zero_pads.
//   K: instruction b covers key rows 16b .. 16b + 15; lane i takes row
//      16b + i/4, LDS chunk i%4, i.e. global chunk (i%4) ^ ((i>>4)&3).
//   V^T: instruction (d, q) covers chunk slots 16q .. 16q + 15 of row d; lane i
//      takes slot 16q + i/4, dword i%4: keys 2 apart pairs of its 8 keys.
//      Wave wv owns rows 8 (wv>>1) + 4 (wv&1) .. + 3, so the row swizzle
//      (d >> 3) & 3 = wv >> 1 is the same for all of its rows.

template <class CF>
__device__ __forceinline__ void stage_kv(const AttnArgs& a, const A5& L, int mem, unsigned char* B, int wv) {
  static_assert(CF::kWaves == 8, "V^T rows are split as 4 per wave");
  const int lane = threadIdx.x & 63;
  const bf16_t* Kg = reinterpret_cast<const bf16_t*>(a.k) + (int64_t)mem * L.N * 32;
  const bf16_t* Vg = reinterpret_cast<const bf16_t*>(a.v) + (int64_t)mem * L.N * 32;
  const int kr = lane >> 2;
  const int koff = kr * 32 + (((lane & 3) ^ ((lane >> 4) & 3)) << 3);
  const int nkb = (L.N + 15) >> 4;
  for (int b = wv; b < nkb; b += CF::kWaves) {
    if (16 * b + kr < L.N)
      __builtin_amdgcn_global_load_lds(Kg + b * 512 + koff, (lds_ptr_t)(B + b * 1024), 16, 0, 0);
  }
  const int sw = wv >> 1;
  const int key = 32 * (lane >> 4) + 4 * (((lane >> 2) & 3) ^ sw) + 16 * ((lane >> 1) & 1) + 2 * (lane & 1);
  const int nq = (4 * L.NP + 15) >> 4;
  for (int r = 0; r < 4; ++r) {
    const int d = 8 * sw + 4 * (wv & 1) + r;
    for (int q = 0; q < nq; ++q) {
      if (key + 128 * q < L.N)
        __builtin_amdgcn_global_load_lds(Vg + d * L.N + 128 * q + key,
                                         (lds_ptr_t)(B + L.off_v + (d * L.pitch_v + 16 * q) * 16), 4, 0, 0);
    }
  }
}

// zeros in every LDS slot of the K / V^T buffers that stage_kv never writes
// and the steps read: key rows N .. NPAD - 1 of K, and in V^T the keys >= N of
// the last 32-key block
template <class CF>
__device__ __forceinline__ void zero_pads(const A5& L, unsigned char* smem) {
  const int tid = threadIdx.x;
  for (int nb = 0; nb < L.NB; ++nb) {
    unsigned char* B = smem + L.off_buf + (size_t)nb * L.buf_bytes;
    for (int x = tid; x < (L.NPAD - L.N) * 16; x += CF::kThreads)
      reinterpret_cast<uint32_t*>(B + L.N * 64)[x] = 0u;
    for (int x = tid; x < 32 * 16; x += CF::kThreads) {
      const int d = x >> 4, jp = (x >> 2) & 3, e = x & 3;
      const int j = jp ^ ((d >> 3) & 3);
      const int key = 32 * (L.NP - 1) + 4 * j + 16 * (e >> 1) + 2 * (e & 1);
      if (key >= L.N)
        *reinterpret_cast<uint32_t*>(B + L.off_v + (d * L.pitch_v + 4 * (L.NP - 1) + jp) * 16 + 4 * e) = 0u;
    }
  }
}

// The prepared tables of every head, (heads, TS4) 4-tuples, built once per
// call and copied to LDS by each workgroup.
__global__ void __launch_bounds__(256) attn_table_kernel(const bf16_t* __restrict__ T, f32x4_t* __restrict__ out,
                                                         const A5 L) {
  warm_args(T, out, L);
  const int x = blockIdx.x * 256 + (int)threadIdx.x;
  const int h = blockIdx.y;
  if (x < L.TS4) out[(size_t)h * L.TS4 + x] = tab_entry(T, L.tg, h, x);
}

// head h's prepared table into LDS by direct global-to-LDS loads (1 KB per
// wave instruction); the last instruction's lanes past TS4 stay off
template <class CF>
__device__ __forceinline__ void tab_copy(const AttnArgs& a, const A5& L, int h, unsigned char* smem, int wv) {
  const int lane = threadIdx.x & 63;
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.tab4) + (size_t)h * L.TS4;
  const int nb = (L.TS4 + 63) >> 6;
  for (int b = wv; b < nb; b += CF::kWaves) {
    if (64 * b + lane < L.TS4)
      __builtin_amdgcn_global_load_lds(src + 64 * b + lane, (lds_ptr_t)(smem + L.off_tab + 1024 * b), 16, 0, 0);
  }
}

// The wave's QT query tiles jt, jt + W, ... of one window.
// q rows of a wave's tiles of one window (loaded a window ahead)
template <class CF>
struct QPre {
  u32x4_t q[CF::kQTM];
};

template <class CF>
__device__ __forceinline__ void q_load(QPre<CF>& qp, const AttnArgs& a, const A5& L, int mem, int jt, int cnt) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const bf16_t* Qg = reinterpret_cast<const bf16_t*>(a.q) + (int64_t)mem * L.N * 32;
#pragma unroll
  for (int u = 0; u < CF::kQTM; ++u) {
    const int qs = 16 * (jt + CF::kWaves * u) + fr;
    qp.q[u] = (u < cnt && qs < L.N) ? *reinterpret_cast<const u32x4_t*>(Qg + qs * 32 + g4 * 8)
                                    : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// The wave's tiles U0 .. U0 + QT - 1 of its list for this window.
template <class CF, int QT, int U0>
__device__ __forceinline__ void attn_tiles(const AttnArgs& a, const A5& L, const Win& wi, int h, int jt,
                                           const QPre<CF>& qp, const unsigned char* B, const unsigned char* smem,
                                           const int* kp) {
  const int lane = threadIdx.x & 63;
  const int fr = lane & 15, g4 = lane >> 4;
  const int N = L.N;
  // table addresses are taken from the LDS base: the query offsets and the
  // -inf slot carry the table's own offset
  const unsigned char* tabb = smem;
  constexpr int ES = CF::kTabEs;
  const int zone = L.zone;
  const int* lp = reinterpret_cast<const int*>(B + L.off_lp);
  int masked = 0;
#pragma unroll
  for (int i = 0; i < CF::kWaves; ++i) masked |= reinterpret_cast<const int*>(B + L.off_red)[i];

  QState<QT> st;
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qs = 16 * (jt + CF::kWaves * (U0 + u)) + fr;
    // the query's key group: same table base (plus its temporal index) and label
    const int ps = pair_slot(qs >> 2);
    st.qaddr[u] = (int)L.off_tab + ES * L.A - kp[ps] - ES * (qs & 3) * L.Rp;
    if constexpr (CF::kPerKey)
      st.qlab[u] = (int)(((uint32_t)lp[ps] >> (8 * (qs & 3)) & 0xffu) * 0x01010101u);
    else
      st.qlab[u] = lp[ps];
    u32x4_t qv = qp.q[U0 + u];
    if (L.qscale != 1.0f) {
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[e] = pack_bf16x2(bflo(qv[e]) * L.qscale, bfhi(qv[e]) * L.qscale);
    }
    st.q[u] = __builtin_bit_cast(bf16x8_t, qv);
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
  // P = exp2(x) with no max first; softmax is shift invariant, so the result
  // stands unless some row left the safe range: its sum outside
  // [2^-100, 2^100] (overflow, or all of the row's terms tiny) or a
  // non-finite accumulator.  Then the wave redoes its tiles with the exact
  // row max subtracted.
  bool exact = L.force_max != 0;
  if (!exact) {
    clear();
    if (masked) attn_pass<0, true, QT, CF>(B, L, tabb, kp2, zone, ones, st);
    else attn_pass<0, false, QT, CF>(B, L, tabb, kp2, zone, ones, st);
    bool bad = false;
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int qs = 16 * (jt + CF::kWaves * (U0 + u)) + fr;
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
  bf16_t* Og = reinterpret_cast<bf16_t*>(a.o);
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qs = 16 * (jt + CF::kWaves * (U0 + u)) + fr;
    if (qs >= N) continue;
    const float inv = __builtin_amdgcn_rcpf(st.os[u][0]);
    if (a.lse && g4 == 0)
      a.lse[(int64_t)wi.mem * N + qs] = __builtin_amdgcn_logf(st.os[u][0]) + (exact ? st.mrow[u] : 0.f);
    u32x4_t pk;
    pk[0] = pack_bf16x2(st.o0[u][0] * inv, st.o0[u][1] * inv);
    pk[1] = pack_bf16x2(st.o0[u][2] * inv, st.o0[u][3] * inv);
    pk[2] = pack_bf16x2(st.o1[u][0] * inv, st.o1[u][1] * inv);
    pk[3] = pack_bf16x2(st.o1[u][2] * inv, st.o1[u][3] * inv);
    *reinterpret_cast<u32x4_t*>(Og + ((int64_t)wi.w * N + qs) * a.C + h * 32 + 8 * g4) = pk;
  }
}

// tiles U0 .. U0 + cnt - 1 (cnt <= 4) of the wave's list for this window
template <class CF, int U0>
__device__ __forceinline__ void tiles_dispatch(int cnt, const AttnArgs& a, const A5& L, const Win& wi, int h, int jt,
                                               const QPre<CF>& qp, const unsigned char* B, const unsigned char* smem,
                                               const int* kp) {
  if constexpr (CF::kQTM >= 4) {
    if (cnt == 4) { attn_tiles<CF, 4, U0>(a, L, wi, h, jt, qp, B, smem, kp); return; }
  }
  if constexpr (CF::kQTM >= 3) {
    if (cnt == 3) { attn_tiles<CF, 3, U0>(a, L, wi, h, jt, qp, B, smem, kp); return; }
  }
  if (cnt == 2) { attn_tiles<CF, 2, U0>(a, L, wi, h, jt, qp, B, smem, kp); return; }
  if (cnt == 1) attn_tiles<CF, 1, U0>(a, L, wi, h, jt, qp, B, smem, kp);
}

// Tile t of the workgroup's run [t0, t1) belongs to wave (t - t0) mod W, so
// the waves' totals over the run differ by at most one tile.  Wave wv's
// tiles of item w: jt, jt + W, ... (cnt of them) of the item's list.
struct TileRun {
  int jt, cnt;
};
template <class CF>
__device__ __forceinline__ TileRun tile_run(int wv, int w, int t0, int t1, int QTT) {
  const int base = w * QTT;
  const int lo = t0 > base ? t0 : base, hi = t1 < base + QTT ? t1 : base + QTT;
  const int first = lo + ((wv - (lo - t0) % CF::kWaves) + CF::kWaves) % CF::kWaves;
  TileRun r;
  r.jt = first - base;
  r.cnt = first < hi ? (hi - first + CF::kWaves - 1) / CF::kWaves : 0;
  return r;
}

}  // namespace

template <class CF>
__global__ void __launch_bounds__(CF::kThreads) attn_mfma_kernel(const AttnArgs a, const A5 L) {
  warm_args_grid(a, L);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // XCD-aware order: consecutive runs (same head, neighbouring windows) go
  // to workgroups on the same XCD and its L2.
  int b = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
  // The query tiles of all (head, window) items, head-major, form one list and
  // each workgroup takes an equal contiguous run of it: with 1.5 windows per
  // workgroup every run spans exactly two windows.  A run that crosses into
  // the next head reloads the bias table at that window boundary.
  int t0, t1;
  run_bounds(L, b, t0, t1);
  if (t0 >= t1) return;
  const int i0 = (int)fdiv((uint32_t)t0, L.fdQTT), i1 = (int)fdiv((uint32_t)(t1 - 1), L.fdQTT);

  int* kp = reinterpret_cast<int*>(smem + L.off_kp);
  stage_offsets<CF>(a, L, kp);
  zero_pads<CF>(L, smem);
  QPre<CF> qcur, qnext;
  Win cur = window_of(a, L, i0);
  TileRun run = tile_run<CF>(wv, i0, t0, t1, L.QTT);
  q_load<CF>(qcur, a, L, cur.mem, run.jt, run.cnt);
  stage_kv<CF>(a, L, cur.mem, smem + L.off_buf, wv);
  tab_copy<CF>(a, L, cur.h, smem, wv);
  stage_labels<CF>(a, L, cur, smem + L.off_buf);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's direct loads are in LDS
  __syncthreads();

  // Window k of the run sits in buffer k & 1 (two buffers) or 0; the next
  // window is staged while this one is computed (after it, with one buffer).
  const int nwin = i1 - i0 + 1;
  for (int k = 0; k < nwin; ++k) {
    const int it = i0 + k;
    const int buf = L.NB == 2 ? (k & 1) : 0;
    const unsigned char* B = smem + L.off_buf + (size_t)buf * L.buf_bytes;
    const bool more = k + 1 < nwin;
    Win nxt{};
    TileRun rnext{};
    if (more) {
      nxt = window_of(a, L, it + 1);
      rnext = tile_run<CF>(wv, it + 1, t0, t1, L.QTT);
      // (BIG: after the compute, keeping its registers free)
      if constexpr (!CF::kBig) q_load<CF>(qnext, a, L, nxt.mem, rnext.jt, rnext.cnt);
      if (L.NB == 2) {
        unsigned char* Bn = smem + L.off_buf + (size_t)(buf ^ 1) * L.buf_bytes;
        stage_kv<CF>(a, L, nxt.mem, Bn, wv);
        stage_labels<CF>(a, L, nxt, Bn);
      }
    }
    if constexpr (CF::kQTM > 4) {
      tiles_dispatch<CF, 0>(run.cnt < 4 ? run.cnt : 4, a, L, cur, cur.h, run.jt, qcur, B, smem, kp);
      if (run.cnt > 4) tiles_dispatch<CF, 4>(run.cnt - 4, a, L, cur, cur.h, run.jt, qcur, B, smem, kp);
    } else {
      tiles_dispatch<CF, 0>(run.cnt, a, L, cur, cur.h, run.jt, qcur, B, smem, kp);
    }
    if (more) {
      if constexpr (CF::kBig) q_load<CF>(qnext, a, L, nxt.mem, rnext.jt, rnext.cnt);
      if (L.NB == 1) {
        __syncthreads();
        unsigned char* Bn = smem + L.off_buf;
        stage_kv<CF>(a, L, nxt.mem, Bn, wv);
        stage_labels<CF>(a, L, nxt, Bn);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (nxt.h != cur.h) {   // every wave is done with the old table
        tab_copy<CF>(a, L, nxt.h, smem, wv);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
      cur = nxt;
      run = rnext;
      qcur = qnext;
    }
  }
}

namespace {

template <class CF>
hipError_t launch_cfg(const AttnArgs& ak, const A5& L, hipStream_t st) {
  const size_t lds = a5_lds(L);
  const int per_cu = lds <= kLdsMax / 2 ? 2 : 1;
  const int64_t tiles = ak.nW * ak.heads * (int64_t)L.QTT;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  int64_t G = cap < tiles ? cap : tiles;
  if (G < ak.heads) G = ak.heads;   // every head gets a workgroup
  A5 LR = L;
  if (!set_runs(LR, tiles, G)) return hipErrorInvalidValue;
  hipError_t e = ensure_dynamic_lds((const void*)attn_mfma_kernel<CF>, lds);
  if (e != hipSuccess) return e;
  attn_mfma_kernel<CF><<<dim3((unsigned)G), dim3(CF::kThreads), lds, st>>>(ak, LR);
  return hipGetLastError();
}

}  // namespace

Tab4Geo tab4_geo(const RelTab& rel, int heads, int N) {
  Tab4Geo t{};
  t.R = rel.R;
  t.Rw = rel.Rw;
  t.TD = rel.rows / rel.R;
  t.TH = rel.R / rel.Rw;
  t.Rp = tab_rp(rel.R);
  t.scalar = N > kMfmaMaxN ? 1 : 0;
  t.TS4 = t.scalar ? ((t.TD + 3) * t.Rp + 1 + 3) / 4 : t.TD * t.Rp + 1;
  t.heads = heads;
  t.fdRp = make_fastdiv((uint32_t)t.Rp);
  t.fdRw = make_fastdiv((uint32_t)t.Rw);
  return t;
}

size_t attention_workspace_bytes(const RelTab& rel, int heads, int N) {
  const Tab4Geo t = tab4_geo(rel, heads, N);
  return ((size_t)heads * t.TS4 * 16 + 255) & ~(size_t)255;
}


bool attention_mfma_supported(vswin_dtype dt, const AttnArgs& a) {
  if (dt != VSWIN_BF16 || a.d != 32) return false;
  if (a.geo.P % 4 != 0 || a.N > kMfmaBigN) return false;
  if (a.mask_m100 && !groups_uniform(a)) return false;
  A5 L;
  return plan_a5(a, L);
}

hipError_t attention_mfma(const AttnArgs& a, hipStream_t st) {
  const int64_t items = a.nW * a.heads;
  if (items <= 0) return hipSuccess;
  AttnArgs ak = a;
  // VSWIN_ATTN_MAXPASS=1 makes every wave take the exact row-max pass (test
  // hook for the path that otherwise runs only for very large logits).
  if (const char* f = getenv("VSWIN_ATTN_MAXPASS")) ak.force_max = atoi(f) != 0;
  A5 L;
  if (!plan_a5(ak, L) || !ak.tab4) return hipErrorInvalidValue;
  if (!ak.tab_ready) {
    attn_table_kernel<<<dim3((unsigned)((L.TS4 + 255) / 256), (unsigned)L.heads), dim3(256), 0, st>>>(
        reinterpret_cast<const bf16_t*>(ak.table), reinterpret_cast<f32x4_t*>(ak.tab4), L);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool uniform = groups_uniform(ak);
  if (ak.mask_m100) {
    if (!uniform) return hipErrorInvalidValue;
    if (L.tg.scalar) return launch_cfg<Cfg<8, 8, true, true>>(ak, L, st);
    return launch_cfg<Cfg<8, 4, false, true>>(ak, L, st);
  }
  if (!uniform) {
    if (L.tg.scalar) return launch_cfg<Cfg<8, 8, true, false, true>>(ak, L, st);
    return launch_cfg<Cfg<8, 4, false, false, true>>(ak, L, st);
  }
  if (L.tg.scalar) return launch_cfg<Cfg<8, 8, true>>(ak, L, st);
  return launch_cfg<Cfg<8, 4>>(ak, L, st);
}

// ===========================================================================
// Backward of the window attention (training), bf16, head_dim 32.
//
// Per (window, head) item, with P = exp2(S2 - lse2) recomputed from the
// forward's log2-domain logits S2 = q' k^T + B log2(e) (q' = q log2(e) /
// sqrt(d)) and the forward's row normaliser lse2:
//   dP = dO v^T,  D_i = sum_e dO_ie O_ie,  dS = P (dP - D)   (natural logits)
//   dv = P^T dO,  dk = dS^T q' / log2(e),  dq = dS k / sqrt(d),
//   dB[offset(i, j), h] += dS_ij          (the relative-position table)
// Two MFMA kernels, one workgroup per item:
//   attn_bwd_kv: each wave owns 16-key tiles and sweeps every query; S and
//     dP come out as (4 queries x 1 key) per lane, so P and dS are already
//     the B operand of dV^T = dO^T P and dK^T = q'^T dS over 32 queries (the
//     transposes staged in pair order), and dS goes into an LDS copy of the
//     head's table gradient (flushed with global atomics);
//   attn_bwd_q: each wave owns 16-query tiles and sweeps every key, S^T and
//     dP^T as in the forward (4 keys x 1 query per lane), dQ^T = k^T dS^T.
// attn_bwd_prep writes the padded row copies (q', k, v, dO), the pair-order
// transposes (q'^T, k^T, dO^T) and D.  The bias table is read in the scalar
// form (a tuple is 4 floats Rp apart; query-side tuples run backwards).
// ===========================================================================
namespace {

struct BwdL {
  A5 L;                       // geometry, table extents, scalar table form
  int pitch;                  // transposed LDS rows: 16-byte chunks, 4 mod 16
  // kernel A LDS
  uint32_t a_q, a_do, a_qt, a_dot, a_lse, a_D, a_lds;
  int ap, mhw;                // temporal groups per window (P / 4), spatial cells (Mh * Mw)
  int gf;                     // windows over 512 tokens: row fragments read from global memory (L2), not LDS
  // kernel B LDS
  uint32_t b_k, b_v, b_kt, b_lds;
  // workgroups per (head, window) item of kernels A and B: part p owns tiles
  // p, p + parts, ... (more than one when that evens out the workgroups per CU)
  int parts;
};

// Stored diagonal sums of dS per item: record (query group mq, key group mk)
// of 7 floats (temporal diagonals -3 .. 3) at ((mk / 4) ng + mq) 4 + mk % 4,
// ng = N / 4 groups: a key tile's 4 key groups and 4 consecutive query groups
// are 16 adjacent records, one contiguous store per wave and step.
__host__ __device__ __forceinline__ int64_t dgrp_floats(int N) {
  const int ng = N / 4;
  return (int64_t)((ng + 3) / 4) * ng * 4 * 7;
}
__host__ __device__ __forceinline__ int64_t dgrp_rec(int ng, int mq, int mk) {
  return ((int64_t)(mk >> 2) * ng + mq) * 4 + (mk & 3);
}

__device__ __forceinline__ void stage_rows16(const bf16_t* src, unsigned char* dst, int nrows, int wv, int nw) {
  const int lane = threadIdx.x & 63;
  const int off = (lane >> 2) * 32 + (((lane & 3) ^ ((lane >> 4) & 3)) << 3);
  for (int b = wv; b < nrows / 16; b += nw)
    __builtin_amdgcn_global_load_lds(src + b * 512 + off, (lds_ptr_t)(dst + b * 1024), 16, 0, 0);
}

// 32 rows of NPAD bf16 (pair order already applied) into rows of `pitch`
// 16-byte chunks, chunk c of row d at c ^ ((d >> 3) & 3)
__device__ __forceinline__ void stage_trows(const bf16_t* src, unsigned char* dst, int NPAD, int pitch, int wv,
                                            int nw) {
  const int lane = threadIdx.x & 63;
  const int kc = NPAD / 8;
  const int nb = (kc + 63) / 64;
  for (int x = wv; x < 32 * nb; x += nw) {
    const int d = x / nb, base = 64 * (x - d * nb);
    const int slot = base + lane;
    if (slot < kc)
      __builtin_amdgcn_global_load_lds(src + (size_t)d * NPAD + ((slot ^ ((d >> 3) & 3)) << 3),
                                       (lds_ptr_t)(dst + ((size_t)d * pitch + base) * 16), 16, 0, 0);
  }
}

__device__ __forceinline__ void stage_f32(const float* src, unsigned char* dst, int n, int wv, int nw) {
  const int lane = threadIdx.x & 63;
  const int nc = n / 4;
  for (int b = wv; b * 64 < nc; b += nw)
    if (64 * b + lane < nc)
      __builtin_amdgcn_global_load_lds(src + 4 * (64 * b + lane), (lds_ptr_t)(dst + 1024 * b), 16, 0, 0);
}

// a lane's value from the lane its quad permutation selects (DPP quad_perm:
// 0xB1 swaps neighbours, 0x4E swaps pairs)
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor(float v, int ctrl) {
  return ctrl == 0xB1 ? quad_perm<0xB1>(v) : quad_perm<0x4E>(v);
}

__device__ __forceinline__ bf16x8_t pack8f(const float* v) {
  u32x4_t p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  return __builtin_bit_cast(bf16x8_t, p);
}

// 8 waves, scalar table (byte step 4); group labels, or one label byte per key
using BwdCF = Cfg<8, 8, true>;
using BwdCFKey = Cfg<8, 8, true, false, true>;

// label of element i (temporal position 4a + i) of a group's label word
template <class CF>
__device__ __forceinline__ int elem_label(int word, int i) {
  if constexpr (CF::kPerKey) return (int)(((uint32_t)word >> (8 * i)) & 0xffu);
  else return word;
}

// P of one (query, key) pair from its log2-domain logit: same region -> exp2(s2 - lse2);
// another region -> 0, or with the -100 mask exp2(s2 - 100 log2(e) - lse2)
__device__ __forceinline__ float pair_p(bool in_range, bool same, int m100, float s2, float l2) {
  const float x = same ? s2 - l2 : s2 - 100.0f * kLog2e - l2;
  return in_range && (same || m100) ? __builtin_amdgcn_exp2f(x) : 0.f;
}

}  // namespace

__global__ void __launch_bounds__(256) attn_bwd_prep_kernel(const AttnBwdArgs b, const BwdL BL) {
  warm_args(b, BL);
  const A5& L = BL.L;
  __shared__ __attribute__((aligned(16))) bf16_t tile[64 * 40];
  // workgroup: one (item, tensor, 64-row block), so that the blocks' loads are
  // in flight together instead of one after the other
  const int nrb = (L.NPAD + 63) / 64;
  const int mem = blockIdx.x / (4 * nrb);
  const int which = (blockIdx.x / nrb) % 4;
  const int r0 = (blockIdx.x % nrb) * 64;
  const int w = (int)fdiv((uint32_t)mem, L.fdH), h = mem - w * L.heads;
  const int N = L.N, NPAD = L.NPAD, C = b.a.C;
  const int t = threadIdx.x;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(b.a.q);
  const bf16_t* k = reinterpret_cast<const bf16_t*>(b.a.k);
  const bf16_t* vt = reinterpret_cast<const bf16_t*>(b.a.v);
  const bf16_t* o = reinterpret_cast<const bf16_t*>(b.a.o);
  const bf16_t* dout = reinterpret_cast<const bf16_t*>(b.dout);
  {   // which: q', k, dO (+ D), v
    bf16_t* rows = which == 0 ? b.qr : which == 1 ? b.kr : which == 2 ? b.dor : b.vr;
    bf16_t* tr = which == 0 ? b.qt : which == 1 ? b.kt : b.dot;
    {
      if (which < 3) {
        // thread t: row r0 + t / 4, 8 channels 8 (t % 4) ..
        const int r = r0 + (t >> 2), c = t & 3;
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        float dsum = 0.f;
        if (r < N) {
          const bf16_t* src = which == 0 ? q + ((int64_t)mem * N + r) * 32
                            : which == 1 ? k + ((int64_t)mem * N + r) * 32
                                         : dout + ((int64_t)w * N + r) * C + h * 32;
          v = *reinterpret_cast<const u32x4_t*>(src + 8 * c);
          if (which == 0 && L.qscale != 1.0f) {   // the forward's q' (same rounding as its q load)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(bflo(v[e]) * L.qscale, bfhi(v[e]) * L.qscale);
          }
          if (which == 2) {
            const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(o + ((int64_t)w * N + r) * C + h * 32 + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) dsum += bflo(v[e]) * bflo(ov[e]) + bfhi(v[e]) * bfhi(ov[e]);
          }
        }
        if (which == 2) {
          dsum += __shfl_xor(dsum, 1);
          dsum += __shfl_xor(dsum, 2);
          if (c == 0 && r < NPAD) b.D[(int64_t)mem * NPAD + r] = dsum;
        }
        if (r < NPAD) *reinterpret_cast<u32x4_t*>(rows + ((int64_t)mem * NPAD + r) * 32 + 8 * c) = v;
        *reinterpret_cast<u32x4_t*>(tile + (t >> 2) * 40 + 8 * c) = v;
        __syncthreads();
        // thread t: dim t / 8, output chunk t % 8 of the 64 rows (pair order
        // inside each 32-row block: chunk g holds rows 4g..4g+3, 16+4g..16+4g+3)
        const int d = t >> 3, cc = t & 7, pl = cc >> 2, g = cc & 3;
        if (r0 + 32 * pl < NPAD) {
          float vals[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vals[e] = bf2f(tile[(32 * pl + 16 * (e >> 2) + 4 * g + (e & 3)) * 40 + d]);
          *reinterpret_cast<bf16x8_t*>(tr + ((int64_t)mem * 32 + d) * NPAD + r0 + 8 * cc) = pack8f(vals);
        }
        __syncthreads();
      } else {
        // V^T -> rows: thread t: dim t / 8, keys r0 + 8 (t % 8) .. + 7
        const int d = t >> 3, kc = t & 7;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int key = r0 + 8 * kc + 4 * hh;
          u32x2_t v = u32x2_t{0u, 0u};
          if (key < N) v = *reinterpret_cast<const u32x2_t*>(vt + ((int64_t)mem * 32 + d) * N + key);
          tile[(8 * kc + 4 * hh + 0) * 40 + d] = (bf16_t)(v[0] & 0xffffu);
          tile[(8 * kc + 4 * hh + 1) * 40 + d] = (bf16_t)(v[0] >> 16);
          tile[(8 * kc + 4 * hh + 2) * 40 + d] = (bf16_t)(v[1] & 0xffffu);
          tile[(8 * kc + 4 * hh + 3) * 40 + d] = (bf16_t)(v[1] >> 16);
        }
        __syncthreads();
        const int r = r0 + (t >> 2), c = t & 3;
        if (r < NPAD)
          *reinterpret_cast<u32x4_t*>(rows + ((int64_t)mem * NPAD + r) * 32 + 8 * c) =
              *reinterpret_cast<const u32x4_t*>(tile + (t >> 2) * 40 + 8 * c);
        __syncthreads();
      }
    }
  }
}

template <class CF, bool GF>
__global__ void __launch_bounds__(512) attn_bwd_kv_kernel(const AttnBwdArgs b, const BwdL BL) {
  warm_args(b, BL);
  constexpr int ES = CF::kTabEs;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const A5& L = BL.L;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, fr = lane & 15, g4 = lane >> 4;
  const int part = (int)blockIdx.x % BL.parts;
  const Win wi = window_of(b.a, L, (int)blockIdx.x / BL.parts);
  const int mem = wi.mem, h = wi.h;
  const int N = L.N, NPAD = L.NPAD, Rp = L.Rp;
  const int ng = N / 4;   // key / query groups of 4 temporal positions
  int* kp = reinterpret_cast<int*>(smem + L.off_kp);
  const int* lp = reinterpret_cast<const int*>(smem + L.off_lp);
  stage_offsets<CF>(b.a, L, kp);
  stage_labels<CF>(b.a, L, wi, smem);
  if constexpr (!GF) {
    stage_rows16(b.qr + (int64_t)mem * NPAD * 32, smem + BL.a_q, NPAD, wv, CF::kWaves);
    stage_rows16(b.dor + (int64_t)mem * NPAD * 32, smem + BL.a_do, NPAD, wv, CF::kWaves);
  }
  stage_trows(b.qt + (int64_t)mem * 32 * NPAD, smem + BL.a_qt, NPAD, BL.pitch, wv, CF::kWaves);
  stage_trows(b.dot + (int64_t)mem * 32 * NPAD, smem + BL.a_dot, NPAD, BL.pitch, wv, CF::kWaves);
  stage_f32(b.lse + (int64_t)mem * N, smem + BL.a_lse, N, wv, CF::kWaves);
  stage_f32(b.D + (int64_t)mem * NPAD, smem + BL.a_D, NPAD, wv, CF::kWaves);
  tab_copy<CF>(b.a, L, h, smem, wv);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const unsigned char* tabb = smem;
  const float* lse = reinterpret_cast<const float*>(smem + BL.a_lse);
  const float* Dl = reinterpret_cast<const float*>(smem + BL.a_D);
  const int sw = (fr >> 2) & 3;
  bf16_t* dqkv = b.dqkv;
  const int C = b.a.C;
  // The wave's key tiles kt = part + parts (wv + 8 j), two per pass (their
  // query-side operands read once for both), then a last single one.
  auto tiles = [&](auto kt_count, int ktA, int ktB) {
    constexpr int KT = decltype(kt_count)::value;
    const int kts[2] = {ktA, ktB};
    int key[KT], klab[KT], kadd[KT];
    bool kval[KT];
    bf16x8_t kf[KT], vf[KT];
    f32x4_t dv0[KT], dv1[KT], dk0[KT], dk1[KT];
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      key[u] = kts[u] * 16 + fr;
      kf[u] = *reinterpret_cast<const bf16x8_t*>(b.kr + ((int64_t)mem * NPAD + key[u]) * 32 + 8 * g4);
      vf[u] = *reinterpret_cast<const bf16x8_t*>(b.vr + ((int64_t)mem * NPAD + key[u]) * 32 + 8 * g4);
      const int kps = pair_slot(key[u] >> 2);
      klab[u] = elem_label<CF>(lp[kps], key[u] & 3);
      kadd[u] = (int)L.off_tab + ES * L.A + kp[kps] + ES * (key[u] & 3) * Rp;
      kval[u] = key[u] < N;
      dv0[u] = dv1[u] = dk0[u] = dk1[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int qb = 0; qb < NPAD; qb += 32) {
      float pv[KT][8], dsv[KT][8];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int qs0 = qb + 16 * s;
        const int qr = qs0 + fr;
        bf16x8_t qa, da;
        if constexpr (GF) {
          qa = *reinterpret_cast<const bf16x8_t*>(b.qr + ((int64_t)mem * NPAD + qr) * 32 + 8 * g4);
          da = *reinterpret_cast<const bf16x8_t*>(b.dor + ((int64_t)mem * NPAD + qr) * 32 + 8 * g4);
        } else {
          qa = *reinterpret_cast<const bf16x8_t*>(smem + BL.a_q + qr * 64 + ((g4 ^ sw) << 4));
          da = *reinterpret_cast<const bf16x8_t*>(smem + BL.a_do + qr * 64 + ((g4 ^ sw) << 4));
        }
        const int qps = pair_slot((qs0 + 4 * g4) >> 2);
        const int qlw = lp[qps];
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lse + qs0 + 4 * g4);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(Dl + qs0 + 4 * g4);
        const int mq = (qs0 >> 2) + g4;
#pragma unroll
        for (int u = 0; u < KT; ++u) {
          const int base = kadd[u] - kp[qps];   // query temporal i: - i Rp
          const float* tp = reinterpret_cast<const float*>(tabb + base);
          const f32x4_t tb = f32x4_t{tp[0], tp[-Rp], tp[-2 * Rp], tp[-3 * Rp]};
          const f32x4_t s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[u], tb, 0, 0, 0);
          const f32x4_t dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da, vf[u], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          float dsl[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float P = pair_p(kval[u] && qs0 + 4 * g4 + i < N, elem_label<CF>(qlw, i) == klab[u],
                                   b.a.mask_m100, s2[i], l4[i]);
            const float ds = P * (dp[i] - d4[i]);
            pv[u][4 * s + i] = P;
            dsv[u][4 * s + i] = ds;
            dsl[i] = ds;
          }
          // dS toward the table gradient.  The 4 lanes of a key group (kk =
          // fr & 3, one quad) hold the 16 pairs of one (query group, key
          // group); pair (kk, i) belongs to the table entry of temporal
          // diagonal kk - i, so the quad forms the 7 diagonal sums (DPP
          // within the quad) and stores them, each (query group, key group)
          // once, for attn_bwd_grp_sum / attn_bwd_dtab_gather: no atomics.
          const int kk = fr & 3;
          float mine0 = 0.f, mine1 = 0.f;
#pragma unroll
          for (int dd = -3; dd <= 3; ++dd) {
            const int i = kk - dd;
            float v = i == 0 ? dsl[0] : i == 1 ? dsl[1] : i == 2 ? dsl[2] : i == 3 ? dsl[3] : 0.f;
            v += quad_xor(v, 0xB1);
            v += quad_xor(v, 0x4E);
            if (dd == kk - 3) mine0 = v;
            if (dd == kk + 1) mine1 = v;
          }
          const int mk = 4 * kts[u] + (fr >> 2);
          if (mq < ng && mk < ng) {
            float* dp7 = b.dgrp + (int64_t)mem * dgrp_floats(N) + dgrp_rec(ng, mq, mk) * 7;
            dp7[kk] = mine0;
            if (kk < 3) dp7[kk + 4] = mine1;
          }
        }
      }
      const int ch = qb / 8 + g4;
      const unsigned char* t0 = smem + (fr * BL.pitch + (ch ^ ((fr >> 3) & 3))) * 16;
      const unsigned char* t1 = smem + ((16 + fr) * BL.pitch + (ch ^ (((16 + fr) >> 3) & 3))) * 16;
      const bf16x8_t do0 = *reinterpret_cast<const bf16x8_t*>(t0 + BL.a_dot);
      const bf16x8_t do1 = *reinterpret_cast<const bf16x8_t*>(t1 + BL.a_dot);
      const bf16x8_t qt0 = *reinterpret_cast<const bf16x8_t*>(t0 + BL.a_qt);
      const bf16x8_t qt1 = *reinterpret_cast<const bf16x8_t*>(t1 + BL.a_qt);
#pragma unroll
      for (int u = 0; u < KT; ++u) {
        const bf16x8_t pb = pack8f(pv[u]), db = pack8f(dsv[u]);
        dv0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(do0, pb, dv0[u], 0, 0, 0);
        dv1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(do1, pb, dv1[u], 0, 0, 0);
        dk0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt0, db, dk0[u], 0, 0, 0);
        dk1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt1, db, dk1[u], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < KT; ++u) {
      if (!kval[u]) continue;
      // lane: dims 4 g4 .. + 3 (and + 16) of key `key`
      bf16_t* row = dqkv + ((int64_t)wi.w * N + key[u]) * 3 * C + h * 32 + 4 * g4;
      const float ks = b.dk_scale;
      *reinterpret_cast<u32x2_t*>(row + 2 * C) =
          u32x2_t{pack_bf16x2(dv0[u][0], dv0[u][1]), pack_bf16x2(dv0[u][2], dv0[u][3])};
      *reinterpret_cast<u32x2_t*>(row + 2 * C + 16) =
          u32x2_t{pack_bf16x2(dv1[u][0], dv1[u][1]), pack_bf16x2(dv1[u][2], dv1[u][3])};
      *reinterpret_cast<u32x2_t*>(row + C) =
          u32x2_t{pack_bf16x2(dk0[u][0] * ks, dk0[u][1] * ks), pack_bf16x2(dk0[u][2] * ks, dk0[u][3] * ks)};
      *reinterpret_cast<u32x2_t*>(row + C + 16) =
          u32x2_t{pack_bf16x2(dk1[u][0] * ks, dk1[u][1] * ks), pack_bf16x2(dk1[u][2] * ks, dk1[u][3] * ks)};
    }
  };
  const int kstep = BL.parts * CF::kWaves;
  int kt = part + BL.parts * wv;
  for (; (kt + kstep) * 16 < N; kt += 2 * kstep) tiles(std::integral_constant<int, 2>{}, kt, kt + kstep);
  if (kt * 16 < N) tiles(std::integral_constant<int, 1>{}, kt, kt);
}

template <class CF, bool GF>
__global__ void __launch_bounds__(512) attn_bwd_q_kernel(const AttnBwdArgs b, const BwdL BL) {
  warm_args(b, BL);
  constexpr int ES = CF::kTabEs;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const A5& L = BL.L;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, fr = lane & 15, g4 = lane >> 4;
  const int part = (int)blockIdx.x % BL.parts;
  const Win wi = window_of(b.a, L, (int)blockIdx.x / BL.parts);
  const int mem = wi.mem, h = wi.h;
  const int N = L.N, NPAD = L.NPAD, Rp = L.Rp;
  int* kp = reinterpret_cast<int*>(smem + L.off_kp);
  const int* lp = reinterpret_cast<const int*>(smem + L.off_lp);
  stage_offsets<CF>(b.a, L, kp);
  stage_labels<CF>(b.a, L, wi, smem);
  if constexpr (!GF) {
    stage_rows16(b.kr + (int64_t)mem * NPAD * 32, smem + BL.b_k, NPAD, wv, CF::kWaves);
    stage_rows16(b.vr + (int64_t)mem * NPAD * 32, smem + BL.b_v, NPAD, wv, CF::kWaves);
  }
  stage_trows(b.kt + (int64_t)mem * 32 * NPAD, smem + BL.b_kt, NPAD, BL.pitch, wv, CF::kWaves);
  tab_copy<CF>(b.a, L, h, smem, wv);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const unsigned char* tabb = smem;
  const int sw = (fr >> 2) & 3;
  const int C = b.a.C;
  // The wave's query tiles qt = part + parts (wv + 8 j), two per pass (their
  // key-side operands read once for both), then a last single one.
  auto tiles = [&](auto qt_count, int qtA, int qtB) {
    constexpr int QT = decltype(qt_count)::value;
    const int qts[2] = {qtA, qtB};
    int q[QT], qlab[QT], qaddr[QT];
    bool qval[QT];
    float l2[QT], Dq[QT];
    bf16x8_t qf[QT], df[QT];
    f32x4_t dq0[QT], dq1[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      q[u] = qts[u] * 16 + fr;
      qval[u] = q[u] < N;
      qf[u] = *reinterpret_cast<const bf16x8_t*>(b.qr + ((int64_t)mem * NPAD + q[u]) * 32 + 8 * g4);
      df[u] = *reinterpret_cast<const bf16x8_t*>(b.dor + ((int64_t)mem * NPAD + q[u]) * 32 + 8 * g4);
      l2[u] = qval[u] ? b.lse[(int64_t)mem * N + q[u]] : 0.f;
      Dq[u] = b.D[(int64_t)mem * NPAD + q[u]];
      const int qps = pair_slot(q[u] >> 2);
      qlab[u] = elem_label<CF>(lp[qps], q[u] & 3);
      qaddr[u] = (int)L.off_tab + ES * L.A - kp[qps] - ES * (q[u] & 3) * Rp;
      dq0[u] = dq1[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int kb = 0; kb < NPAD; kb += 32) {
      float dsv[QT][8];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int ks0 = kb + 16 * s;
        const int kr = ks0 + fr;
        bf16x8_t ka, va;
        if constexpr (GF) {
          ka = *reinterpret_cast<const bf16x8_t*>(b.kr + ((int64_t)mem * NPAD + kr) * 32 + 8 * g4);
          va = *reinterpret_cast<const bf16x8_t*>(b.vr + ((int64_t)mem * NPAD + kr) * 32 + 8 * g4);
        } else {
          ka = *reinterpret_cast<const bf16x8_t*>(smem + BL.b_k + kr * 64 + ((g4 ^ sw) << 4));
          va = *reinterpret_cast<const bf16x8_t*>(smem + BL.b_v + kr * 64 + ((g4 ^ sw) << 4));
        }
        const int kps = pair_slot((ks0 + 4 * g4) >> 2);
        const int klw = lp[kps];
#pragma unroll
        for (int u = 0; u < QT; ++u) {
          const float* tp = reinterpret_cast<const float*>(tabb + qaddr[u] + kp[kps]);
          const f32x4_t tb = f32x4_t{tp[0], tp[Rp], tp[2 * Rp], tp[3 * Rp]};
          const f32x4_t s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[u], tb, 0, 0, 0);
          const f32x4_t dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, df[u], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float P = pair_p(qval[u] && ks0 + 4 * g4 + i < N, elem_label<CF>(klw, i) == qlab[u],
                                   b.a.mask_m100, s2[i], l2[u]);
            dsv[u][4 * s + i] = P * (dp[i] - Dq[u]);
          }
        }
      }
      const int ch = kb / 8 + g4;
      const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(
          smem + BL.b_kt + (fr * BL.pitch + (ch ^ ((fr >> 3) & 3))) * 16);
      const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t*>(
          smem + BL.b_kt + ((16 + fr) * BL.pitch + (ch ^ (((16 + fr) >> 3) & 3))) * 16);
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        const bf16x8_t db = pack8f(dsv[u]);
        dq0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, db, dq0[u], 0, 0, 0);
        dq1[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, db, dq1[u], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      if (!qval[u]) continue;
      bf16_t* row = b.dqkv + ((int64_t)wi.w * N + q[u]) * 3 * C + h * 32 + 4 * g4;
      const float qs = b.dq_scale;
      *reinterpret_cast<u32x2_t*>(row) =
          u32x2_t{pack_bf16x2(dq0[u][0] * qs, dq0[u][1] * qs), pack_bf16x2(dq0[u][2] * qs, dq0[u][3] * qs)};
      *reinterpret_cast<u32x2_t*>(row + 16) =
          u32x2_t{pack_bf16x2(dq1[u][0] * qs, dq1[u][1] * qs), pack_bf16x2(dq1[u][2] * qs, dq1[u][3] * qs)};
    }
  };
  const int qstep = BL.parts * CF::kWaves;
  int qt = part + BL.parts * wv;
  for (; (qt + qstep) * 16 < N; qt += 2 * qstep) tiles(std::integral_constant<int, 2>{}, qt, qt + qstep);
  if (qt * 16 < N) tiles(std::integral_constant<int, 1>{}, qt, qt);
}

// Sum of the stored diagonal sums over the windows of each head: gsum[h][e]
// = sum_w dgrp[(w heads + h) E + e], E = dgrp_floats(N) (coalesced:
// consecutive threads take consecutive e).
__global__ void __launch_bounds__(256) attn_bwd_grp_sum_kernel(const float* __restrict__ dgrp,
                                                                float* __restrict__ gsum, int64_t nW, int heads,
                                                                int64_t E) {
  const int h = blockIdx.y;
  const int64_t e = blockIdx.x * 256 + (int64_t)threadIdx.x;
  if (e >= E) return;
  // four partial sums (windows w mod 4), combined in a fixed order
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  const float* p = dgrp + (int64_t)h * E + e;
  const int64_t stride = (int64_t)heads * E;
  int64_t w = 0;
#pragma unroll 2
  for (; w + 4 <= nW; w += 4) {
    s0 += p[w * stride];
    s1 += p[(w + 1) * stride];
    s2 += p[(w + 2) * stride];
    s3 += p[(w + 3) * stride];
  }
  for (; w < nW; ++w) s0 += p[w * stride];
  gsum[(int64_t)h * E + e] = (s0 + s1) + (s2 + s3);
}

// Table gradient in the scalar index space: entry y = (dt + TD/2) Rp +
// (dh + TH/2) Rw + (dw + Rw/2) of head h gathers, from the window sums, the
// diagonal sums of every (query group, key group) pair whose spatial cells
// differ by (dh, dw) and whose temporal groups and diagonal give
// dt = 4 (ak - aq) + dd.  One wave per entry, lanes over the query cells;
// deterministic (no atomics).
__global__ void __launch_bounds__(256) attn_bwd_dtab_gather_kernel(const float* __restrict__ gsum,
                                                                    float* __restrict__ out, const BwdL BL,
                                                                    WinGeo g) {
  warm_args(gsum, out, BL, g);
  const A5& L = BL.L;
  const int h = blockIdx.y;
  const int nd = L.TD * L.Rp;
  const int y = blockIdx.x * 4 + ((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (y >= nd) return;
  const int u = y / L.Rp, rem = y - u * L.Rp;
  const int v = rem / L.Rw, x = rem - v * L.Rw;
  const int ng = L.N / 4;
  const float* gs = gsum + (int64_t)h * dgrp_floats(L.N);
  float s = 0.f;
  if (rem < L.R) {
    const int dt = u - L.TD / 2, dh = v - L.TH / 2, dw = x - L.Rw / 2;
    for (int cq = lane; cq < BL.mhw; cq += 64) {
      const int qh = cq / g.Mw, qw = cq - qh * g.Mw;
      const int kh = qh + dh, kw = qw + dw;
      if (kh < 0 || kh >= g.Mh || kw < 0 || kw >= g.Mw) continue;
      const int ck = kh * g.Mw + kw;
      for (int aq = 0; aq < BL.ap; ++aq)
        for (int ak = 0; ak < BL.ap; ++ak) {
          const int dd = dt - 4 * (ak - aq);
          if (dd >= -3 && dd <= 3) s += gs[dgrp_rec(ng, aq * BL.mhw + cq, ak * BL.mhw + ck) * 7 + dd + 3];
        }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  // straight into the (rows, heads) table layout: entry (u, v, x) is row
  // (TD-1-u) R + (TH-1-v) Rw + (Rw-1-x), the inverse of ts_entry's index map
  // (every row has exactly one scalar index; indices with rem >= R are padding)
  if (lane == 0 && rem < L.R)
    out[((int64_t)(L.TD - 1 - u) * L.R + (L.TH - 1 - v) * L.Rw + (L.Rw - 1 - x)) * L.heads + h] = s;
}


namespace {

bool plan_bwd(const AttnArgs& a, BwdL& B) {
  B = BwdL{};
  A5& L = B.L;
  if (!plan_a5(a, L)) return false;
  // scalar table form, whatever N
  L.tg = tab4_geo(a.rel, a.heads, kMfmaMaxN + 1);
  L.TS4 = L.tg.TS4;
  const int kc = L.NPAD / 8;
  B.pitch = kc + ((4 - kc) % 16 + 16) % 16;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 15) & ~(size_t)15;
    return (uint32_t)o;
  };
  L.off_kp = take((size_t)L.NP * 8 * 4);
  L.off_lp = take((size_t)L.NP * 8 * 4);
  L.off_red = take(4 * kMaxWaves);
  L.off_tab = take((size_t)L.TS4 * 16);
  const size_t common = off;
  const size_t trows = (size_t)32 * B.pitch * 16;
  // the row copies (q', dO for the key-owned kernel, k, v for the query-owned
  // one) sit in LDS while they fit with the transposes; beyond that (windows of
  // more than 512 tokens) the MFMA row fragments come from global memory
  B.gf = (size_t)L.NPAD * 64 * 2 + 2 * trows + common + (size_t)L.NPAD * 8 > kLdsMax ? 1 : 0;
  const size_t rows = B.gf ? 0 : (size_t)L.NPAD * 64;
  B.a_q = take(rows);
  B.a_do = take(rows);
  B.a_qt = take(trows);
  B.a_dot = take(trows);
  B.a_lse = take((size_t)L.NPAD * 4);
  B.a_D = take((size_t)L.NPAD * 4);
  B.a_lds = (uint32_t)off;
  B.ap = a.geo.P / 4;
  B.mhw = a.geo.Mh * a.geo.Mw;
  off = common;
  B.b_k = take(rows);
  B.b_v = take(rows);
  B.b_kt = take(trows);
  B.b_lds = (uint32_t)off;
  L.zone = 0;
  return B.a_lds <= kLdsMax && B.b_lds <= kLdsMax;
}

}  // namespace

bool attention_bwd_supported(vswin_dtype dt, const AttnArgs& a) {
  if (!attention_mfma_supported(dt, a)) return false;
  BwdL B;
  return plan_bwd(a, B);
}

size_t attention_bwd_workspace_bytes(const AttnArgs& a) {
  BwdL B;
  if (!plan_bwd(a, B)) return 0;
  const A5& L = B.L;
  const size_t items = (size_t)a.nW * a.heads;
  const size_t arr = ((size_t)items * L.NPAD * 32 * 2 + 255) & ~(size_t)255;
  const size_t D = ((size_t)items * L.NPAD * 4 + 255) & ~(size_t)255;
  const size_t tabs = ((size_t)a.heads * L.TS4 * 16 + 255) & ~(size_t)255;
  const size_t grp = ((size_t)items * dgrp_floats(a.N) * 4 + 255) & ~(size_t)255;
  const size_t gsum = ((size_t)a.heads * dgrp_floats(a.N) * 4 + 255) & ~(size_t)255;
  return 7 * arr + D + tabs + grp + gsum;
}

hipError_t attention_bwd(const AttnBwdArgs& in, hipStream_t st) {
  const int64_t items = in.a.nW * in.a.heads;
  BwdL B;
  if (!plan_bwd(in.a, B) || !in.work || !in.dtable || !in.lse) return hipErrorInvalidValue;
  const A5& L = B.L;
  {
    // one workgroup per CU at a time (LDS): split the items so that the last
    // round of workgroups is as full as the others, when that shortens the
    // launch (e.g. 384 items on 256 CUs: 2 rounds of whole items against 3
    // rounds of halves, 1.5 items long)
    const int64_t cus = device_cu_count();
    B.parts = 1;
    double best = (double)((items + cus - 1) / cus);
    for (int p = 2; p <= 4; ++p) {
      const double t = (double)((items * p + cus - 1) / cus) / p;
      if (t < best - 1e-9 && (L.N + 15) / 16 >= p * 8) {
        best = t;
        B.parts = p;
      }
    }
  }
  AttnBwdArgs b = in;
  char* w = reinterpret_cast<char*>(in.work);
  const size_t arr = ((size_t)items * L.NPAD * 32 * 2 + 255) & ~(size_t)255;
  bf16_t** slots[7] = {&b.qr, &b.kr, &b.vr, &b.dor, &b.qt, &b.kt, &b.dot};
  for (int i = 0; i < 7; ++i) *slots[i] = reinterpret_cast<bf16_t*>(w + i * arr);
  size_t off = 7 * arr;
  b.D = reinterpret_cast<float*>(w + off);
  off += ((size_t)items * L.NPAD * 4 + 255) & ~(size_t)255;
  b.a.tab4 = w + off;
  off += ((size_t)in.a.heads * L.TS4 * 16 + 255) & ~(size_t)255;
  b.dgrp = reinterpret_cast<float*>(w + off);
  off += ((size_t)items * dgrp_floats(in.a.N) * 4 + 255) & ~(size_t)255;
  float* gsum = reinterpret_cast<float*>(w + off);
  b.dq_scale = 1.0f / sqrtf((float)in.a.d);
  b.dk_scale = 1.0f / kLog2e;
  if (items <= 0) return hipSuccess;
  attn_table_kernel<<<dim3((unsigned)((L.TS4 + 255) / 256), (unsigned)L.heads), dim3(256), 0, st>>>(
      reinterpret_cast<const bf16_t*>(in.a.table), reinterpret_cast<f32x4_t*>(b.a.tab4), L);
  attn_bwd_prep_kernel<<<dim3((unsigned)(items * 4 * ((L.NPAD + 63) / 64))), dim3(256), 0, st>>>(b, B);
  auto run = [&](auto kv, auto qk) -> hipError_t {
    hipError_t e = ensure_dynamic_lds((const void*)kv, B.a_lds);
    if (e != hipSuccess) return e;
    e = ensure_dynamic_lds((const void*)qk, B.b_lds);
    if (e != hipSuccess) return e;
    kv<<<dim3((unsigned)(items * B.parts)), dim3(512), B.a_lds, st>>>(b, B);
    qk<<<dim3((unsigned)(items * B.parts)), dim3(512), B.b_lds, st>>>(b, B);
    return hipGetLastError();
  };
  const bool uni = groups_uniform(in.a);
  hipError_t e;
  if (B.gf)
    e = uni ? run(attn_bwd_kv_kernel<BwdCF, true>, attn_bwd_q_kernel<BwdCF, true>)
            : run(attn_bwd_kv_kernel<BwdCFKey, true>, attn_bwd_q_kernel<BwdCFKey, true>);
  else
    e = uni ? run(attn_bwd_kv_kernel<BwdCF, false>, attn_bwd_q_kernel<BwdCF, false>)
            : run(attn_bwd_kv_kernel<BwdCFKey, false>, attn_bwd_q_kernel<BwdCFKey, false>);
  if (e != hipSuccess) return e;
  const int64_t E = dgrp_floats(in.a.N);
  attn_bwd_grp_sum_kernel<<<dim3((unsigned)((E + 255) / 256), (unsigned)in.a.heads), dim3(256), 0, st>>>(
      b.dgrp, gsum, in.a.nW, in.a.heads, E);
  const int nd = L.TD * L.Rp;
  attn_bwd_dtab_gather_kernel<<<dim3((unsigned)((nd + 3) / 4), (unsigned)in.a.heads), dim3(256), 0, st>>>(
      gsum, in.dtable, B, in.a.geo);
  return hipGetLastError();
}

}  // namespace vswin
