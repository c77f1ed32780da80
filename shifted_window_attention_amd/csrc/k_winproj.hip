// Window projections of the attention branch for C in {96, 128} (bf16):
//
//   qkv_proj:  window rows  <- LN1(x) gathered through pad + roll + partition
//              (eq. 1, first line; the mmaction2 walk-through's op order),
//              q, k, v       = rows * Wqkv^T + bqkv, split by head (eq. 2 input)
//   out_proj:  z[token]      = x[token] + o[row] * Wproj^T + bproj, scattered
//              back through reverse partition + roll + crop (eq. 1 residual)
//
// Both keep the weight matrix resident in LDS in a persistent workgroup per
// CU slot; each wave owns 16-row tiles from gather to store with the next
// tile's rows fetched while the current one computes, and no barrier after
// the weight load.  v_mfma_f32_16x16x32_bf16, K = C in C/32 steps.
//
// Register layouts.  Lane (fr, g) of a wave holds columns 32j + 8g .. + 7
// (j < C/32) of tile row fr: exactly its k-chunks of an MFMA operand, so LN
// runs in registers (4 lanes share a row: xor 16, 32) and the same registers
// serve as the A operand (rows on the MFMA row side: V^T) or the B operand.
// Weight rows of each 32-feature group are read in pair order (tile p, row
// 4g + i holds feature 8g + 4p + i), so after a tile pair a lane holds 8
// consecutive output features of its row: one 16-byte store.  V^T comes out
// of the swapped product with 4 consecutive tokens of one feature per lane.
//
// LDS weight rows: 16-byte chunk q of row r at q ^ ((r >> 2) & 3) for
// 192-byte rows (C = 96), at q ^ (r & 15) for 256-byte rows (C = 128):
// conflict-free fragment reads.
#include "vswin_kernels.h"

namespace vswin {

namespace {

constexpr int kWpWaves = 8;
constexpr int kWpThreads = 64 * kWpWaves;

// LDS row of weight feature f when the features of each 32-group are read
// in pair order: f = 8g + 4p + i -> 16p + 4g + i.
__device__ __forceinline__ int pair_row(int f) {
  return (f & ~31) | (((f >> 2) & 1) << 4) | (((f >> 3) & 3) << 2) | (f & 3);
}

__device__ __forceinline__ void unpack8(const u32x4_t& v, float f[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bflo(v[e]);
    f[2 * e + 1] = bfhi(v[e]);
  }
}
__device__ __forceinline__ u32x4_t pack8(const float f[8]) {
  u32x4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
  return v;
}

template <int C>
__device__ __forceinline__ int wswz(int r) {
  return C == 128 ? (r & 15) : ((r >> 2) & 3);
}

__device__ __forceinline__ int pair_row_inv(int r) {
  return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Weight matrix (F x C, row-major) into LDS by direct global-to-LDS loads
// (no registers): LDS row r holds weight row inv(r), its 16-byte chunks
// swizzled; a wave instruction fills 1 KB of consecutive LDS chunks (lane i:
// chunk 64 b + i), each lane loading the global chunk that belongs there.
// The caller waits for vmcnt and a barrier.
template <int C, int F, int THREADS = kWpThreads, class Inv>
__device__ __forceinline__ void stage_weights(const bf16_t* __restrict__ W, unsigned char* Ws, Inv inv) {
  constexpr int KC = C / 8;
  constexpr int NB = F * KC / 64;
  static_assert(NB * 64 == F * KC, "weight staging shape");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  for (int b = wave; b < NB; b += THREADS / 64) {
    const int c = 64 * b + lane;
    const int r = c / KC, qp = c - r * KC;
    __builtin_amdgcn_global_load_lds(W + (int64_t)inv(r) * C + ((qp ^ wswz<C>(r)) << 3),
                                     (lds_ptr_t)(Ws + 1024 * b), 16, 0, 0);
  }
}

// one 16-byte weight fragment: rows r0 + fr (r0 a multiple of 16), k-chunk kc
template <int C>
__device__ __forceinline__ bf16x8_t wfrag(const unsigned char* Ws, int r0, int fr, int kc) {
  const int r = r0 + fr;
  return *reinterpret_cast<const bf16x8_t*>(Ws + r * (C * 2) + ((kc ^ wswz<C>(r)) << 4));
}

}  // namespace

struct QkvParams {
  const bf16_t* x;      // token rows (B*T*H*W, C)
  const bf16_t* ln_g;   // LN1 gamma, beta (C); ln == 0: rows are taken as they are
  const bf16_t* ln_b;
  float eps;
  int ln;
  const bf16_t* w;      // (3C, C)
  const bf16_t* bias;   // (3C) or NULL
  bf16_t *q, *k, *v;    // (nW*heads, N, d); v transposed (nW*heads, d, N) when vt
  int vt;
  float qscale;         // multiplier of q after the bias
  int M;                // window rows (nW * N)
  int heads, d;
  FastDiv fd;           // division by d
  WinGeo geo;
  // the attention's prepared tables (tg) of `table` go to tab4 (none when
  // tab4 is NULL): written by the waves that get no tile when tab_idle, else
  // by the workgroups from tile_blocks on
  int tile_blocks;
  int tab_idle;
  const bf16_t* table;
  f32x4_t* tab4;
  Tab4Geo tg;
};

namespace {

template <int C>
struct QkvLds {
  static constexpr size_t w = (size_t)3 * C * C * 2;
  static constexpr size_t bytes = w + (size_t)5 * C * 2;   // + bias (3C), LN gamma, beta
};

// tile rows of one wave: lane (fr, g) holds columns 32j + 8g .. + 7 of row fr
template <int C>
struct RowTile {
  u32x4_t a[C / 32];
  int live;             // the row is a real token (not a pad slot, not past the end)
};

// gathered window rows of x (zeros for pad slots and rows past M)
template <int C>
__device__ __forceinline__ void gather_rows(RowTile<C>& rt, const QkvParams& pr, int64_t t) {
  const int lane = threadIdx.x & 63, fr = lane & 15, g = lane >> 4;
  const int m = (int)(t * 16) + fr;
  int64_t src = -1;
  if (m < pr.M) {
    int lab;
    src = row_source(pr.geo, m, lab);
  }
  rt.live = src >= 0;
#pragma unroll
  for (int j = 0; j < C / 32; ++j)
    rt.a[j] = src >= 0 ? *reinterpret_cast<const u32x4_t*>(pr.x + src * C + 32 * j + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

// One workgroup of 16 waves per CU (four waves per SIMD), the weights staged
// once per CU.
constexpr int kQkvWaves = 16;
constexpr int kQkvThreads = 64 * kQkvWaves;

template <int C>
__global__ void __launch_bounds__(kQkvThreads, 1) qkv_wave_kernel(QkvParams pr) {
  warm_args_grid(pr);
  using L = QkvLds<C>;
  constexpr int KS = C / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  if ((int)blockIdx.x >= pr.tile_blocks) {
    const int n = pr.tg.TS4 * pr.tg.heads;
    for (int e = ((int)blockIdx.x - pr.tile_blocks) * kQkvThreads + (int)threadIdx.x; e < n;
         e += ((int)gridDim.x - pr.tile_blocks) * kQkvThreads) {
      const int h = e / pr.tg.TS4;
      pr.tab4[e] = tab_entry(pr.table, pr.tg, h, e - h * pr.tg.TS4);
    }
    return;
  }
  unsigned char* Ws = lds;
  bf16_t* bias_s = reinterpret_cast<bf16_t*>(lds + L::w);   // 3C bias, then LN gamma (C), beta (C)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, g = lane >> 4;
  const int64_t ntiles = ((int64_t)pr.M + 15) / 16;
  const int64_t nw = (int64_t)pr.tile_blocks * kQkvWaves;
  int64_t t = (int64_t)blockIdx.x * kQkvWaves + wave;
  const int vt = pr.vt;
  if (pr.tab4 && pr.tab_idle && t >= ntiles) {
    const int n = pr.tg.TS4 * pr.tg.heads;
    const int nidle = (int)(nw - ntiles);
    for (int e = (int)(t - ntiles) * 64 + lane; e < n; e += nidle * 64) {
      const int h = e / pr.tg.TS4;
      pr.tab4[e] = tab_entry(pr.table, pr.tg, h, e - h * pr.tg.TS4);
    }
  }

  RowTile<C> cur;
  if (t < ntiles) gather_rows<C>(cur, pr, t);
  // q and k rows (and v rows unless transposed) in pair order
  stage_weights<C, 3 * C, kQkvThreads>(pr.w, Ws, [vt](int r) { return (r < 2 * C || !vt) ? pair_row_inv(r) : r; });
  for (int c = tid; c < 5 * C / 8; c += kQkvThreads) {
    const bf16_t* src = c < 3 * C / 8 ? (pr.bias ? pr.bias + c * 8 : nullptr)
                                      : (!pr.ln ? nullptr
                                                : (c < 4 * C / 8 ? pr.ln_g + (c - 3 * C / 8) * 8
                                                                 : pr.ln_b + (c - 4 * C / 8) * 8));
    *reinterpret_cast<u32x4_t*>(bias_s + c * 8) = src ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0u, 0u, 0u, 0u};
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's weight blocks are in LDS
  __syncthreads();

  const int N = pr.geo.N, d = pr.d;
  for (; t < ntiles; t += nw) {
    RowTile<C> nxt;
    if (t + nw < ntiles) gather_rows<C>(nxt, pr, t + nw);
    // ---- LN1 (4 lanes per row); pad rows stay zero (the grid is padded after the norm)
    bf16x8_t af[KS];
    {
      float xv[KS][8];
#pragma unroll
      for (int j = 0; j < KS; ++j) unpack8(cur.a[j], xv[j]);
      if (pr.ln) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) s += xv[j][e];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        const float mean = s * (1.0f / C);
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float dd = xv[j][e] - mean;
            sq += dd * dd;
          }
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        const float rstd = 1.0f / sqrtf(sq * (1.0f / C) + pr.eps);
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          float gg[8], bb[8];
          unpack8(*reinterpret_cast<const u32x4_t*>(bias_s + 3 * C + 32 * j + 8 * g), gg);
          unpack8(*reinterpret_cast<const u32x4_t*>(bias_s + 4 * C + 32 * j + 8 * g), bb);
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[j][e] = cur.live ? (xv[j][e] - mean) * rstd * gg[e] + bb[e] : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < KS; ++j) af[j] = __builtin_bit_cast(bf16x8_t, pack8(xv[j]));
    }
    const int m = (int)(t * 16) + fr;
    const int w = (int)fdiv((uint32_t)m, pr.geo.fN);
    const bool mok = m < pr.M;
    // ---- q, k (and v unless transposed): 8 consecutive features of row fr
    // per lane and pair; pair jq runs over the 32-feature groups of q, k, v
    const int npair = (vt ? 2 : 3) * (C / 32);
#pragma unroll 1
    for (int jq = 0; jq < npair; ++jq) {
      const int wn = jq / (C / 32), jj = jq - wn * (C / 32);
      bf16_t* out = wn == 0 ? pr.q : (wn == 1 ? pr.k : pr.v);
      bf16_t* row = out + (int64_t)w * N * C + (m - w * N) * d;
      const float osc = wn == 0 ? pr.qscale : 1.0f;
      const int c = 32 * jj + 8 * g;
      const int h = (int)fdiv((uint32_t)c, pr.fd);
      const int coff = h * N * d + (c - h * d);
      {
        f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
          for (int p = 0; p < 2; ++p)
            acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag<C>(Ws, wn * C + 32 * jj + 16 * p, fr, 4 * kk + g),
                                                             af[kk], acc[p], 0, 0, 0);
        float b8[8], v8[8];
        unpack8(*reinterpret_cast<const u32x4_t*>(bias_s + wn * C + 32 * jj + 8 * g), b8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v8[i] = (acc[0][i] + b8[i]) * osc;
          v8[4 + i] = (acc[1][i] + b8[4 + i]) * osc;
        }
        if (mok) *reinterpret_cast<u32x4_t*>(row + coff) = pack8(v8);
      }
    }
    // ---- V^T
    if (vt) {
      // V^T: lane holds tokens 16t + 4g .. + 3 of feature 16nt + fr; N and the
      // row offset are multiples of 4, so the 4 tokens share a window
      const int m4 = (int)(t * 16) + 4 * g;
      const int w4 = (int)fdiv((uint32_t)m4, pr.geo.fN);
      bf16_t* vb = pr.v + (int64_t)w4 * C * N + (m4 - w4 * N);
#pragma unroll 1
      for (int nt = 0; nt < C / 16; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk], wfrag<C>(Ws, 2 * C + 16 * nt, fr, 4 * kk + g), acc,
                                                        0, 0, 0);
        const float b = bf2f(bias_s[2 * C + 16 * nt + fr]);
        u32x2_t pk;
        pk[0] = pack_bf16x2(acc[0] + b, acc[1] + b);
        pk[1] = pack_bf16x2(acc[2] + b, acc[3] + b);
        if (m4 < pr.M) *reinterpret_cast<u32x2_t*>(vb + (16 * nt + fr) * N) = pk;
      }
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// out_proj: o rows (window slot order) * Wproj^T + b, scattered to tokens
// ---------------------------------------------------------------------------
struct ProjParams {
  const bf16_t* o;      // (M, C) window rows
  const bf16_t* w;      // (C, C)
  const bf16_t* bias;   // (C) or NULL
  const bf16_t* res;    // residual tokens (bf16) or NULL
  void* out;            // res ? fp32 z : bf16 y, token rows
  int M;
  WinGeo geo;
};

namespace {

template <int C>
struct ProjLds {
  static constexpr size_t w = (size_t)C * C * 2;
  static constexpr size_t bytes = w + (size_t)C * 2;
};

template <int C, bool RES>
struct ProjTile {
  u32x4_t a[C / 32];    // o row fr, columns 32j + 8g .. + 7
  u32x4_t r[C / 32];    // residual x[src], same columns (RES)
  int src;
};

template <int C, bool RES>
__device__ __forceinline__ void proj_load(ProjTile<C, RES>& pt, const ProjParams& pr, int64_t t) {
  const int lane = threadIdx.x & 63, fr = lane & 15, g = lane >> 4;
  const int m = (int)(t * 16) + fr;
  int src = -1;
  if (m < pr.M) {
    int lab;
    src = (int)row_source(pr.geo, m, lab);
  }
  pt.src = src;
#pragma unroll
  for (int j = 0; j < C / 32; ++j) {
    pt.a[j] = m < pr.M ? *reinterpret_cast<const u32x4_t*>(pr.o + (int64_t)m * C + 32 * j + 8 * g)
                       : u32x4_t{0u, 0u, 0u, 0u};
    if constexpr (RES)
      pt.r[j] = src >= 0 ? *reinterpret_cast<const u32x4_t*>(pr.res + (int64_t)src * C + 32 * j + 8 * g)
                         : u32x4_t{0u, 0u, 0u, 0u};
  }
}

}  // namespace

// four waves per SIMD (two workgroups per CU): each wave's tile loads are in
// flight at once rather than prefetched a tile ahead
template <int C, bool RES>
__global__ void __launch_bounds__(kWpThreads, 4) out_proj_kernel(ProjParams pr) {
  warm_args_grid(pr);
  using L = ProjLds<C>;
  constexpr int KS = C / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* Ws = lds;
  bf16_t* bias_s = reinterpret_cast<bf16_t*>(lds + L::w);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, g = lane >> 4;
  const int64_t ntiles = ((int64_t)pr.M + 15) / 16;
  const int64_t nw = (int64_t)gridDim.x * kWpWaves;
  int64_t t = (int64_t)blockIdx.x * kWpWaves + wave;

  ProjTile<C, RES> cur;
  if (t < ntiles) proj_load<C, RES>(cur, pr, t);
  stage_weights<C, C>(pr.w, Ws, [](int r) { return pair_row_inv(r); });
  for (int c = tid; c < C / 8; c += kWpThreads)
    *reinterpret_cast<u32x4_t*>(bias_s + c * 8) =
        pr.bias ? *reinterpret_cast<const u32x4_t*>(pr.bias + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's weight blocks are in LDS
  __syncthreads();
  if (t >= ntiles) return;

  for (;;) {
    for (int jj = 0; jj < C / 32; ++jj) {
      f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfrag<C>(Ws, 32 * jj + 16 * p, fr, 4 * kk + g),
                                                           __builtin_bit_cast(bf16x8_t, cur.a[kk]), acc[p], 0, 0, 0);
      float b8[8], v8[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(bias_s + 32 * jj + 8 * g), b8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v8[i] = acc[0][i] + b8[i];
        v8[4 + i] = acc[1][i] + b8[4 + i];
      }
      // keep the next pair's fragment loads below this pair (register pressure)
      __builtin_amdgcn_sched_barrier(0);
      if (cur.src < 0) continue;   // pad slot or past the end
      const int64_t off = (int64_t)cur.src * C + 32 * jj + 8 * g;
      if constexpr (RES) {
        float r8[8];
        unpack8(cur.r[jj], r8);
        float* z = reinterpret_cast<float*>(pr.out) + off;
        *reinterpret_cast<float4*>(z) = make_float4(v8[0] + r8[0], v8[1] + r8[1], v8[2] + r8[2], v8[3] + r8[3]);
        *reinterpret_cast<float4*>(z + 4) = make_float4(v8[4] + r8[4], v8[5] + r8[5], v8[6] + r8[6], v8[7] + r8[7]);
      } else {
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(pr.out) + off) = pack8(v8);
      }
    }
    t += nw;
    if (t >= ntiles) break;
    proj_load<C, RES>(cur, pr, t);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

// persistent grid: per_cu workgroups per CU, no more than the tiles need
unsigned wave_grid(int64_t M, int per_cu) {
  const int64_t tiles = (M + 15) / 16;
  int64_t g = (tiles + kWpWaves - 1) / kWpWaves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

bool winproj_supported(vswin_dtype dt, int C, int d, int N, int vt) {
  if (dt != VSWIN_BF16 || (C != 96 && C != 128) || d % 8 != 0) return false;
  return !vt || N % 4 == 0;
}

hipError_t qkv_proj(const void* x, const void* ln_g, const void* ln_b, float eps, int ln, const void* W,
                    const void* bias, void* q, void* k, void* v, int vt, float qscale, int64_t M, int C, int heads,
                    int d, const WinGeo& geo, const void* table, void* tab4, const Tab4Geo& tg, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  QkvParams pr{(const bf16_t*)x, (const bf16_t*)ln_g, (const bf16_t*)ln_b, eps, ln, (const bf16_t*)W,
               (const bf16_t*)bias, (bf16_t*)q, (bf16_t*)k, (bf16_t*)v, vt, qscale, (int)M, heads, d,
               make_fastdiv((uint32_t)d), geo};
  {
    const int64_t tiles = (M + 15) / 16;
    int64_t g = (tiles + kQkvWaves - 1) / kQkvWaves;
    const int64_t cap = device_cu_count();
    pr.tile_blocks = (int)(g > cap ? cap : (g < 1 ? 1 : g));
  }
  int extra = 0;
  if (tab4 && table) {
    pr.table = (const bf16_t*)table;
    pr.tab4 = (f32x4_t*)tab4;
    pr.tg = tg;
    const int64_t n = (int64_t)tg.TS4 * tg.heads;
    const int64_t idle = (int64_t)pr.tile_blocks * kQkvWaves - (M + 15) / 16;
    pr.tab_idle = idle > 0 ? 1 : 0;
    if (!pr.tab_idle) {
      extra = (int)((n + kQkvThreads - 1) / kQkvThreads);
      if (extra > 64) extra = 64;
    }
  }
  auto go = [&](auto kern, size_t lds) -> hipError_t {
    hipError_t e = ensure_dynamic_lds((const void*)kern, lds);
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)(pr.tile_blocks + extra)), dim3(kQkvThreads), lds, st>>>(pr);
    return hipGetLastError();
  };
  if (C == 96) return go(qkv_wave_kernel<96>, QkvLds<96>::bytes);
  if (C == 128) return go(qkv_wave_kernel<128>, QkvLds<128>::bytes);
  return hipErrorInvalidValue;
}

hipError_t out_proj(const void* o, const void* W, const void* bias, const void* res, void* out, int64_t M, int C,
                    const WinGeo& geo, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  ProjParams pr{(const bf16_t*)o, (const bf16_t*)W, (const bf16_t*)bias, (const bf16_t*)res, out, (int)M, geo};
  auto go = [&](auto kern, size_t lds) -> hipError_t {
    hipError_t e = ensure_dynamic_lds((const void*)kern, lds);
    if (e != hipSuccess) return e;
    kern<<<dim3(wave_grid(M, 2)), dim3(kWpThreads), lds, st>>>(pr);
    return hipGetLastError();
  };
  if (C == 96)
    return res ? go(out_proj_kernel<96, true>, ProjLds<96>::bytes) : go(out_proj_kernel<96, false>, ProjLds<96>::bytes);
  if (C == 128)
    return res ? go(out_proj_kernel<128, true>, ProjLds<128>::bytes)
               : go(out_proj_kernel<128, false>, ProjLds<128>::bytes);
  return hipErrorInvalidValue;
}

}  // namespace vswin
