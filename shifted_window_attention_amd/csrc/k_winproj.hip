// Window projections of the attention branch for C in {96, 128} (bf16):
//
//   qkv_proj:  window rows  <- LN1(x) gathered through pad + roll + partition
//              (eq. 1, first line; the mmaction2 walk-through's op order),
//              q, k, v       = rows * Wqkv^T + bqkv, split by head (eq. 2 input)
//   out_proj:  z[token]      = x[token] + o[row] * Wproj^T + bproj, scattered
//              back through reverse partition + roll + crop (eq. 1 residual)
//
// One workgroup owns a tile of window rows and every output feature, so each
// row is fetched and normalised once; the whole weight matrix sits in LDS.
// Both use v_mfma_f32_16x16x32_bf16 with K = C taken in three or four steps.
//
// Store layout.  An MFMA output tile gives a lane four consecutive rows of
// one column.  Reading the weight rows of a 32-feature group in the order
// 8g + 4p + i  (p = which 16-row tile, g = lane group, i = element) gives
// lane group g the eight consecutive features 8g .. 8g + 7 from the tile
// pair, so each lane writes one 16-byte vector and a wave writes 16 whole
// 64-byte head rows.  For V stored transposed (feature-major, the layout the
// attention kernel reads) the same is done on the token side: the tokens of
// a 32-row group are read as 8g + 4p + i, and a lane holds eight consecutive
// tokens of one feature.
#include "vswin_kernels.h"

namespace vswin {

namespace {

// LDS row of weight feature f when the features of each 32-group are read
// in pair order (see the header comment): f = 8g + 4p + i -> 16p + 4g + i.
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

// Copy W (F x C, row-major) into LDS rows of pitch LD, row f going to LDS
// row perm(f).  Each pass moves NTHR / (C/8) whole rows in 16-byte chunks;
// a thread keeps the same chunk column in every pass.
template <int C, int F, int LD, int NTHR, class Perm>
__device__ __forceinline__ void stage_weights(const bf16_t* __restrict__ W, bf16_t* Ws, Perm perm) {
  constexpr int CPR = C / 8;           // chunks per row
  constexpr int RP = NTHR / CPR;       // rows per pass
  static_assert(NTHR % CPR == 0 && F % RP == 0, "weight staging shape");
  constexpr int PASSES = F / RP;
  const int tr = (int)threadIdx.x / CPR, tk = ((int)threadIdx.x - tr * CPR) * 8;
  constexpr int BATCH = PASSES < 8 ? PASSES : 8;
#pragma unroll
  for (int p0 = 0; p0 < PASSES; p0 += BATCH) {
    u32x4_t v[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (p0 + j < PASSES) v[j] = *reinterpret_cast<const u32x4_t*>(W + (int64_t)((p0 + j) * RP + tr) * C + tk);
#pragma unroll
    for (int j = 0; j < BATCH; ++j)
      if (p0 + j < PASSES) *reinterpret_cast<u32x4_t*>(Ws + perm((p0 + j) * RP + tr) * LD + tk) = v[j];
  }
}

constexpr int kQkvBM = 64;       // window rows per workgroup
constexpr int kQkvThreads = 384; // 6 waves: 2 row halves x {q, k, v}

template <int C>
struct QkvLds {
  static constexpr int LD = C + 8;   // bf16 pitch: 16-byte multiple, rows spread over banks
  static constexpr size_t w_off = 0;
  static constexpr size_t a_off = (size_t)3 * C * LD * 2;
  static constexpr size_t bytes = a_off + (size_t)kQkvBM * LD * 2;
};

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
};

template <int C>
__global__ void __launch_bounds__(kQkvThreads) qkv_proj_kernel(QkvParams pr) {
  using L = QkvLds<C>;
  constexpr int LD = L::LD;
  constexpr int NT = C / 16;          // 16-feature tiles per wave (one of q, k, v)
  constexpr int MT = 2;               // 16-row tiles per wave (32 rows)
  constexpr int CPT = C / 32;         // 8-element chunks per thread of an A row (4 threads per row)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  bf16_t* Ws = reinterpret_cast<bf16_t*>(lds + L::w_off);
  bf16_t* As = reinterpret_cast<bf16_t*>(lds + L::a_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.x * kQkvBM;
  const int vt = pr.vt;

  // ---- A rows: 4 threads per row, waves 0-3 (issued first: the longest latency)
  u32x4_t av[CPT];
  const int arow = tid >> 2, aq = tid & 3;
  bool live = false;
  if (wave < 4) {
    const int m = m0 + arow;
    int64_t src = -1;
    if (m < pr.M) {
      int lab;
      src = row_source(pr.geo, m, lab);
    }
    live = src >= 0;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      av[i] = live ? *reinterpret_cast<const u32x4_t*>(pr.x + src * C + (aq + 4 * i) * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // ---- weights: q and k rows (and v rows unless transposed) in pair order
  stage_weights<C, 3 * C, LD, kQkvThreads>(pr.w, Ws, [vt](int f) { return (f < 2 * C || !vt) ? pair_row(f) : f; });
  // ---- LN1 of the A rows (pads stay zero: the grid is padded after the norm)
  if (wave < 4) {
    if (pr.ln) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += bflo(av[i][e]) + bfhi(av[i][e]);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      const float mean = s * (1.0f / C);
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d0 = bflo(av[i][e]) - mean, d1 = bfhi(av[i][e]) - mean;
          sq += d0 * d0 + d1 * d1;
        }
      sq += __shfl_xor(sq, 1);
      sq += __shfl_xor(sq, 2);
      const float rstd = 1.0f / sqrtf(sq * (1.0f / C) + pr.eps);
      if (live) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          const int k0 = (aq + 4 * i) * 8;
          float xv[8], gv[8], bv[8];
          unpack8(av[i], xv);
          unpack8(*reinterpret_cast<const u32x4_t*>(pr.ln_g + k0), gv);
          unpack8(*reinterpret_cast<const u32x4_t*>(pr.ln_b + k0), bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = (xv[e] - mean) * rstd * gv[e] + bv[e];
          av[i] = pack8(xv);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) *reinterpret_cast<u32x4_t*>(As + arow * LD + (aq + 4 * i) * 8) = av[i];
  }
  __syncthreads();

  // ---- MFMA: wave (wm, wn) computes rows wm*32 .. +31 of q (wn 0), k (1), v (2)
  const int wm = wave / 3, wn = wave - 3 * (wave / 3);
  const bool swap = (wn == 2) && vt;   // V^T: tokens on the MFMA row side
  const int fr = lane & 15, g = lane >> 4, fk = g * 8;
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // A fragment rows: natural, or token pair order 8(fr/4) + 4 mt + fr%4 for V^T
  int arow_of[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    arow_of[mt] = wm * 32 + (swap ? (8 * (fr >> 2) + 4 * mt + (fr & 3)) : (mt * 16 + fr));
  // bias values of this lane's output features (no wait inside the store loop)
  u32x4_t bq[NT / 2];
  float bv[NT];
  {
    const bf16_t* bias = pr.bias ? pr.bias + wn * C : nullptr;
    if (!swap) {
#pragma unroll
      for (int j = 0; j < NT / 2; ++j)
        bq[j] = bias ? *reinterpret_cast<const u32x4_t*>(bias + 32 * j + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bv[nt] = bias ? bf2f(bias[nt * 16 + fr]) : 0.f;
    }
  }
  const bf16_t* wbase = Ws + (wn * C + fr) * LD + fk;
#pragma unroll
  for (int k = 0; k < C; k += 32) {
    bf16x8_t af[MT], wf[NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) af[mt] = *reinterpret_cast<const bf16x8_t*>(As + arow_of[mt] * LD + k + fk);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wf[nt] = *reinterpret_cast<const bf16x8_t*>(wbase + nt * 16 * LD + k);
    if (swap) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], wf[nt], acc[mt][nt], 0, 0, 0);
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt], af[mt], acc[mt][nt], 0, 0, 0);
    }
  }

  // ---- epilogue (bias values were loaded before the MFMAs)
  const int N = pr.geo.N, d = pr.d;
  if (!swap) {
    // lane: token row wm*32 + mt*16 + fr, features 32 j + 8 g .. + 7 of q/k/v,
    // stored at ((w*heads + h)*N + t)*d + e = w*N*C + (h*N*d + e) + t*d
    bf16_t* out = wn == 0 ? pr.q : (wn == 1 ? pr.k : pr.v);
    const float osc = wn == 0 ? pr.qscale : 1.0f;
    int coff[NT / 2];
#pragma unroll
    for (int j = 0; j < NT / 2; ++j) {
      const int c = 32 * j + 8 * g;
      const int h = (int)fdiv((uint32_t)c, pr.fd);
      coff[j] = h * N * d + (c - h * d);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + wm * 32 + mt * 16 + fr;
      if (m >= pr.M) continue;
      const int w = (int)fdiv((uint32_t)m, pr.geo.fN);
      bf16_t* row = out + (int64_t)w * N * C + (m - w * N) * d;
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        float v8[8], b8[8];
        unpack8(bq[j], b8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v8[i] = (acc[mt][2 * j][i] + b8[i]) * osc;
          v8[4 + i] = (acc[mt][2 * j + 1][i] + b8[4 + i]) * osc;
        }
        *reinterpret_cast<u32x4_t*>(row + coff[j]) = pack8(v8);
      }
    }
  } else {
    // lane: feature c = nt*16 + fr of v, tokens wm*32 + 8 g .. + 7, stored at
    // ((w*heads + h)*d + e)*N + t = (w*C + c)*N + t.  N and the row offsets
    // are multiples of 4, so a 4-run of tokens never leaves its window; with
    // N % 8 == 0 neither does the 8-run.
    const int mr = m0 + wm * 32 + 8 * g;
    if ((N & 7) == 0) {
      if (mr < pr.M) {
        const int w = (int)fdiv((uint32_t)mr, pr.geo.fN);
        bf16_t* base = pr.v + (int64_t)w * C * N + (mr - w * N);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v8[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v8[i] = acc[0][nt][i] + bv[nt];
            v8[4 + i] = acc[1][nt][i] + bv[nt];
          }
          *reinterpret_cast<u32x4_t*>(base + (nt * 16 + fr) * N) = pack8(v8);
        }
      }
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int m = mr + 4 * half;
        if (m >= pr.M) continue;
        const int w = (int)fdiv((uint32_t)m, pr.geo.fN);
        bf16_t* base = pr.v + (int64_t)w * C * N + (m - w * N);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x2_t p;
          p[0] = pack_bf16x2(acc[half][nt][0] + bv[nt], acc[half][nt][1] + bv[nt]);
          p[1] = pack_bf16x2(acc[half][nt][2] + bv[nt], acc[half][nt][3] + bv[nt]);
          *reinterpret_cast<u32x2_t*>(base + (nt * 16 + fr) * N) = p;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// out_proj: o rows (window slot order) * Wproj^T + b, scattered to tokens
// ---------------------------------------------------------------------------
constexpr int kProjBM = 128;

template <int C>
struct ProjLds {
  static constexpr int LD = C + 8;
  static constexpr int THREADS = 2 * (C / 32) * 64;   // 2 row halves x C/32 feature pairs
  static constexpr size_t w_off = 0;
  static constexpr size_t a_off = (size_t)C * LD * 2;
  static constexpr size_t s_off = a_off + (size_t)kProjBM * LD * 2;
  static constexpr size_t bytes = s_off + kProjBM * 4;
};

struct ProjParams {
  const bf16_t* o;      // (M, C) window rows
  const bf16_t* w;      // (C, C)
  const bf16_t* bias;   // (C) or NULL
  const bf16_t* res;    // residual tokens (bf16) or NULL
  void* out;            // res ? fp32 z : bf16 y, token rows
  int M;
  WinGeo geo;
};

template <int C, bool RES>
__global__ void __launch_bounds__(ProjLds<C>::THREADS) out_proj_kernel(ProjParams pr) {
  using L = ProjLds<C>;
  constexpr int LD = L::LD;
  constexpr int NTHR = L::THREADS;
  constexpr int MT = 4;                         // 64 rows per wave
  constexpr int CPR = C / 8;
  constexpr int ACH = kProjBM * CPR / NTHR;     // A chunks per thread (4)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  bf16_t* Ws = reinterpret_cast<bf16_t*>(lds + L::w_off);
  bf16_t* As = reinterpret_cast<bf16_t*>(lds + L::a_off);
  int* srcs = reinterpret_cast<int*>(lds + L::s_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = blockIdx.x * kProjBM;

  u32x4_t av[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * NTHR;
    const int r = c / CPR;
    av[i] = (m0 + r < pr.M) ? *reinterpret_cast<const u32x4_t*>(pr.o + (int64_t)(m0 + r) * C + (c - r * CPR) * 8)
                            : u32x4_t{0u, 0u, 0u, 0u};
  }
  if (tid < kProjBM) {
    const int m = m0 + tid;
    int lab;
    srcs[tid] = m < pr.M ? (int)row_source(pr.geo, m, lab) : -1;
  }
  stage_weights<C, C, LD, NTHR>(pr.w, Ws, [](int f) { return pair_row(f); });
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * NTHR;
    const int r = c / CPR;
    *reinterpret_cast<u32x4_t*>(As + r * LD + (c - r * CPR) * 8) = av[i];
  }
  __syncthreads();

  const int wm = wave & 1, wn = wave >> 1;      // rows wm*64.., features 32 wn .. + 31
  const int fr = lane & 15, g = lane >> 4, fk = g * 8;
  const int c = wn * 32 + 8 * g;
  const u32x4_t bq = pr.bias ? *reinterpret_cast<const u32x4_t*>(pr.bias + c) : u32x4_t{0u, 0u, 0u, 0u};
  f32x4_t acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < C; k += 32) {
    bf16x8_t af[MT], wf[2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      af[mt] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + mt * 16 + fr) * LD + k + fk);
#pragma unroll
    for (int p = 0; p < 2; ++p)
      wf[p] = *reinterpret_cast<const bf16x8_t*>(Ws + (wn * 32 + p * 16 + fr) * LD + k + fk);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        acc[mt][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[p], af[mt], acc[mt][p], 0, 0, 0);
  }

  float b8[8];
  unpack8(bq, b8);
  // residual rows first, so that no load waits behind the stores
  int src[MT];
  u32x4_t rv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    src[mt] = srcs[wm * 64 + mt * 16 + fr];
    if constexpr (RES)
      rv[mt] = src[mt] >= 0 ? *reinterpret_cast<const u32x4_t*>(pr.res + (int64_t)src[mt] * C + c)
                            : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (src[mt] < 0) continue;   // pad slot or past the end
    float v8[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v8[i] = acc[mt][0][i] + b8[i];
      v8[4 + i] = acc[mt][1][i] + b8[4 + i];
    }
    const int64_t off = (int64_t)src[mt] * C + c;
    if constexpr (RES) {
      float r8[8];
      unpack8(rv[mt], r8);
      float* z = reinterpret_cast<float*>(pr.out) + off;
      *reinterpret_cast<float4*>(z) = make_float4(v8[0] + r8[0], v8[1] + r8[1], v8[2] + r8[2], v8[3] + r8[3]);
      *reinterpret_cast<float4*>(z + 4) = make_float4(v8[4] + r8[4], v8[5] + r8[5], v8[6] + r8[6], v8[7] + r8[7]);
    } else {
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(pr.out) + off) = pack8(v8);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool winproj_supported(vswin_dtype dt, int C, int d, int N, int vt) {
  if (dt != VSWIN_BF16 || (C != 96 && C != 128) || d % 8 != 0) return false;
  return !vt || N % 4 == 0;
}

hipError_t qkv_proj(const void* x, const void* ln_g, const void* ln_b, float eps, int ln, const void* W,
                    const void* bias, void* q, void* k, void* v, int vt, float qscale, int64_t M, int C, int heads,
                    int d, const WinGeo& geo, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  QkvParams pr{(const bf16_t*)x, (const bf16_t*)ln_g, (const bf16_t*)ln_b, eps, ln, (const bf16_t*)W,
               (const bf16_t*)bias, (bf16_t*)q, (bf16_t*)k, (bf16_t*)v, vt, qscale, (int)M, heads, d, make_fastdiv((uint32_t)d), geo};
  const unsigned grid = (unsigned)((M + kQkvBM - 1) / kQkvBM);
  auto go = [&](auto kern, size_t lds) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    kern<<<dim3(grid), dim3(kQkvThreads), lds, st>>>(pr);
    return hipGetLastError();
  };
  if (C == 96) return go(qkv_proj_kernel<96>, QkvLds<96>::bytes);
  if (C == 128) return go(qkv_proj_kernel<128>, QkvLds<128>::bytes);
  return hipErrorInvalidValue;
}

hipError_t out_proj(const void* o, const void* W, const void* bias, const void* res, void* out, int64_t M, int C,
                    const WinGeo& geo, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  ProjParams pr{(const bf16_t*)o, (const bf16_t*)W, (const bf16_t*)bias, (const bf16_t*)res, out, (int)M, geo};
  const unsigned grid = (unsigned)((M + kProjBM - 1) / kProjBM);
  auto go = [&](auto kern, size_t lds, int threads) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    kern<<<dim3(grid), dim3(threads), lds, st>>>(pr);
    return hipGetLastError();
  };
  if (C == 96)
    return res ? go(out_proj_kernel<96, true>, ProjLds<96>::bytes, ProjLds<96>::THREADS)
               : go(out_proj_kernel<96, false>, ProjLds<96>::bytes, ProjLds<96>::THREADS);
  if (C == 128)
    return res ? go(out_proj_kernel<128, true>, ProjLds<128>::bytes, ProjLds<128>::THREADS)
               : go(out_proj_kernel<128, false>, ProjLds<128>::bytes, ProjLds<128>::THREADS);
  return hipErrorInvalidValue;
}

}  // namespace vswin
