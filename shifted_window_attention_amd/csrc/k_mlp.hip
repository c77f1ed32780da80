// Second half of the Video Swin block (eq. 1): y = z^ + MLP(LN2(z^)),
// MLP = Linear(C, 4C) -> GELU -> Linear(4C, C), fused in one kernel so the
// 4C-wide hidden activations never leave the chip.
//
// One workgroup handles 64 tokens: LN2 of its z^ rows (fp32) into a bf16 LDS
// tile, then for each chunk of 64 hidden units: H = GELU(A W1_c^T + b1_c)
// (MFMA, kept in LDS as bf16) and acc += H W2_c^T (MFMA, fp32 registers);
// finally y = z^ + acc + b2 rounded to bf16.  The next chunk's weights are
// fetched into registers while the current chunk computes.
//
// GELU comes from a piecewise linear table of its values (gelu_table.h).
#include "gelu_table.h"
#include "vswin_kernels.h"

namespace vswin {


// With PROJ the output projection runs in front: z^ = x + o Wp^T + bp for the
// workgroup's 64 tokens (o gathered from window-row order, Wp fragments read
// from L2) stays in registers in the layout of the fc2 accumulators, and LN2's
// row statistics combine the two feature halves of a token through LDS.
struct MlpProj {
  const bf16_t* o;    // attention output, window rows (Lp, C)
  const bf16_t* x;    // block input token rows (L, C): the residual
  const bf16_t* wp;   // (C, C)
  const bf16_t* bp;   // (C) or NULL
  WinGeo geo;
};

template <int C, bool PROJ>
__global__ void __launch_bounds__(256, 2) mlp_fused_kernel(const float* __restrict__ zh, const bf16_t* __restrict__ g2,
                                                        const bf16_t* __restrict__ b2ln, const bf16_t* __restrict__ W1,
                                                        const bf16_t* __restrict__ b1, const bf16_t* __restrict__ W2,
                                                        const bf16_t* __restrict__ bo, bf16_t* __restrict__ y,
                                                        int64_t L, float eps, const MlpProj pj) {
  warm_args(zh, g2, b2ln, W1, b1, W2, bo, y, L, eps, pj);
  constexpr int BM = 64, HC = 64, HID = 4 * C, NCH = HID / HC;
  constexpr int LDA = C + 8, LDH = HC + 8;
  constexpr int NT2 = C / 32;            // GEMM2 feature tiles of 16 per wave (C/2 features)
  constexpr int W1CH = HC * C / 8;       // 16-byte chunks of one W1 chunk
  constexpr int W2CH = C * HC / 8;
  constexpr int RW1 = (W1CH + 255) / 256, RW2 = (W2CH + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDA];
  __shared__ __attribute__((aligned(16))) bf16_t Hs[BM * LDH];
  __shared__ __attribute__((aligned(16))) bf16_t W1s[HC * LDA];
  __shared__ __attribute__((aligned(16))) bf16_t W2s[C * LDH];
  __shared__ float2 gtab[kGeluEntries];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 15, g4 = lane >> 4, fk = g4 * 8;
  const int64_t m0 = (int64_t)blockIdx.x * BM;

  u32x4_t r1[RW1], r2[RW2];
  auto fetch = [&](int hc) {
#pragma unroll
    for (int i = 0; i < RW1; ++i) {
      const int c = tid + 256 * i;
      if (c < W1CH) {
        const int r = c / (C / 8), k = (c % (C / 8)) * 8;
        r1[i] = *reinterpret_cast<const u32x4_t*>(W1 + (int64_t)(hc * HC + r) * C + k);
      }
    }
#pragma unroll
    for (int i = 0; i < RW2; ++i) {
      const int c = tid + 256 * i;
      if (c < W2CH) {
        const int r = c / (HC / 8), k = (c % (HC / 8)) * 8;
        r2[i] = *reinterpret_cast<const u32x4_t*>(W2 + (int64_t)r * HID + hc * HC + k);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < RW1; ++i) {
      const int c = tid + 256 * i;
      if (c < W1CH) {
        const int r = c / (C / 8), k = (c % (C / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(&W1s[r * LDA + k]) = r1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < RW2; ++i) {
      const int c = tid + 256 * i;
      if (c < W2CH) {
        const int r = c / (HC / 8), k = (c % (HC / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(&W2s[r * LDH + k]) = r2[i];
      }
    }
  };

  fetch(0);
  // z^ of the lane's tokens wm*32 + 16i + fr, features wn*(C/2) + 16j + 4*g4 .. +3 (PROJ)
  float zr[PROJ ? 2 : 1][PROJ ? NT2 : 1][4];
  if constexpr (PROJ) {
    __shared__ float red[2][2][BM];   // [pass][feature half][token]
    f32x4_t pacc[2][NT2];
#pragma unroll
    for (int j = 0; j < NT2; ++j) {
      float bb[4] = {0.f, 0.f, 0.f, 0.f};
      if (pj.bp) load4(pj.bp, wn * (C / 2) + j * 16 + 4 * g4, bb);
      pacc[0][j] = pacc[1][j] = f32x4_t{bb[0], bb[1], bb[2], bb[3]};
    }
    int64_t orow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t tok = m0 + wm * 32 + i * 16 + fr;
      orow[i] = tok < L ? token_row(pj.geo, (int)tok) : 0;
    }
#pragma unroll
    for (int kk = 0; kk < C / 32; ++kk) {
      bf16x8_t of[2], wf[NT2];
#pragma unroll
      for (int i = 0; i < 2; ++i) of[i] = *reinterpret_cast<const bf16x8_t*>(pj.o + orow[i] * C + 32 * kk + 8 * g4);
#pragma unroll
      for (int j = 0; j < NT2; ++j)
        wf[j] = *reinterpret_cast<const bf16x8_t*>(pj.wp + (int64_t)(wn * (C / 2) + j * 16 + fr) * C + 32 * kk + 8 * g4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT2; ++j)
          pacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], of[i], pacc[i][j], 0, 0, 0);
    }
    // + residual; partial sums over the wave's feature half
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t tok = m0 + wm * 32 + i * 16 + fr;
#pragma unroll
      for (int j = 0; j < NT2; ++j) {
        float xr[4] = {0.f, 0.f, 0.f, 0.f};
        if (tok < L) load4(pj.x, tok * C + wn * (C / 2) + j * 16 + 4 * g4, xr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          zr[i][j][e] = tok < L ? xr[e] + pacc[i][j][e] : 0.f;
          part[i] += zr[i][j][e];
        }
      }
      part[i] += __shfl_xor(part[i], 16);
      part[i] += __shfl_xor(part[i], 32);
      if (g4 == 0) red[0][wn][wm * 32 + i * 16 + fr] = part[i];
    }
    __syncthreads();
    float mean[2], q[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = wm * 32 + i * 16 + fr;
      mean[i] = (red[0][0][t] + red[0][1][t]) * (1.0f / C);
#pragma unroll
      for (int j = 0; j < NT2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dd = zr[i][j][e] - mean[i];
          q[i] += dd * dd;
        }
      q[i] += __shfl_xor(q[i], 16);
      q[i] += __shfl_xor(q[i], 32);
      if (g4 == 0) red[1][wn][t] = q[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = wm * 32 + i * 16 + fr;
      const float rstd = 1.0f / sqrtf((red[1][0][t] + red[1][1][t]) * (1.0f / C) + eps);
      const bool live = m0 + t < L;
#pragma unroll
      for (int j = 0; j < NT2; ++j) {
        const int n = wn * (C / 2) + j * 16 + 4 * g4;
        float gg[4], bb[4], o[4];
        load4(g2, n, gg);
        load4(b2ln, n, bb);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = live ? (zr[i][j][e] - mean[i]) * rstd * gg[e] + bb[e] : 0.f;
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[0], o[1]);
        pk[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2_t*>(&As[t * LDA + n]) = pk;
      }
    }
  } else
  // ---- LN2: 4 lanes per token row, C/4 values each
  {
    constexpr int PER = C / 4;
    const int row = tid >> 2, part = tid & 3;
    const int64_t m = m0 + row;
    float v[PER];
    if (m < L) {
      const float* src = zh + m * C + part * PER;
#pragma unroll
      for (int i = 0; i < PER; i += 4) {
        const float4 t = *reinterpret_cast<const float4*>(src + i);
        v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) v[i] = 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s += v[i];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const float mean = s * (1.0f / C);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) { const float dd = v[i] - mean; q += dd * dd; }
    q += __shfl_xor(q, 1);
    q += __shfl_xor(q, 2);
    const float rstd = 1.0f / sqrtf(q * (1.0f / C) + eps);
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      float gg[4], bb[4], o[4];
      load4(g2, part * PER + i, gg);
      load4(b2ln, part * PER + i, bb);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = (v[i + k] - mean) * rstd * gg[k] + bb[k];
      u32x2_t pk;
      pk[0] = pack_bf16x2(o[0], o[1]);
      pk[1] = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<u32x2_t*>(&As[row * LDA + part * PER + i]) = pk;
    }
  }
  stash();
  gelu_table_build(gtab, tid, 256);
  __syncthreads();

  f32x4_t acc2[2][NT2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NT2; ++j) acc2[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int hc = 0; hc < NCH; ++hc) {
    if (hc + 1 < NCH) fetch(hc + 1);
    // GEMM1: wave tile 32 tokens x 32 hidden; D = W1_c rows x A rows^T
    f32x4_t acc1[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc1[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < C; k += 32) {
      bf16x8_t af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 32 + i * 16 + fr) * LDA + k + fk]);
        wf[i] = *reinterpret_cast<const bf16x8_t*>(&W1s[(wn * 32 + i * 16 + fr) * LDA + k + fk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc1[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc1[i][j], 0, 0, 0);
    }
    // bias + GELU -> Hs[token][hidden]; lane: token fr, hidden 4*g4 .. +3
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int hcol = wn * 32 + j * 16 + 4 * g4;
        float bb[4] = {0.f, 0.f, 0.f, 0.f}, o[4];
        if (b1) load4(b1, hc * HC + hcol, bb);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = gelu_tab(gtab, acc1[i][j][k] + bb[k]);
        u32x2_t pk;
        pk[0] = pack_bf16x2(o[0], o[1]);
        pk[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2_t*>(&Hs[(wm * 32 + i * 16 + fr) * LDH + hcol]) = pk;
      }
    __syncthreads();
    // GEMM2: wave tile 32 tokens x C/2 features; D = W2_c rows x H rows^T
#pragma unroll
    for (int k = 0; k < HC; k += 32) {
      bf16x8_t hf[2], wf[NT2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        hf[i] = *reinterpret_cast<const bf16x8_t*>(&Hs[(wm * 32 + i * 16 + fr) * LDH + k + fk]);
#pragma unroll
      for (int j = 0; j < NT2; ++j)
        wf[j] = *reinterpret_cast<const bf16x8_t*>(&W2s[(wn * (C / 2) + j * 16 + fr) * LDH + k + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT2; ++j)
          acc2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], hf[i], acc2[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (hc + 1 < NCH) {
      stash();
      __syncthreads();
    }
  }
  // ---- y = z^ + acc + b2; lane: token fr, features 4*g4 .. +3 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 32 + i * 16 + fr;
    if (m >= L) continue;
#pragma unroll
    for (int j = 0; j < NT2; ++j) {
      const int n = wn * (C / 2) + j * 16 + 4 * g4;
      float r[4], bb[4], o[4];
      if constexpr (PROJ) {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = zr[i][j][e];
      } else {
        load4(zh, m * C + n, r);
      }
      if (bo) load4(bo, n, bb);
      else bb[0] = bb[1] = bb[2] = bb[3] = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = r[k] + acc2[i][j][k] + bb[k];
      store4(y, m * C + n, o);
    }
  }
}

// ---------------------------------------------------------------------------
// C = 96: the whole MLP weight set (W1 384x96 and W2 96x384, 147 KB) stays in
// LDS for the kernel's lifetime; one workgroup per CU, and each wave owns
// 16-token tiles from start to end with no barrier after the weight load.
//   * LN2 in registers: lane (token fr, group g) holds z^ columns
//     32j + 8g .. +7 (j = 0..2), which are at once its k-chunks of the fc1
//     operand and its output columns of the residual.
//   * fc1 runs on 32 hidden units at a time as a pair of 16-row MFMA tiles
//     whose W1 rows are read in pair order (hidden 8g + 4p + i at tile row
//     4g + i), so a lane ends with hidden units 8g .. 8g + 7 of its token:
//     after bias and GELU that is exactly the lane's k-chunk of the fc2
//     operand, and the hidden activations never leave registers.
//   * fc2 accumulates 6 output tiles (W2 rows in pair order too), so the
//     lane's 8 consecutive output columns go out as one 16-byte store.
// LDS: W1 rows of 192 B with chunk q of row r at q ^ ((r >> 2) & 3); W2 rows
// of 768 B with chunk q at q ^ (r & 15): conflict-free 16-byte reads.
// ---------------------------------------------------------------------------
namespace {

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kMlpWaves = 8;                 // at most, per workgroup (the launch picks 4..8)
constexpr int kMlpThreads = 64 * kMlpWaves;
constexpr int kMlpC = 96, kMlpHid = 4 * kMlpC;
constexpr size_t kMlpW1 = (size_t)kMlpHid * kMlpC * 2;
constexpr size_t kMlpVec = kMlpHid * 4 + 3 * kMlpC * 2;     // b1 (fp32), LN2 gamma / beta, fc2 bias
constexpr size_t kMlpLds = 2 * kMlpW1 + kMlpVec + kGeluEntriesU * 8;

struct ZTile {
  float z[3][8];     // columns 32j + 8g .. + 7 of token fr
};

__device__ __forceinline__ void ztile_load(ZTile& zt, const float* __restrict__ zh, int64_t L, int64_t t) {
  const int lane = threadIdx.x & 63, fr = lane & 15, g = lane >> 4;
  const int64_t tok = t * 16 + fr;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    if (tok < L) {
      const float4 a = *reinterpret_cast<const float4*>(zh + tok * kMlpC + 32 * j + 8 * g);
      const float4 b = *reinterpret_cast<const float4*>(zh + tok * kMlpC + 32 * j + 8 * g + 4);
      zt.z[j][0] = a.x; zt.z[j][1] = a.y; zt.z[j][2] = a.z; zt.z[j][3] = a.w;
      zt.z[j][4] = b.x; zt.z[j][5] = b.y; zt.z[j][6] = b.z; zt.z[j][7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) zt.z[j][e] = 0.f;
    }
  }
}

// With the output projection in front (PROJ): a token tile's inputs are its
// attention output rows o (gathered from window-row space) and its residual
// rows x, both bf16.
struct ProjTileIn {
  u32x4_t o[3], x[3];   // k-chunk g of o's 32-column block kk; x columns 32j + 8g .. + 7
};

}  // namespace

struct MlpArgs {
  const float* zh;       // !PROJ: z^ token rows (L, C), fp32
  const bf16_t* o;       // PROJ: attention output, window rows (Lp, C)
  const bf16_t* x;       // PROJ: block input token rows (L, C): the residual
  const bf16_t* wp;      // PROJ: (C, C) projection weight, bias bp (C) or NULL
  const bf16_t* bp;
  WinGeo geo;            // PROJ: token -> window row
  const bf16_t *g2, *b2ln, *W1, *b1, *W2, *bo;
  bf16_t* y;
  int64_t L;
  float eps;
};

namespace {

__device__ __forceinline__ void proj_tile_load(ProjTileIn& pt, const MlpArgs& a, int64_t t) {
  const int lane = threadIdx.x & 63, fr = lane & 15, g = lane >> 4;
  const int64_t tok = t * 16 + fr;
  const bool ok = tok < a.L;
  const int64_t m = ok ? token_row(a.geo, (int)tok) : 0;
  const int64_t tx = ok ? tok : 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    pt.o[j] = *reinterpret_cast<const u32x4_t*>(a.o + m * kMlpC + 32 * j + 8 * g);
    pt.x[j] = *reinterpret_cast<const u32x4_t*>(a.x + tx * kMlpC + 32 * j + 8 * g);
  }
}

__device__ __forceinline__ int pair_row_inv(int r) {
  return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

}  // namespace

template <bool PROJ>
__global__ void __launch_bounds__(kMlpThreads) mlp_pair_kernel(const MlpArgs a) {
  warm_args_grid(a);
  constexpr int C = kMlpC, HID = kMlpHid;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* W1s = lds;                 // HID rows x 192 B
  unsigned char* W2s = lds + kMlpW1;        // C rows x 768 B
  float* b1s = reinterpret_cast<float*>(lds + 2 * kMlpW1);   // 64 x fc1 bias + kGeluU0, fp32
  bf16_t* vecs = reinterpret_cast<bf16_t*>(b1s + HID);       // LN2 gamma, beta, fc2 bias (C each)
  float2* phi = reinterpret_cast<float2*>(lds + 2 * kMlpW1 + kMlpVec);   // GELU bins in u (gelu_table_build_u)
  const bf16_t* __restrict__ W1 = a.W1;
  const bf16_t* __restrict__ W2 = a.W2;
  const bf16_t* __restrict__ b1 = a.b1;
  const int64_t L = a.L;
  const float eps = a.eps;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwv = (int)(blockDim.x >> 6), nthr = (int)blockDim.x;
  const int fr = lane & 15, g = lane >> 4;
  // a wave owns a pair of 16-token tiles (2 t2, 2 t2 + 1): the weight
  // fragments of every chunk serve both, and the two tiles' chains are
  // independent work for the same wave
  const int64_t npairs = ((L + 15) / 16 + 1) / 2;
  const int64_t nw = (int64_t)gridDim.x * nwv;
  int64_t t2 = (int64_t)blockIdx.x * nwv + wave;

  ZTile z[2];
  ProjTileIn pin[2];
  auto load_inputs = [&](int64_t tp) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (PROJ) proj_tile_load(pin[u], a, 2 * tp + u);
      else ztile_load(z[u], a.zh, L, 2 * tp + u);
    }
  };
  // the projection weight's 18 MFMA A fragments (output tile nt covers
  // pair-order rows 16 nt .. + 15), read from L2 with the first pair's inputs
  // and held until that pair's projection is done
  bf16x8_t wpf[PROJ ? 6 : 1][3];
  u32x4_t bpr[3];   // the projection bias, columns 32j + 8g .. + 7 (bf16)
  auto load_wp = [&]() {
    if constexpr (PROJ) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        bpr[j] = a.bp ? *reinterpret_cast<const u32x4_t*>(a.bp + 32 * j + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int nt = 0; nt < 6; ++nt)
#pragma unroll
        for (int kk = 0; kk < 3; ++kk)
          wpf[nt][kk] =
              *reinterpret_cast<const bf16x8_t*>(a.wp + pair_row_inv(16 * nt + fr) * C + 32 * kk + 8 * g);
    }
  };
  if (t2 < npairs) {
    load_inputs(t2);
    load_wp();
  }
  // the small vectors and the GELU table into LDS first: their loads (and the
  // first pair's inputs, issued before them) have landed once these stores
  // are done, so nothing that the first pair's projection and LN2 statistics
  // read below is waited for behind the weight transfer
  for (int c = tid; c < HID; c += nthr) b1s[c] = 64.0f * (b1 ? bf2f(b1[c]) : 0.f) + kGeluU0;
  gelu_table_build_u(phi, tid, nthr);
  for (int c = tid; c < 3 * (C / 8); c += nthr) {
    const int which = c / (C / 8), q = c - which * (C / 8);
    const bf16_t* src = which == 0 ? a.g2 : (which == 1 ? a.b2ln : a.bo);
    *reinterpret_cast<u32x4_t*>(vecs + which * C + q * 8) =
        src ? *reinterpret_cast<const u32x4_t*>(src + q * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // every earlier load has landed (the builtin tells the compiler so; an asm
  // wait would not, and it would wait for the weight transfer before the
  // projection below)
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0); expcnt, lgkmcnt left alone
  // W1 and W2 go straight from global memory into their swizzled LDS layouts
  // (global_load_lds: a wave instruction fills 1 KB of consecutive LDS chunks
  // from per-lane addresses), in flight while the first pair's projection and
  // LN2 statistics run (registers and lane swaps only: no LDS access, which
  // would wait for the transfer); LDS chunk (r, qp) holds global row
  // pair_row_inv(r), chunk qp ^ swizzle(r)
  {
    constexpr int NB = HID * (C / 8) / 64;   // 1 KB blocks per matrix
    static_assert(NB * 64 == HID * (C / 8), "weight staging shape");
    for (int b = wave; b < NB; b += nwv) {
      const int c = 64 * b + lane;
      const int r1 = c / (C / 8), qp1 = c - r1 * (C / 8);
      __builtin_amdgcn_global_load_lds(W1 + pair_row_inv(r1) * C + ((qp1 ^ ((r1 >> 2) & 3)) << 3),
                                       (lds_ptr_t)(W1s + 1024 * b), 16, 0, 0);
      const int r2 = c / (HID / 8), qp2 = c - r2 * (HID / 8);
      __builtin_amdgcn_global_load_lds(W2 + pair_row_inv(r2) * HID + ((qp2 ^ (r2 & 15)) << 3),
                                       (lds_ptr_t)(W2s + 1024 * b), 16, 0, 0);
    }
  }

  const int swz1 = (fr >> 2) & 3;   // W1 rows 32c + 16p + fr: ((row >> 2) & 3) = (fr >> 2) & 3
  // front of a pair, in two parts.  front1: (PROJ) z^ = x + o Wp^T + bp into
  // z, and LN2's mean and 64 / std per token (registers and lane swaps only);
  // front2: 64 LN2(z^) into af with gamma and beta from LDS.
  bf16x8_t af[2][3];
  float mean[2], rstd[2];
  auto front1 = [&]() {
    if constexpr (PROJ) {
      // 6 output tiles (pair order) of 16 tokens for each tile of the pair, the
      // accumulators starting at the bias
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4_t acc[6];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          float bb[8];
          unpack8(bpr[j], bb);
          acc[2 * j] = f32x4_t{bb[0], bb[1], bb[2], bb[3]};
          acc[2 * j + 1] = f32x4_t{bb[4], bb[5], bb[6], bb[7]};
        }
#pragma unroll
        for (int kk = 0; kk < 3; ++kk)
#pragma unroll
          for (int nt = 0; nt < 6; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wpf[nt][kk], __builtin_bit_cast(bf16x8_t, pin[u].o[kk]),
                                                              acc[nt], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          float xv[8];
          unpack8(pin[u].x[j], xv);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            z[u].z[j][i] = xv[i] + acc[2 * j][i];
            z[u].z[j][4 + i] = xv[4 + i] + acc[2 * j + 1][i];
          }
        }
      }
    }
    // LN2 statistics of the lane's token in each tile (4 lanes share a token)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm += z[u].z[j][e];
      sm = row4_sum(sm);
      mean[u] = sm * (1.0f / C);
      float q2 = 0.f;
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dd = z[u].z[j][e] - mean[u];
          q2 += dd * dd;
        }
      q2 = row4_sum(q2);
      // 64 LN2(z^): the power-of-two scale leaves every rounding unchanged
      rstd[u] = 64.0f / sqrtf(q2 * (1.0f / C) + eps);
    }
  };
  auto front2 = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        float gg[8], bb[8], v[8];
        unpack8(*reinterpret_cast<const u32x4_t*>(vecs + 32 * j + 8 * g), gg);
        unpack8(*reinterpret_cast<const u32x4_t*>(vecs + C + 32 * j + 8 * g), bb);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (z[u].z[j][e] - mean[u]) * rstd[u] * gg[e] + 64.0f * bb[e];
        af[u][j] = __builtin_bit_cast(bf16x8_t, pack8(v));
      }
  };
  if (t2 < npairs) front1();
  // every wave's weight blocks are in LDS (every wave reaches this barrier)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t2 < npairs) front2();

  // chunk ch's LDS reads: W1 rows 32 ch .. + 31 (pair order) and the fc1
  // accumulators' start (64 b1 + U0); W2 columns 32 ch .. + 31
  auto load_w1 = [&](int ch, bf16x8_t (&w1f)[2][3], f32x4_t& bA, f32x4_t& bB) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const unsigned char* row = W1s + (32 * ch + 16 * p + fr) * (C * 2);
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) w1f[p][kk] = *reinterpret_cast<const bf16x8_t*>(row + (((4 * kk + g) ^ swz1) << 4));
    }
    bA = *reinterpret_cast<const f32x4_t*>(b1s + 32 * ch + 8 * g);
    bB = *reinterpret_cast<const f32x4_t*>(b1s + 32 * ch + 8 * g + 4);
  };
  auto load_w2 = [&](int ch, bf16x8_t (&w2f)[6]) {
#pragma unroll
    for (int nt = 0; nt < 6; ++nt) {
      const int r = 16 * nt + fr;
      w2f[nt] = *reinterpret_cast<const bf16x8_t*>(W2s + r * (HID * 2) + (((4 * ch + g) ^ (r & 15)) << 4));
    }
  };
  // fc1 of one chunk for both tiles: u = 64 x + U0 of hidden units 8g .. + 7
  auto fc1 = [&](const bf16x8_t (&w1f)[2][3], const f32x4_t& bA, const f32x4_t& bB, f32x4_t (&a1)[2][2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      a1[u][0] = bA;
      a1[u][1] = bB;
    }
#pragma unroll
    for (int kk = 0; kk < 3; ++kk)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          a1[u][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1f[p][kk], af[u][kk], a1[u][p], 0, 0, 0);
  };
  // GELU of one chunk's fc1 output (the fc2 operand of each tile)
  auto gelu = [&](const f32x4_t (&a1)[2][2], bf16x8_t (&hf)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = gelu_tab_u(phi, i < 4 ? a1[u][0][i] : a1[u][1][i - 4]);
      hf[u] = __builtin_bit_cast(bf16x8_t, pack8(h));
    }
  };
  auto fc2 = [&](const bf16x8_t (&hf)[2], const bf16x8_t (&w2f)[6], f32x4_t (&acc2)[2][6]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int nt = 0; nt < 6; ++nt)
        acc2[u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[nt], hf[u], acc2[u][nt], 0, 0, 0);
  };
  auto gelu_fc2 = [&](const f32x4_t (&a1)[2][2], const bf16x8_t (&w2f)[6], f32x4_t (&acc2)[2][6]) {
    bf16x8_t hf[2];
    gelu(a1, hf);
    fc2(hf, w2f, acc2);
  };
  // one pipelined step: the fc1 products of chunk ch + 1 (into nxt) are
  // issued beside the GELU of chunk ch (from cur), whose table reads and VALU
  // work do not depend on them; then chunk ch's W2 fragments and fc2
  auto step = [&](int ch, const f32x4_t (&cur)[2][2], f32x4_t (&nxt)[2][2], f32x4_t (&acc2)[2][6]) {
    bf16x8_t hf[2];
    {
      bf16x8_t w1f[2][3];
      f32x4_t bA, bB;
      load_w1(ch + 1, w1f, bA, bB);
      __builtin_amdgcn_sched_barrier(0);
      fc1(w1f, bA, bB, nxt);
      gelu(cur, hf);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t w2f[6];
    load_w2(ch, w2f);
    fc2(hf, w2f, acc2);
  };

  for (; t2 < npairs; t2 += nw) {
    // ---- fc1 -> GELU -> fc2 over 12 chunks of 32 hidden units, both tiles,
    // software-pipelined by one chunk.  The fc2 accumulators start at
    // z^ + b2, so the block output is their final value (z^ is not held).
    f32x4_t acc2[2][6];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        float ob[8];
        unpack8(*reinterpret_cast<const u32x4_t*>(vecs + 2 * C + 32 * j + 8 * g), ob);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc2[u][2 * j][i] = z[u].z[j][i] + ob[i];
          acc2[u][2 * j + 1][i] = z[u].z[j][4 + i] + ob[4 + i];
        }
      }
    static_assert(HID / 32 == 12, "chunk count");
    f32x4_t a1A[2][2], a1B[2][2];
    {
      bf16x8_t w1f[2][3];
      f32x4_t bA, bB;
      load_w1(0, w1f, bA, bB);
      fc1(w1f, bA, bB, a1A);
    }
    // two steps per iteration, so that the two fc1 outputs swap roles
    // without register copies
#pragma unroll 1
    for (int ch = 0; ch < 10; ch += 2) {
      step(ch, a1A, a1B, acc2);
      step(ch + 1, a1B, a1A, acc2);
    }
    step(10, a1A, a1B, acc2);
    {
      bf16x8_t w2f[6];
      load_w2(11, w2f);
      gelu_fc2(a1B, w2f, acc2);
    }
    // ---- y = z^ + b2 + fc2: lane holds columns 32j + 8g .. + 7 of token fr of each tile
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t tok = (2 * t2 + u) * 16 + fr;
      if (tok < L) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          float o[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[i] = acc2[u][2 * j][i];
            o[4 + i] = acc2[u][2 * j + 1][i];
          }
          *reinterpret_cast<u32x4_t*>(a.y + tok * C + 32 * j + 8 * g) = pack8(o);
        }
      }
    }
    if (t2 + nw < npairs) {
      load_inputs(t2 + nw);
      load_wp();
      front1();
      front2();
    }
  }
}

namespace {
template <bool PROJ>
hipError_t launch_mlp_wave(const MlpArgs& a, hipStream_t st) {
  const int ncu = device_cu_count();
  const int64_t pairs = ((a.L + 15) / 16 + 1) / 2;
  // one workgroup per CU (the weights fill its LDS) with just enough waves for
  // one pair each (Swin-T stage 1: 1568 pairs on 224 CUs x 7 waves rather than
  // 196 x 8), at least 4 and at most 8; larger inputs loop
  int64_t wpg = (pairs + ncu - 1) / ncu;
  wpg = wpg < 4 ? 4 : (wpg > kMlpWaves ? kMlpWaves : wpg);
  int64_t grid = (pairs + wpg - 1) / wpg;
  if (grid > ncu) grid = ncu;
  hipError_t e = ensure_dynamic_lds((const void*)mlp_pair_kernel<PROJ>, kMlpLds);
  if (e != hipSuccess) return e;
  mlp_pair_kernel<PROJ><<<dim3((unsigned)grid), dim3((unsigned)(64 * wpg)), kMlpLds, st>>>(a);
  return hipGetLastError();
}
}  // namespace

bool proj_mlp_supported(vswin_dtype dt, int C, int hid) {
  return dt == VSWIN_BF16 && (C == 96 || C == 128) && hid == 4 * C;
}

hipError_t proj_mlp(const void* o, const void* x, const void* wp, const void* bp, const void* g2, const void* b2ln,
                    const void* W1, const void* b1, const void* W2, const void* bo, void* y, int64_t L, int C,
                    float eps, const WinGeo& geo, hipStream_t st) {
  if (L <= 0) return hipSuccess;
  if (C == 128) {
    if (L > 0x7fffffff) return hipErrorInvalidValue;
    const MlpProj pj{(const bf16_t*)o, (const bf16_t*)x, (const bf16_t*)wp, (const bf16_t*)bp, geo};
    hipLaunchKernelGGL((mlp_fused_kernel<128, true>), dim3((unsigned)((L + 63) / 64)), dim3(256), 0, st, nullptr,
                       (const bf16_t*)g2, (const bf16_t*)b2ln, (const bf16_t*)W1, (const bf16_t*)b1,
                       (const bf16_t*)W2, (const bf16_t*)bo, (bf16_t*)y, L, eps, pj);
    return hipGetLastError();
  }
  if (C != 96) return hipErrorInvalidValue;
  MlpArgs a{};
  a.o = (const bf16_t*)o; a.x = (const bf16_t*)x; a.wp = (const bf16_t*)wp; a.bp = (const bf16_t*)bp;
  a.geo = geo;
  a.g2 = (const bf16_t*)g2; a.b2ln = (const bf16_t*)b2ln;
  a.W1 = (const bf16_t*)W1; a.b1 = (const bf16_t*)b1; a.W2 = (const bf16_t*)W2; a.bo = (const bf16_t*)bo;
  a.y = (bf16_t*)y; a.L = L; a.eps = eps;
  return launch_mlp_wave<true>(a, st);
}

bool mlp_fused_supported(vswin_dtype dt, int C, int hid) {
  return dt == VSWIN_BF16 && hid == 4 * C && (C == 96 || C == 128);
}

hipError_t mlp_fused(const float* zh, const void* g2, const void* b2ln, const void* W1, const void* b1,
                     const void* W2, const void* bo, void* y, int64_t L, int C, float eps, hipStream_t st) {
  if (L <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((L + 63) / 64);
  if (C == 96) {
    MlpArgs a{};
    a.zh = zh;
    a.g2 = (const bf16_t*)g2; a.b2ln = (const bf16_t*)b2ln;
    a.W1 = (const bf16_t*)W1; a.b1 = (const bf16_t*)b1; a.W2 = (const bf16_t*)W2; a.bo = (const bf16_t*)bo;
    a.y = (bf16_t*)y; a.L = L; a.eps = eps;
    return launch_mlp_wave<false>(a, st);
  } else if (C == 128)
    hipLaunchKernelGGL((mlp_fused_kernel<128, false>), dim3(blocks), dim3(256), 0, st, zh, (const bf16_t*)g2,
                       (const bf16_t*)b2ln, (const bf16_t*)W1, (const bf16_t*)b1, (const bf16_t*)W2,
                       (const bf16_t*)bo, (bf16_t*)y, L, eps, MlpProj{});
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace vswin
