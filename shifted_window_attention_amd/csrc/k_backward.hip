// Backward pass of the Video Swin block (training), bf16 activations with
// fp32 accumulation (§3.1 / eq. 1 and §3.2 / eq. 2 of "Video Swin
// Transformer", differentiated step by step):
//   * weight gradients dW = dY^T X of the linear layers: `wgrad_kernel`, MFMA
//     with the token dimension as the contraction (both operands staged
//     token-contiguous in LDS by transposing 16-byte row loads), one fp32
//     partial per group of 256-token chunks; the bias gradient (column sums of
//     dY) in the same pass; the partials of every weight gradient of a
//     backward call summed by one `wgrad_reduce_kernel` launch;
//   * LayerNorm backward `ln_bwd_kernel`: one wave per token row, the
//     statistics recomputed, dx = (dxh - mean(dxh) - xh mean(dxh xh)) / sigma
//     with dxh = dy g, plus a residual gradient; dg, db as per-wave partials;
//   * GELU x Phi(x) and its derivative Phi(x) + x phi(x) (erff);
//   * the gather of an fp32 token-row gradient into bf16 window rows (zeros
//     for pad slots) and the weight transposes the input-gradient GEMMs use.
#include "vswin_kernels.h"

#include <math.h>

#include <type_traits>

namespace vswin {

namespace {

constexpr int kWgChunk = 256;     // tokens per staged chunk
constexpr int kWgPitch = 264;     // LDS row pitch (bf16) of the token-contiguous operands
constexpr int kMaxParts = 256;    // fp32 partials of one weight gradient at most
constexpr int kWgBlocks = 256;    // workgroups a weight gradient aims for (one per CU: a chunk fills most of LDS)

__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_d(float x) {
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.39894228040143268f * __expf(-0.5f * x * x);
}

__device__ __forceinline__ void unpack8f(const u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bflo(v[i]);
    f[2 * i + 1] = bfhi(v[i]);
  }
}
__device__ __forceinline__ u32x4_t pack8u(const float* f) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

}  // namespace


// h = GELU(a) (bwd = 0) or da = dh * GELU'(a) written over dh (bwd = 1); n % 8 == 0
__global__ void __launch_bounds__(256) gelu_kernel(const bf16_t* __restrict__ a, bf16_t* __restrict__ io, int64_t n,
                                                   int bwd) {
  for (int64_t i = (blockIdx.x * 256 + (int64_t)threadIdx.x) * 8; i < n; i += (int64_t)gridDim.x * 256 * 8) {
    float x[8], y[8];
    unpack8f(*reinterpret_cast<const u32x4_t*>(a + i), x);
    if (bwd) {
      float g[8];
      unpack8f(*reinterpret_cast<const u32x4_t*>(io + i), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = g[e] * gelu_d(x[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = gelu_f(x[e]);
    }
    *reinterpret_cast<u32x4_t*>(io + i) = pack8u(y);
  }
}

// window row m of `out` (bf16) = token row src(m) of `in` (fp32), 0 for pads
__global__ void __launch_bounds__(256) gather_f32_bf16_kernel(const float* __restrict__ in, bf16_t* __restrict__ out,
                                                               int64_t slots, int C, const WinGeo geo) {
  warm_args_grid(in, out, slots, C, geo);
  const int per = C / 8;
  for (int64_t x = blockIdx.x * 256 + (int64_t)threadIdx.x; x < slots * per; x += (int64_t)gridDim.x * 256) {
    const int64_t m = x / per;
    const int c = (int)(x - m * per) * 8;
    int lab;
    const int64_t src = row_source(geo, (int)m, lab);
    float v[8];
    if (src >= 0) {
      const float4 a = *reinterpret_cast<const float4*>(in + src * C + c);
      const float4 b = *reinterpret_cast<const float4*>(in + src * C + c + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    *reinterpret_cast<u32x4_t*>(out + m * C + c) = pack8u(v);
  }
}

// LayerNorm backward, LPR lanes per row (64 / LPR rows per wave in flight),
// C <= LPR * J.  x: TX (fp32 / bf16), dy: bf16, res (nullable): TR added to
// dx, out: TO.  part: per workgroup, dg then db (2C), the row groups' sums
// combined in LDS.
template <typename TX, typename TR, typename TO, int LPR, int J>
__global__ void __launch_bounds__(256) ln_bwd_kernel(const TX* __restrict__ x, const bf16_t* __restrict__ g,
                                                     const bf16_t* __restrict__ dy, const TR* __restrict__ res,
                                                     TO* __restrict__ out, float* __restrict__ part, int64_t rows,
                                                     int C, float eps) {
  warm_args_grid(x, g, dy, res, out, part, rows, C, eps);
  const int l16 = threadIdx.x % LPR;
  const int64_t grp = blockIdx.x * (256 / LPR) + threadIdx.x / LPR, ng = (int64_t)gridDim.x * (256 / LPR);
  float dgs[J], dbs[J], gv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    dgs[j] = dbs[j] = 0.f;
    const int c = l16 + LPR * j;
    gv[j] = c < C ? bf2f(g[c]) : 0.f;
  }
  const float invC = 1.0f / C;
  for (int64_t r = grp; r < rows; r += ng) {
    float xv[J], dv[J];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = l16 + LPR * j;
      xv[j] = c < C ? Elem<TX>::load(x, r * C + c) : 0.f;
      dv[j] = c < C ? bf2f(dy[r * C + c]) : 0.f;
      s += xv[j];
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    const float mu = s * invC;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = l16 + LPR * j;
      const float d = c < C ? xv[j] - mu : 0.f;
      q += d * d;
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) q += __shfl_xor(q, o);
    const float rstd = 1.0f / sqrtf(q * invC + eps);
    float a = 0.f, bsum = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float xh = (xv[j] - mu) * rstd;
      const float dxh = dv[j] * gv[j];
      a += dxh;
      bsum += dxh * xh;
      dgs[j] += dv[j] * xh;
      dbs[j] += dv[j];
      xv[j] = xh;
      dv[j] = dxh;
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) {
      a += __shfl_xor(a, o);
      bsum += __shfl_xor(bsum, o);
    }
    a *= invC;
    bsum *= invC;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = l16 + LPR * j;
      if (c < C) {
        float v = rstd * (dv[j] - a - xv[j] * bsum);
        if (res) v += Elem<TR>::load(res, r * C + c);
        Elem<TO>::store(out, r * C + c, v);
      }
    }
  }
  // the workgroup's row groups into one partial: the wave's groups by
  // shuffles (lanes LPR apart), then the 4 waves' sums through LDS, in a
  // fixed order
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      dgs[j] += __shfl_xor(dgs[j], o);
      dbs[j] += __shfl_xor(dbs[j], o);
    }
  __shared__ float red[4][2 * 768];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) < LPR) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = l16 + LPR * j;
      if (c < C) {
        red[wave][c] = dgs[j];
        red[wave][C + c] = dbs[j];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * C; i += 256)
    part[(int64_t)blockIdx.x * 2 * C + i] = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
}

// An 8 x 8 block of bf16 rows (8 tokens m0 .. m0 + 7 of row pitch ld, 8
// channels from column c0) into LDS transposed: channel rows r0 .. r0 + 7
// (pitch kWgPitch), tokens t0 .. t0 + 7.  Each output dword pairs one
// channel of two consecutive tokens (a byte permute of the two tokens'
// dwords); rows past M are zero.
__device__ __forceinline__ void stage_t8x8(const bf16_t* __restrict__ X, int64_t ld, int64_t m0, int64_t M, int c0,
                                           bf16_t* dst, int r0, int t0) {
  u32x4_t r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r[i] = m0 + i < M ? *reinterpret_cast<const u32x4_t*>(X + (m0 + i) * ld + c0) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // input dword j: channels 2j (low half), 2j + 1 (high half)
    u32x4_t lo, hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // output dword q: tokens 2q (low half), 2q + 1 (high half)
      lo[q] = __builtin_amdgcn_perm(r[2 * q + 1][j], r[2 * q][j], 0x05040100u);
      hi[q] = __builtin_amdgcn_perm(r[2 * q + 1][j], r[2 * q][j], 0x07060302u);
    }
    *reinterpret_cast<u32x4_t*>(dst + (r0 + 2 * j) * kWgPitch + t0) = lo;
    *reinterpret_cast<u32x4_t*>(dst + (r0 + 2 * j + 1) * kWgPitch + t0) = hi;
  }
}

// Weight-gradient partials, one row of NO KI + NO floats per part p: the
// NO x KI sums over the tokens of chunks p, p + P, ... of A[m, n] * B[m, k],
// then the NO column sums of A (written by the k-block-0 workgroups).
// A: (M, NO), B: (M, KI), bf16 rows.
// Workgroup tile BN n x BK k, 4 waves sharing the (BN/16) (BK/16) output
// tiles in 2 x 2 blocks; MFMA A operand = A^T rows (n) and B operand = B^T
// rows (k), both token-contiguous in LDS.  Larger tiles re-read the operands
// fewer times.
template <int BN, int BK>
__global__ void __launch_bounds__(256) wgrad_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
                                                    float* __restrict__ part, int64_t M, int NO, int KI,
                                                    int nparts) {
  warm_args(A, B, part, M, NO, KI, nparts);
  extern __shared__ __attribute__((aligned(16))) unsigned char wg_lds[];
  bf16_t* At = reinterpret_cast<bf16_t*>(wg_lds);
  bf16_t* Bt = At + BN * kWgPitch;
  const int nblk = NO / BN, kblk = KI / BK;
  int bid = blockIdx.x;
  const int p = bid / (nblk * kblk);
  bid -= p * nblk * kblk;
  const int nb = bid / kblk, kb = bid - nb * kblk;
  const int n0 = nb * BN, k0 = kb * BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g4 = lane >> 4;
  // the (BN/16) x (BK/16) output tiles as 2 x 2 blocks of TN x TK tiles, one
  // block per wave: per 32-token step a wave reads TN A and TK B fragments
  // for its TN TK MFMAs
  static_assert(BN % 32 == 0 && BK % 32 == 0, "2 x 2 wave blocks of 16 x 16 tiles");
  constexpr int TN = BN / 32, TK = BK / 32, TPW = TN * TK;
  const int nt0 = (wave & 1) * TN, kt0 = (wave >> 1) * TK;
  constexpr int CSG = BN <= 32 ? 8 : (BN <= 64 ? 4 : 2);   // threads per column of the bias sums
  static_assert(BN * CSG <= 256, "column-sum threads");
  f32x4_t acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float cs = 0.f;
  const int64_t nchunks = (M + kWgChunk - 1) / kWgChunk;
  for (int64_t ch = p; ch < nchunks; ch += nparts) {
    const int64_t mc = ch * kWgChunk;
    __syncthreads();
    // the chunk's 256 tokens of A (BN channels) and B (BK channels) into LDS,
    // transposed in 8 x 8 blocks; consecutive threads take consecutive
    // channel blocks of the same 8 tokens (coalesced 16-byte loads)
    constexpr int NBA = (BN / 8) * (kWgChunk / 8), NBB = (BK / 8) * (kWgChunk / 8);
    for (int bI = tid; bI < NBA + NBB; bI += 256) {
      if (bI < NBA) {
        const int cb = bI % (BN / 8), tb = bI / (BN / 8);
        stage_t8x8(A, NO, mc + 8 * tb, M, n0 + 8 * cb, At, 8 * cb, 8 * tb);
      } else {
        const int b2 = bI - NBA;
        const int cb = b2 % (BK / 8), tb = b2 / (BK / 8);
        stage_t8x8(B, KI, mc + 8 * tb, M, k0 + 8 * cb, Bt, 8 * cb, 8 * tb);
      }
    }
    __syncthreads();
#pragma unroll 2
    for (int s = 0; s < kWgChunk / 32; ++s) {
      bf16x8_t a[TN], b[TK];
#pragma unroll
      for (int i = 0; i < TN; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(At + (16 * (nt0 + i) + fr) * kWgPitch + 32 * s + 8 * g4);
#pragma unroll
      for (int j = 0; j < TK; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bt + (16 * (kt0 + j) + fr) * kWgPitch + 32 * s + 8 * g4);
#pragma unroll
      for (int j = 0; j < TK; ++j)
#pragma unroll
        for (int i = 0; i < TN; ++i)
          acc[j * TN + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[j * TN + i], 0, 0, 0);
    }
    if (kb == 0 && tid < BN * CSG) {
      // column sums: thread -> n = tid / CSG, tokens (tid % CSG) * 256 / CSG ..
      const int n = tid / CSG, q = tid % CSG;
      float sm = 0.f;
      for (int t = 0; t < kWgChunk / CSG; ++t) sm += bf2f(At[n * kWgPitch + q * (kWgChunk / CSG) + t]);
      cs += sm;
    }
  }
  // lane: n = n0 + 16 nt + 4 g4 + r, k = k0 + 16 kt + fr
  float* prow = part + (int64_t)p * ((int64_t)NO * KI + NO);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int nt = nt0 + i % TN, kt = kt0 + i / TN;
    const int k = k0 + 16 * kt + fr;
#pragma unroll
    for (int r = 0; r < 4; ++r) prow[(int64_t)(n0 + 16 * nt + 4 * g4 + r) * KI + k] = acc[i][r];
  }
  if (kb == 0) {
#pragma unroll
    for (int o = 1; o < CSG; o <<= 1) cs += __shfl_xor(cs, o);
    if (tid % CSG == 0 && tid < BN * CSG) prow[(int64_t)NO * KI + n0 + tid / CSG] = cs;
  }
}

__global__ void __launch_bounds__(256) zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + (int64_t)threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
unsigned grid_for(int64_t work, int64_t per_block, int64_t cap = 4096) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}
}  // namespace

// dst (C x R) = src (R x C)^T, bf16, 32 x 32 tiles through LDS; up to 4
// matrices in one launch, blockIdx.z picking the job
__global__ void __launch_bounds__(256) transpose_jobs_kernel(const TransposeJobs jobs) {
  warm_args(jobs);
  const TransposeJob& j = jobs.job[blockIdx.z];
  __shared__ bf16_t t[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  if (c0 >= j.C || r0 >= j.R) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const bf16_t* src = (const bf16_t*)j.src;
  bf16_t* dst = (bf16_t*)j.dst;
  for (int i = ty; i < 32; i += 8)
    if (r0 + i < j.R && c0 + tx < j.C) t[i][tx] = src[(int64_t)(r0 + i) * j.C + c0 + tx];
  __syncthreads();
  for (int i = ty; i < 32; i += 8)
    if (c0 + i < j.C && r0 + tx < j.R) dst[(int64_t)(c0 + i) * j.R + r0 + tx] = t[tx][i];
}

hipError_t transpose_jobs(const TransposeJobs& jobs, hipStream_t st) {
  if (jobs.n <= 0) return hipSuccess;
  int mr = 1, mc = 1;
  for (int i = 0; i < jobs.n; ++i) {
    mr = jobs.job[i].R > mr ? jobs.job[i].R : mr;
    mc = jobs.job[i].C > mc ? jobs.job[i].C : mc;
  }
  transpose_jobs_kernel<<<dim3((unsigned)((mc + 31) / 32), (unsigned)((mr + 31) / 32), (unsigned)jobs.n), dim3(256),
                          0, st>>>(jobs);
  return hipGetLastError();
}


hipError_t gelu_apply(const void* a, void* io, int64_t n, int bwd, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  gelu_kernel<<<dim3(grid_for(n / 8, 256)), dim3(256), 0, st>>>((const bf16_t*)a, (bf16_t*)io, n, bwd);
  return hipGetLastError();
}

hipError_t gather_f32_bf16(const float* in, void* out, int64_t slots, int C, const WinGeo& geo, hipStream_t st) {
  if (slots <= 0) return hipSuccess;
  if (C % 8) return hipErrorInvalidValue;
  gather_f32_bf16_kernel<<<dim3(grid_for(slots * (C / 8), 256)), dim3(256), 0, st>>>(in, (bf16_t*)out, slots, C, geo);
  return hipGetLastError();
}

// workgroups of ln_bwd: up to 2048, each 256 / LPR row groups
int ln_bwd_blocks(int64_t rows, int C) {
  const int per = C <= 256 ? 16 : 4;
  const int64_t b = (rows + per - 1) / per;
  return (int)(b < 2048 ? b : 2048);
}

size_t ln_bwd_part_bytes(int64_t rows, int C) { return (size_t)ln_bwd_blocks(rows, C) * 2 * C * 4; }

hipError_t ln_bwd(int x_fp32, const void* x, const void* g, const void* dy, int res_fp32, const void* res,
                  int out_fp32, void* out, float* part, float* dg, float* db, int64_t rows, int C, float eps,
                  LnRed& red, hipStream_t st) {
  red = LnRed{part, dg, db, 0, C};
  if (rows <= 0) return hipSuccess;
  if (C > 768) return hipErrorInvalidValue;
  const int nb = ln_bwd_blocks(rows, C);
  const dim3 grid((unsigned)nb), block(256);
  const bf16_t* gb = (const bf16_t*)g;
  const bf16_t* dyb = (const bf16_t*)dy;
  auto go = [&](auto LJ) -> hipError_t {
    constexpr int LP = decltype(LJ)::value / 100, JJ = decltype(LJ)::value % 100;
    if (x_fp32 && !res_fp32 && out_fp32)
      ln_bwd_kernel<float, bf16_t, float, LP, JJ><<<grid, block, 0, st>>>((const float*)x, gb, dyb, (const bf16_t*)res,
                                                                      (float*)out, part, rows, C, eps);
    else if (!x_fp32 && res_fp32 && !out_fp32)
      ln_bwd_kernel<bf16_t, float, bf16_t, LP, JJ><<<grid, block, 0, st>>>((const bf16_t*)x, gb, dyb, (const float*)res,
                                                                       (bf16_t*)out, part, rows, C, eps);
    else if (!x_fp32 && !res_fp32 && !out_fp32)
      ln_bwd_kernel<bf16_t, bf16_t, bf16_t, LP, JJ><<<grid, block, 0, st>>>((const bf16_t*)x, gb, dyb,
                                                                        (const bf16_t*)res, (bf16_t*)out, part, rows,
                                                                        C, eps);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  };
  hipError_t e;
  // template value = 100 * lanes per row + elements per lane
  if (C <= 96) e = go(std::integral_constant<int, 1606>{});
  else if (C <= 128) e = go(std::integral_constant<int, 1608>{});
  else if (C <= 256) e = go(std::integral_constant<int, 1616>{});
  else e = go(std::integral_constant<int, 6412>{});
  red.np = nb;
  return e;
}

// dg = sum over workgroups of part[b][0:C], db of part[b][C:2C]; one
// workgroup per output, blockIdx.y = job
__global__ void __launch_bounds__(256) ln_reduce_kernel(const LnReds jobs) {
  warm_args(jobs);
  const LnRed& j = jobs.job[blockIdx.y];
  const int i = blockIdx.x;
  if (i >= 2 * j.C) return;   // the whole workgroup
  __shared__ float red[256];
  float s = 0.f;
  for (int p = (int)threadIdx.x; p < j.np; p += 256) s += j.part[(int64_t)p * 2 * j.C + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (i < j.C) j.dg[i] = red[0];
    else j.db[i - j.C] = red[0];
  }
}

hipError_t ln_reduce(const LnReds& jobs, hipStream_t st) {
  if (jobs.n <= 0) return hipSuccess;
  int cmax = 1;
  for (int i = 0; i < jobs.n; ++i) cmax = jobs.job[i].C > cmax ? jobs.job[i].C : cmax;
  ln_reduce_kernel<<<dim3((unsigned)(2 * cmax), (unsigned)jobs.n), dim3(256), 0, st>>>(jobs);
  return hipGetLastError();
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t st) {
  if (!p || n <= 0) return hipSuccess;
  zero_f32_kernel<<<dim3(grid_for(n, 256)), dim3(256), 0, st>>>(p, n);
  return hipGetLastError();
}

namespace {
// output tiles of the wgrad kernel the launcher picks for (NO, KI)
int64_t wgrad_tiles(int NO, int KI) {
  if (NO % 96 == 0 && KI % 96 == 0) return (int64_t)(NO / 96) * (KI / 96);
  if (NO % 96 == 0 && KI % 128 == 0) return (int64_t)(NO / 96) * (KI / 128);
  if (NO % 32 == 0 && KI % 128 == 0) return (int64_t)(NO / 32) * (KI / 128);
  if (NO % 32 == 0 && KI % 96 == 0) return (int64_t)(NO / 32) * (KI / 96);
  return (int64_t)(NO / 32) * (KI / 32);
}
// token partitions of one weight gradient: 64, or more where the output
// has so few tiles that 64 partitions leave CUs idle (enough for kWgBlocks
// workgroups, at most kMaxParts), and at most one per 256-token chunk
int64_t wgrad_parts(int64_t M, int NO, int KI) {
  const int64_t nchunks = (M + kWgChunk - 1) / kWgChunk;
  const int64_t tiles = wgrad_tiles(NO, KI);
  int64_t np = (kWgBlocks + tiles - 1) / tiles;
  if (np < 64) np = 64;
  if (np > kMaxParts) np = kMaxParts;
  return np < nchunks ? np : nchunks;
}
}  // namespace

size_t wgrad_part_bytes(int64_t M, int NO, int KI) {
  return (size_t)wgrad_parts(M, NO, KI) * ((size_t)NO * KI + NO) * 4;
}

hipError_t wgrad_partials(const void* A, const void* B, float* dW, float* db, float* part, int64_t M, int NO, int KI,
                          WgradJob& job, hipStream_t st) {
  if (NO % 32 || KI % 32) return hipErrorInvalidValue;
  const int64_t nw = (int64_t)NO * KI;
  job = WgradJob{part, dW, db, 0, nw + (db ? NO : 0), nw, nw + NO};
  if (M <= 0) return hipSuccess;   // no tokens: the reduction writes zeros
  const int np = (int)wgrad_parts(M, NO, KI);
  job.np = np;
  // n tile 96 where it divides NO, else 32; k tile 96 or 128 where it divides
  // KI, else 32
  auto launch = [&](auto kern, int bn, int bk) -> hipError_t {
    const size_t lds = (size_t)(bn + bk) * kWgPitch * 2;
    hipError_t e = ensure_dynamic_lds((const void*)kern, lds);
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)(np * (NO / bn) * (KI / bk))), dim3(256), lds, st>>>((const bf16_t*)A, (const bf16_t*)B,
                                                                             part, M, NO, KI, np);
    return hipGetLastError();
  };
  if (NO % 96 == 0 && KI % 96 == 0) return launch(wgrad_kernel<96, 96>, 96, 96);
  if (NO % 96 == 0 && KI % 128 == 0) return launch(wgrad_kernel<96, 128>, 96, 128);
  if (NO % 32 == 0 && KI % 128 == 0) return launch(wgrad_kernel<32, 128>, 32, 128);
  if (NO % 32 == 0 && KI % 96 == 0) return launch(wgrad_kernel<32, 96>, 32, 96);
  return launch(wgrad_kernel<32, 32>, 32, 32);
}

// every job's dW and db from its partial rows, one launch (blockIdx.y = job):
// a workgroup takes 64 consecutive outputs, its 4 waves sum every fourth
// partial row (so a long partial list is read 4 rows at a time) and one
// wave adds the 4 sums (fixed order: the result does not depend on timing)
__global__ void __launch_bounds__(256) wgrad_reduce_kernel(const WgradJobs jobs) {
  warm_args_grid(jobs);
  const WgradJob& j = jobs.job[blockIdx.y];
  __shared__ float red[4][64];
  const int o = (int)threadIdx.x & 63, g = (int)threadIdx.x >> 6;
  for (int64_t i0 = (int64_t)blockIdx.x * 64; i0 < j.n; i0 += (int64_t)gridDim.x * 64) {
    const int64_t i = i0 + o;
    float s = 0.f;
    if (i < j.n) {
#pragma unroll 8
      for (int p = g; p < j.np; p += 4) s += j.part[(int64_t)p * j.stride + i];
    }
    __syncthreads();
    red[g][o] = s;
    __syncthreads();
    if (g == 0 && i < j.n) {
      const float t = (red[0][o] + red[1][o]) + (red[2][o] + red[3][o]);
      if (i < j.n1) j.dW[i] = t;
      else j.db[i - j.n1] = t;
    }
  }
}

hipError_t wgrad_reduce(const WgradJobs& jobs, hipStream_t st) {
  if (jobs.n <= 0) return hipSuccess;
  int64_t nmax = 1;
  for (int i = 0; i < jobs.n; ++i) nmax = jobs.job[i].n > nmax ? jobs.job[i].n : nmax;
  wgrad_reduce_kernel<<<dim3(grid_for(nmax, 64), (unsigned)jobs.n), dim3(256), 0, st>>>(jobs);
  return hipGetLastError();
}

}  // namespace vswin
