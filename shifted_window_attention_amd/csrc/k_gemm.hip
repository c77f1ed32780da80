// Linear layers of the Video Swin block (qkv, proj, fc1, fc2, patch embed,
// patch merge): out = A (M x K) * W^T + bias with a fused epilogue.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 (fp32 accumulate).  The kernel
// computes C^T tiles -- MFMA operand A = 16 weight rows (features), operand
// B = 16 activation rows (tokens), both K-contiguous in global memory and in
// LDS -- so each lane ends with 4 consecutive output features of one token
// and the epilogue writes 8- or 16-byte vectors.  Block tile 128 tokens x BN
// features, 4 waves as 2 x 2, K staged 32 at a time through double-buffered
// LDS with an 80-byte row pitch (conflict-free 16-byte fragment reads).
// fp32 path: v_mfma_f32_16x16x4_f32 with the same C^T tiling (a plain
// LDS-tiled FMA kernel for feature counts that are not a multiple of 4).
#include "vswin_kernels.h"

#include <type_traits>

namespace vswin {

__device__ __forceinline__ float gelu_erf(float x) {
  // exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

template <typename T, Epi KIND>
struct EpiDev {
  EpiArgs a;
  // block computes token-major fragments (V^T output of the qkv projection)
  __device__ __forceinline__ bool swapped(int n0) const {
    if constexpr (KIND == Epi::kQKV) return a.vt && n0 >= 2 * a.C;
    else return false;
  }
  // four consecutive window rows m4..m4+3 (same window) of feature n
  __device__ __forceinline__ void store_t(int64_t m4, int n, float v[4]) const {
    if constexpr (KIND == Epi::kQKV) {
      const float b = a.bias ? Elem<T>::load((const T*)a.bias, n) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += b;
      const int c = n - 2 * a.C;
      const int h = c / a.d;
      const int e = c - h * a.d;
      const int w = (int)m4 / a.N;
      const int t = (int)m4 - w * a.N;
      store4((T*)a.out3, ((int64_t)(w * a.heads + h) * a.d + e) * a.N + t, v);
    }
  }
  __device__ __forceinline__ int64_t row_ctx(int64_t m) const {
    if constexpr (KIND == Epi::kProjRes || KIND == Epi::kProjOut) {
      int lab;
      const int w = (int)m / a.N;
      return slot_source(a.geo, w, (int)m - w * a.N, lab);
    } else {
      return m;
    }
  }
  __device__ __forceinline__ void store(int64_t m, int64_t rc, int n0, float v[4]) const {
    if (a.bias) {
      float bb[4];
      load4((const T*)a.bias, n0, bb);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += bb[i];
    }
    if constexpr (KIND == Epi::kBias) {
      store4((T*)a.out, m * a.ld_out + n0, v);
    } else if constexpr (KIND == Epi::kGelu) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = gelu_erf(v[i]);
      store4((T*)a.out, m * a.ld_out + n0, v);
    } else if constexpr (KIND == Epi::kRes) {
      float r[4];
      load4((const float*)a.res, m * a.ld_out + n0, r);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += r[i];
      store4((T*)a.out, m * a.ld_out + n0, v);
    } else if constexpr (KIND == Epi::kQKV) {
      const int which = n0 / a.C;
      const int c = n0 - which * a.C;
      const int h = c / a.d;
      const int e = c - h * a.d;
      const int w = (int)m / a.N;
      const int t = (int)m - w * a.N;
      T* base = (T*)(which == 0 ? a.out : (which == 1 ? a.out2 : a.out3));
      store4(base, ((int64_t)(w * a.heads + h) * a.N + t) * a.d + e, v);
    } else if constexpr (KIND == Epi::kProjRes) {
      if (rc < 0) return;
      float r[4];
      load4((const T*)a.res, rc * a.C + n0, r);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += r[i];
      store4((float*)a.out, rc * a.C + n0, v);
    } else {  // kProjOut
      if (rc < 0) return;
      store4((T*)a.out, rc * a.C + n0, v);
    }
  }
};

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM
// ---------------------------------------------------------------------------
constexpr int kBM = 128, kBK = 32, kLDK = 40;

template <int BN, class E>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                        int64_t M, int N, int K, E epi) {
  warm_args(A, W, M, N, K, epi);
  constexpr int WN = BN / 2;
  constexpr int NT = WN / 16;
  constexpr int MT = 4;
  constexpr int WCH = (BN * 4 + 255) / 256;   // 16-byte weight chunks per thread
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kBM * kLDK];
  __shared__ __attribute__((aligned(16))) bf16_t Ws[2][BN * kLDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nb = N / BN;
  const int64_t bm = blockIdx.x / nb;
  const int bn = (int)(blockIdx.x - bm * nb);
  const int64_t m0 = bm * kBM;
  const int n0 = bn * BN;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[2], rw[WCH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 2, kc = (c & 3) * 8;
      const int64_t m = m0 + r;
      if (m < M) ra[i] = *reinterpret_cast<const u32x4_t*>(A + m * K + kt * kBK + kc);
      else ra[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + 256 * i;
      if (c < BN * 4) {
        const int r = c >> 2, kc = (c & 3) * 8;
        rw[i] = *reinterpret_cast<const u32x4_t*>(W + (int64_t)(n0 + r) * K + kt * kBK + kc);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 2, kc = (c & 3) * 8;
      *reinterpret_cast<u32x4_t*>(&As[buf][r * kLDK + kc]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int c = tid + 256 * i;
      if (c < BN * 4) {
        const int r = c >> 2, kc = (c & 3) * 8;
        *reinterpret_cast<u32x4_t*>(&Ws[buf][r * kLDK + kc]) = rw[i];
      }
    }
  };

  const int nk = K / kBK;
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  auto mainloop = [&](auto swap_tag) {
    constexpr bool SWAP = decltype(swap_tag)::value;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      bf16x8_t af[MT], wf[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8_t*>(&As[buf][(wm * 64 + mt * 16 + fr) * kLDK + fk]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        wf[nt] = *reinterpret_cast<const bf16x8_t*>(&Ws[buf][(wn * WN + nt * 16 + fr) * kLDK + fk]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (SWAP)   // rows = tokens, cols = features
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], wf[nt], acc[mt][nt], 0, 0, 0);
          else                  // rows = features, cols = tokens
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt], af[mt], acc[mt][nt], 0, 0, 0);
        }
      if (kt + 1 < nk) sstore(buf ^ 1);
      __syncthreads();
    }
    if constexpr (SWAP) {
      // lane: feature column fr, tokens 4*(lane>>4) .. +3 of each 16-row tile
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m4 = m0 + wm * 64 + mt * 16 + (lane >> 4) * 4;
        if (m4 >= M) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
          epi.store_t(m4, n0 + wn * WN + nt * 16 + fr, v);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = m0 + wm * 64 + mt * 16 + fr;
        if (m >= M) continue;
        const int64_t rc = epi.row_ctx(m);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + wn * WN + nt * 16 + (lane >> 4) * 4;
          float v[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
          epi.store(m, rc, n, v);
        }
      }
    }
  };
  if (epi.swapped(n0)) mainloop(std::true_type{});
  else mainloop(std::false_type{});
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM for K a multiple of 64: block tile 128 tokens x BN features,
// 4 waves as 2 x 2, K staged 64 at a time through a ring of S LDS stages
// filled by global_load_lds_dwordx4 (one wave instruction moves 8 rows of 128
// bytes straight into LDS: no register staging, no LDS store instructions).
// Up to S - 1 stages are in flight while one is multiplied.  A stage holds
// the 128 A rows and then the BN W rows, 128 bytes each; the 16-byte chunk c
// of row r sits at chunk c ^ ((r >> 1) & 7), so the 16 rows of a fragment
// read fall on 16 distinct 4-bank groups.  Workgroup b takes tile number
// (b mod 8) * share + b / 8: the tiles of one XCD are consecutive (all
// feature tiles of a token block share that XCD's L2).
// The loads are issued from inline assembly and waited for with explicit
// vmcnt counts: the compiler's own tracking of LDS DMA would wait for every
// outstanding stage before reading any of them.  M0 carries the LDS address
// of each load and is used for nothing else in this kernel.
// ---------------------------------------------------------------------------
constexpr int kDBK = 64;

template <int BN, int S>
struct DmaTile {
  static constexpr int kRows = kBM + BN;           // LDS rows per stage
  static constexpr int kStage = kRows * 128;        // bytes per stage
  static constexpr int kPerWave = kRows / 8 / 4;    // DMA instructions per wave per stage
  static constexpr int kLds = S * kStage;
  static_assert(kRows % 32 == 0, "rows per stage must split over 4 waves x 8 rows");
  static_assert(S >= 2 && S <= 4, "2 to 4 stages");
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_byte)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// wait until at most `stages` stages of D loads each are outstanding
template <int S, int D>
__device__ __forceinline__ void wait_stages(int stages) {
  if constexpr (S == 2) {
    wait_vm_lgkm0<0>();
  } else if constexpr (S == 3) {
    if (stages > 0) wait_vm_lgkm0<D>();
    else wait_vm_lgkm0<0>();
  } else {
    if (stages > 2) wait_vm_lgkm0<3 * D>();
    else if (stages > 1) wait_vm_lgkm0<2 * D>();
    else if (stages > 0) wait_vm_lgkm0<D>();
    else wait_vm_lgkm0<0>();
  }
}

template <int BN, int S, class E>
__global__ void __launch_bounds__(256) gemm_bf16_dma_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                            int64_t M, int N, int K, E epi, int tq, int tr) {
  warm_args(A, W, M, N, K, epi, tq, tr);
  using T = DmaTile<BN, S>;
  constexpr int WN = BN / 2;
  constexpr int NT = WN / 16;
  constexpr int MT = 4;
  constexpr int D = T::kPerWave;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // XCD-contiguous tile numbering
  const int b = blockIdx.x, xcd = b & 7;
  const int tile = xcd * tq + min(xcd, tr) + (b >> 3);
  const int nb = N / BN;
  const int bm = tile / nb;
  const int bn = tile - bm * nb;
  const int64_t m0 = (int64_t)bm * kBM;
  const int n0 = bn * BN;

  // per-lane source pointers of this wave's DMA instructions (stage 0)
  const bf16_t* gp[D];
  uint32_t lo[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int j = wave + 4 * i;                 // instruction index: rows 8j .. 8j + 7 of the stage
    const int row = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    if (row < kBM) {
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;                    // rows past M load row M - 1 (never stored)
      gp[i] = A + m * K + 8 * c;
    } else {
      gp[i] = W + (int64_t)(n0 + row - kBM) * K + 8 * c;
    }
    lo[i] = __builtin_amdgcn_readfirstlane(8 * j * 128);
  }
  auto issue = [&](int kt, int slot) {   // stage kt (K columns 64 kt ..) into LDS slot
    const uint32_t sb = lds0 + (uint32_t)(slot * T::kStage);
#pragma unroll
    for (int i = 0; i < D; ++i) lds_dma16(gp[i] + (int64_t)kt * kDBK, sb + lo[i]);
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, g4 = lane >> 4;
  const int sx = (fr >> 1) & 7;
  const int xo0 = ((g4 ^ sx) << 4), xo1 = (((4 + g4) ^ sx) << 4);
  const int nk = K / kDBK;
  auto mainloop = [&](auto swap_tag) {
    constexpr bool SWAP = decltype(swap_tag)::value;
    auto frags = [&](int slot, int s, bf16x8_t (&af)[MT], bf16x8_t (&wf)[NT]) {
      const unsigned char* st = smem + slot * T::kStage;
      const int xo = s ? xo1 : xo0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8_t*>(st + (wm * 64 + mt * 16 + fr) * 128 + xo);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        wf[nt] = *reinterpret_cast<const bf16x8_t*>(st + (kBM + wn * WN + nt * 16 + fr) * 128 + xo);
    };
    auto mma = [&](const bf16x8_t (&af)[MT], const bf16x8_t (&wf)[NT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (SWAP)   // rows = tokens, cols = features
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], wf[nt], acc[mt][nt], 0, 0, 0);
          else                  // rows = features, cols = tokens
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt], af[mt], acc[mt][nt], 0, 0, 0);
        }
    };
    // Stage kt lands in slot kt % S.  A step waits for the next stage, reads
    // its first half (32 k) of fragments while the current stage's second
    // half multiplies, then its second half while the first half multiplies;
    // a slot is refilled (stage kt + S) as soon as every wave holds all of
    // stage kt's fragments.  The wait and barrier open the loop body: placed
    // after the products, they make the compiler move the accumulators
    // between registers at every step.
    const int pre = nk < S ? nk : S;
    for (int q = 0; q < pre; ++q) issue(q, q);
    wait_stages<S, D>(pre - 1);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    bf16x8_t a0[MT], w0[NT], a1[MT], w1[NT];
    frags(0, 0, a0, w0);
    frags(0, 1, a1, w1);
    mma(a0, w0);
    int slot = 0;
    for (int kt = 0; kt + 1 < nk; ++kt) {
      asm volatile("" ::: "memory");
      // stage kt + 1 landed; stages kt + 2 .. kt + S - 1 may be in flight
      wait_stages<S, D>((kt + S - 1 < nk - 1 ? kt + S - 1 : nk - 1) - (kt + 1));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + S < nk) issue(kt + S, slot);
      slot = slot == S - 1 ? 0 : slot + 1;
      frags(slot, 0, a0, w0);
      mma(a1, w1);
      frags(slot, 1, a1, w1);
      mma(a0, w0);
    }
    mma(a1, w1);
    if constexpr (SWAP) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m4 = m0 + wm * 64 + mt * 16 + g4 * 4;
        if (m4 >= M) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
          epi.store_t(m4, n0 + wn * WN + nt * 16 + fr, v);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = m0 + wm * 64 + mt * 16 + fr;
        if (m >= M) continue;
        const int64_t rc = epi.row_ctx(m);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + wn * WN + nt * 16 + g4 * 4;
          float v[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
          epi.store(m, rc, n, v);
        }
      }
    }
  };
  if (epi.swapped(n0)) mainloop(std::true_type{});
  else mainloop(std::false_type{});
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM with the whole K extent (K <= 128) staged in one batch:
// one global round trip and one barrier per workgroup.  The A rows can be
// gathered through the window map and layer-normalised on the way into LDS
// (LN1 + pad + roll + partition fused into the qkv projection).
// ---------------------------------------------------------------------------
struct APrologue {
  int mode;              // 0: rows of A; 1: gather x rows by slot; 2: gather + LayerNorm
  const bf16_t* x;       // modes 1, 2: token rows (B*T*H*W, K)
  const bf16_t* g;       // mode 2: LN gamma, beta (K)
  const bf16_t* b;
  float eps;
  WinGeo geo;
};

template <int BN, int KK, class E>
__global__ void __launch_bounds__(256) gemm_bf16_fullk_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                              int64_t M, int N, E epi, APrologue pro) {
  warm_args(A, W, M, N, epi, pro);
  constexpr int WN = BN / 2;
  constexpr int NT = WN / 16;
  constexpr int MT = 4;
  constexpr int LD = KK + 8;                 // row pitch (elements): 16-byte multiple, rows spread over banks
  constexpr int HALF = KK / 2;               // elements per thread of one A row (2 threads per row)
  constexpr int ACH = HALF / 8;              // 16-byte chunks per thread of one A row
  constexpr int WCH = (BN * KK / 8 + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[kBM * LD];
  __shared__ __attribute__((aligned(16))) bf16_t Ws[BN * LD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nb = N / BN;
  const int64_t bm = blockIdx.x / nb;
  const int bn = (int)(blockIdx.x - bm * nb);
  const int64_t m0 = bm * kBM;
  const int n0 = bn * BN;

  // ---- issue all global loads: this thread's half of one A row, its W chunks
  const int arow = tid >> 1, ahalf = tid & 1;
  const int64_t am = m0 + arow;
  const bf16_t* asrc = nullptr;
  if (am < M) {
    if (pro.mode == 0) {
      asrc = A + am * KK;
    } else {
      int lab;
      const int w = (int)am / pro.geo.N;
      const int64_t src = slot_source(pro.geo, w, (int)am - w * pro.geo.N, lab);
      if (src >= 0) asrc = pro.x + src * KK;
    }
  }
  u32x4_t av[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i)
    av[i] = asrc ? *reinterpret_cast<const u32x4_t*>(asrc + ahalf * HALF + i * 8) : u32x4_t{0u, 0u, 0u, 0u};
  u32x4_t wv[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + 256 * i;
    if (c < BN * KK / 8) {
      const int r = c / (KK / 8), k = (c % (KK / 8)) * 8;
      wv[i] = *reinterpret_cast<const u32x4_t*>(W + (int64_t)(n0 + r) * KK + k);
    }
  }
  // ---- optional LayerNorm of the A row (two threads per row)
  if (pro.mode == 2) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < ACH; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += bflo(av[i][e]) + bfhi(av[i][e]);
    s += __shfl_xor(s, 1);
    const float mean = s * (1.0f / KK);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < ACH; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = bflo(av[i][e]) - mean, d1 = bfhi(av[i][e]) - mean;
        q += d0 * d0 + d1 * d1;
      }
    q += __shfl_xor(q, 1);
    const float rstd = 1.0f / sqrtf(q * (1.0f / KK) + pro.eps);
    if (asrc) {
#pragma unroll
      for (int i = 0; i < ACH; ++i) {
        const int k0 = ahalf * HALF + i * 8;
        const u32x4_t gg = *reinterpret_cast<const u32x4_t*>(pro.g + k0);
        const u32x4_t bb = *reinterpret_cast<const u32x4_t*>(pro.b + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = (bflo(av[i][e]) - mean) * rstd * bflo(gg[e]) + bflo(bb[e]);
          const float hi = (bfhi(av[i][e]) - mean) * rstd * bfhi(gg[e]) + bfhi(bb[e]);
          av[i][e] = pack_bf16x2(lo, hi);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < ACH; ++i)
    *reinterpret_cast<u32x4_t*>(&As[arow * LD + ahalf * HALF + i * 8]) = av[i];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + 256 * i;
    if (c < BN * KK / 8) {
      const int r = c / (KK / 8), k = (c % (KK / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(&Ws[r * LD + k]) = wv[i];
    }
  }
  __syncthreads();

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto run = [&](auto swap_tag) {
    constexpr bool SWAP = decltype(swap_tag)::value;
#pragma unroll
    for (int k = 0; k < KK; k += 32) {
      bf16x8_t af[MT], wf[NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * 64 + mt * 16 + fr) * LD + k + fk]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        wf[nt] = *reinterpret_cast<const bf16x8_t*>(&Ws[(wn * WN + nt * 16 + fr) * LD + k + fk]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (SWAP)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], wf[nt], acc[mt][nt], 0, 0, 0);
          else
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nt], af[mt], acc[mt][nt], 0, 0, 0);
        }
    }
    if constexpr (SWAP) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m4 = m0 + wm * 64 + mt * 16 + (lane >> 4) * 4;
        if (m4 >= M) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float v[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
          epi.store_t(m4, n0 + wn * WN + nt * 16 + fr, v);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = m0 + wm * 64 + mt * 16 + fr;
        if (m >= M) continue;
        const int64_t rc = epi.row_ctx(m);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + wn * WN + nt * 16 + (lane >> 4) * 4;
          float v[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
          epi.store(m, rc, n, v);
        }
      }
    }
  };
  if (epi.swapped(n0)) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// fp32 MFMA GEMM: v_mfma_f32_16x16x4_f32 (fp32 operands, fp32 accumulate).
// Block tile 64 tokens x 64 features, 4 waves as 2 x 2 of 32 x 32; K staged
// 16 at a time through LDS (row pitch 17 floats: conflict-free column
// reads).  As in the bf16 kernel the product is C^T (operand A = weight rows,
// operand B = token rows), so a lane ends with 4 consecutive features of one
// token for the epilogue.
// ---------------------------------------------------------------------------
template <class E>
__global__ void __launch_bounds__(256) gemm_f32_mfma_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                            int64_t M, int N, int K, E epi) {
  warm_args(A, W, M, N, K, epi);
  __shared__ float As[64 * 17];
  __shared__ float Ws[64 * 17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, g4 = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int nb = (N + 63) / 64;
  const int64_t bm = blockIdx.x / nb;
  const int bn = (int)(blockIdx.x - bm * nb);
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, kk = idx & 15;
      const int64_t m = bm * 64 + r;
      const int n = bn * 64 + r;
      As[r * 17 + kk] = (m < M && k0 + kk < K) ? A[m * K + k0 + kk] : 0.f;
      Ws[r * 17 + kk] = (n < N && k0 + kk < K) ? W[(int64_t)n * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      float af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = As[(wm * 32 + i * 16 + fr) * 17 + 4 * k4 + g4];
        wf[i] = Ws[(wn * 32 + i * 16 + fr) * 17 + 4 * k4 + g4];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(wf[j], af[i], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane: token wm*32 + i*16 + fr, features wn*32 + j*16 + 4 g4 .. + 3
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = bm * 64 + wm * 32 + i * 16 + fr;
    if (m >= M) continue;
    const int64_t rc = epi.row_ctx(m);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = bn * 64 + wn * 32 + j * 16 + 4 * g4;
      if (n >= N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      epi.store(m, rc, n, v);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA GEMM (64 x 64 tile, 4 x 4 outputs per thread): feature counts that
// are not a multiple of 4
// ---------------------------------------------------------------------------
template <class E>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                       int64_t M, int N, int K, E epi) {
  warm_args(A, W, M, N, K, epi);
  __shared__ float As[16][68];
  __shared__ float Ws[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int nb = (N + 63) / 64;
  const int64_t bm = blockIdx.x / nb;
  const int bn = (int)(blockIdx.x - bm * nb);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, kk = idx & 15;
      const int64_t m = bm * 64 + r;
      const int n = bn * 64 + r;
      As[kk][r] = (m < M && k0 + kk < K) ? A[m * K + k0 + kk] : 0.f;
      Ws[kk][r] = (n < N && k0 + kk < K) ? W[(int64_t)n * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; w[i] = Ws[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = bm * 64 + ty * 4 + i;
    const int n = bn * 64 + tx * 4;
    if (m < M && n < N) {
      const int64_t rc = epi.row_ctx(m);
      float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      epi.store(m, rc, n, v);
    }
  }
}

// tile of the staged-K kernel for this shape: feature width (0: not served)
// and LDS stages.  F is the width every feature tile must stay inside (q, k,
// v for the qkv projection).  64-wide feature tiles (24 KB per stage) let
// several workgroups share a CU; the stage count trades depth for
// residency: with at most one tile per CU, four stages (one workgroup per
// CU); up to two, three stages (two per CU); more, two stages (three per
// CU).  Measured on the Swin-T backbone's projections (K = 192 .. 3072).
struct DmaChoice {
  int bn, stages;
};
static DmaChoice dma_choice(int64_t M, int N, int K, int F) {
  DmaChoice c{0, 2};
  if (K % kDBK != 0 || K < kDBK || M <= 0) return c;
  if (N % 64 == 0 && F % 64 == 0) c.bn = 64;
  else if (N % 96 == 0 && F % 96 == 0) c.bn = 96;
  else return c;
  const int64_t tiles = (M + kBM - 1) / kBM * (N / c.bn);
  c.stages = tiles <= 256 ? 4 : (tiles <= 512 ? 3 : 2);
  return c;
}

template <Epi KIND>
static hipError_t launch_kind(vswin_dtype dt, const void* A, const void* W, int64_t M, int N, int K,
                              const EpiArgs& e, const APrologue& pro, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (dt == VSWIN_BF16 && (K == 96 || K == 128)) {
    EpiDev<bf16_t, KIND> epi{e};
    const int64_t mb = (M + kBM - 1) / kBM;
    const int F = KIND == Epi::kQKV ? e.C : N;
    auto go = [&](auto kern, int bn) {
      kern<<<dim3((unsigned)(mb * (N / bn))), dim3(256), 0, st>>>((const bf16_t*)A, (const bf16_t*)W, M, N, epi, pro);
    };
    if (K == 96) {
      if (N % 96 == 0 && F % 96 == 0) go(gemm_bf16_fullk_kernel<96, 96, EpiDev<bf16_t, KIND>>, 96);
      else if (N % 64 == 0 && F % 64 == 0) go(gemm_bf16_fullk_kernel<64, 96, EpiDev<bf16_t, KIND>>, 64);
      else go(gemm_bf16_fullk_kernel<32, 96, EpiDev<bf16_t, KIND>>, 32);
    } else {
      if (N % 128 == 0 && F % 128 == 0) go(gemm_bf16_fullk_kernel<128, 128, EpiDev<bf16_t, KIND>>, 128);
      else if (N % 64 == 0 && F % 64 == 0) go(gemm_bf16_fullk_kernel<64, 128, EpiDev<bf16_t, KIND>>, 64);
      else go(gemm_bf16_fullk_kernel<32, 128, EpiDev<bf16_t, KIND>>, 32);
    }
  } else if (dt == VSWIN_BF16 && pro.mode == 0 && dma_choice(M, N, K, KIND == Epi::kQKV ? e.C : N).bn != 0) {
    EpiDev<bf16_t, KIND> epi{e};
    const DmaChoice ch = dma_choice(M, N, K, KIND == Epi::kQKV ? e.C : N);
    const int64_t tiles = (M + kBM - 1) / kBM * (N / ch.bn);
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    auto go = [&](auto kern, int lds) -> hipError_t {
      const hipError_t le = ensure_dynamic_lds((const void*)kern, lds);
      if (le != hipSuccess) return le;
      kern<<<dim3((unsigned)tiles), dim3(256), lds, st>>>((const bf16_t*)A, (const bf16_t*)W, M, N, K, epi,
                                                         (int)(tiles / 8), (int)(tiles % 8));
      return hipGetLastError();
    };
#define VSWIN_DMA_GO(BN_, S_)                                                       \
  if (ch.bn == BN_ && ch.stages == S_)                                              \
    return go(gemm_bf16_dma_kernel<BN_, S_, EpiDev<bf16_t, KIND>>, DmaTile<BN_, S_>::kLds);
    VSWIN_DMA_GO(64, 2) VSWIN_DMA_GO(64, 3) VSWIN_DMA_GO(64, 4)
    VSWIN_DMA_GO(96, 2) VSWIN_DMA_GO(96, 3) VSWIN_DMA_GO(96, 4)
#undef VSWIN_DMA_GO
    return hipErrorInvalidValue;
  } else if (dt == VSWIN_BF16) {
    if (pro.mode != 0) return hipErrorInvalidValue;   // gathered A rows need the full-K kernel
    EpiDev<bf16_t, KIND> epi{e};
    const int64_t mb = (M + kBM - 1) / kBM;
    auto go = [&](auto kern, int bn) {
      const int64_t blocks = mb * (N / bn);
      kern<<<dim3((unsigned)blocks), dim3(256), 0, st>>>((const bf16_t*)A, (const bf16_t*)W, M, N, K, epi);
    };
    // the qkv projection needs every feature tile inside one of q, k, v
    const int F = KIND == Epi::kQKV ? e.C : N;
    if (N % 128 == 0 && F % 128 == 0) go(gemm_bf16_kernel<128, EpiDev<bf16_t, KIND>>, 128);
    else if (N % 96 == 0 && F % 96 == 0) go(gemm_bf16_kernel<96, EpiDev<bf16_t, KIND>>, 96);
    else if (N % 64 == 0 && F % 64 == 0) go(gemm_bf16_kernel<64, EpiDev<bf16_t, KIND>>, 64);
    else go(gemm_bf16_kernel<32, EpiDev<bf16_t, KIND>>, 32);
  } else {
    if (pro.mode != 0) return hipErrorInvalidValue;
    EpiDev<float, KIND> epi{e};
    const int64_t blocks = ((M + 63) / 64) * ((N + 63) / 64);
    if (N % 4 == 0)
      gemm_f32_mfma_kernel<EpiDev<float, KIND>><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
          (const float*)A, (const float*)W, M, N, K, epi);
    else
      gemm_f32_kernel<EpiDev<float, KIND>><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
          (const float*)A, (const float*)W, M, N, K, epi);
  }
  return hipGetLastError();
}

bool gemm_can_gather(vswin_dtype dt, int K) { return dt == VSWIN_BF16 && (K == 96 || K == 128); }

hipError_t gemm(vswin_dtype dt, const void* A, const void* W, int64_t M, int N, int K, const EpiArgs& e,
                hipStream_t st, const GatherA* ga) {
  APrologue pro{};
  if (ga) {
    pro.mode = ga->ln ? 2 : 1;
    pro.x = (const bf16_t*)ga->x;
    pro.g = (const bf16_t*)ga->g;
    pro.b = (const bf16_t*)ga->b;
    pro.eps = ga->eps;
    pro.geo = ga->geo;
  }
  switch (e.kind) {
    case Epi::kBias: return launch_kind<Epi::kBias>(dt, A, W, M, N, K, e, pro, st);
    case Epi::kQKV: return launch_kind<Epi::kQKV>(dt, A, W, M, N, K, e, pro, st);
    case Epi::kProjRes: return launch_kind<Epi::kProjRes>(dt, A, W, M, N, K, e, pro, st);
    case Epi::kProjOut: return launch_kind<Epi::kProjOut>(dt, A, W, M, N, K, e, pro, st);
    case Epi::kGelu: return launch_kind<Epi::kGelu>(dt, A, W, M, N, K, e, pro, st);
    case Epi::kRes: return launch_kind<Epi::kRes>(dt, A, W, M, N, K, e, pro, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vswin
