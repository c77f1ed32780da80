// Shared host/device definitions of the vswin HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vswin.h"

namespace vswin {

// ---------------------------------------------------------------------------
// Division by a run-time invariant 1 <= d < 2^31 of dividends 0 <= n < 2^31
// with one multiply-high, an add and a shift (Granlund and Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994, sec. 4):
// s = ceil(log2 d), mul = floor(2^32 (2^s - d) / d) + 1, and then
// n / d = (mulhi(n, mul) + n) >> s.  With n < 2^31 the sum stays below 2^32.
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d, mul, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  if (d == 0) return FastDiv{0u, 0u, 0u};   // placeholder for an empty extent; never divided by
  uint32_t s = 0;
  while (((uint64_t)1 << s) < d) ++s;
  const uint64_t mul = ((((uint64_t)1 << s) - d) << 32) / d + 1;
  return FastDiv{d, (uint32_t)mul, s};
}
__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  return (hi + n) >> f.s;
}

// ---------------------------------------------------------------------------
// Window geometry of one block after the clamp, as the kernels see it.
// The permutation it encodes (pages: §3.2, fig. 3; the mmaction2 walk-through
// op order LN -> pad -> roll -> partition):
//   padded grid (Tp, Hp, Wp) = sizes rounded up to the window, zeros appended
//   at the end; the padded grid is rolled by -shift, so rolled position r
//   holds padded coordinate (r + s) mod n; windows (b, wt, wh, ww) and slots
//   (pt, ph, pw) are row-major.
// ---------------------------------------------------------------------------
struct WinGeo {
  int T, H, W;        // real token grid
  int Tp, Hp, Wp;     // padded grid
  int P, Mh, Mw;      // effective window
  int st, sh, sw;     // effective shift
  int nwh, nww;       // windows along H and W (nwt = Tp / P)
  int N;              // tokens per window
  int nws;            // windows per clip
  int pad_visible;    // pads keep their positional label
  int slot_perm;      // window rows in attention slot order (see slot_to_natural)
  // divisors of the slot <-> token maps (set by geo_divisors)
  FastDiv fN, fnws, fwpl, fnww, fmhw, fMw;
  FastDiv fT, fH, fW, fP, fMh;
};

inline void geo_divisors(WinGeo& g) {
  g.fN = make_fastdiv((uint32_t)g.N);
  g.fnws = make_fastdiv((uint32_t)g.nws);
  g.fwpl = make_fastdiv((uint32_t)(g.nwh * g.nww));
  g.fnww = make_fastdiv((uint32_t)g.nww);
  g.fmhw = make_fastdiv((uint32_t)(g.Mh * g.Mw));
  g.fMw = make_fastdiv((uint32_t)g.Mw);
  g.fT = make_fastdiv((uint32_t)g.T);
  g.fH = make_fastdiv((uint32_t)g.H);
  g.fW = make_fastdiv((uint32_t)g.W);
  g.fP = make_fastdiv((uint32_t)g.P);
  g.fMh = make_fastdiv((uint32_t)g.Mh);
}

// Order of the rows of one window inside the block's buffers.  Natural order
// is (pt, ph, pw) row-major.  The MFMA attention path (P % 4 == 0) stores
// slot k = 4 m + i for the token (pt = 4 a + i, ph, pw) with m = (a, ph, pw)
// row-major: four consecutive slots differ only in their temporal coordinate,
// so their relative-position rows are r, r + R, r + 2R, r + 3R.
__host__ __device__ inline int slot_to_natural(const WinGeo& g, int k) {
  if (!g.slot_perm) return k;
  const int m = k >> 2, i = k & 3;
  const int mhw = g.Mh * g.Mw;
  const int a = (int)fdiv((uint32_t)m, g.fmhw);
  return (4 * a + i) * mhw + (m - a * mhw);
}

// Region label of one axis (rolled position r, padded length n, window w,
// shift s): slices [0, n-w), [n-w, n-s), [n-s, n) of the rolled grid.
__host__ __device__ inline int axis_label(int r, int n, int w, int s) {
  return s == 0 ? 0 : (r < n - w ? 0 : (r < n - s ? 1 : 2));
}

constexpr int kPadLabel = 255;

// Source token (flat b,t,h,w) of window slot (w, n), or -1 for a pad slot;
// `label` receives the slot's region label.
// 32-bit index math: the plan rejects grids with 2^31 or more window slots.
__host__ __device__ inline int64_t slot_source(const WinGeo& g, int w, int slot, int& label) {
  const int n = slot_to_natural(g, slot);
  const int b = (int)fdiv((uint32_t)w, g.fnws);
  const int wr = w - b * g.nws;
  const int wpl = g.nwh * g.nww;
  const int wt = (int)fdiv((uint32_t)wr, g.fwpl);
  const int rem = wr - wt * wpl;
  const int wh = (int)fdiv((uint32_t)rem, g.fnww);
  const int ww = rem - wh * g.nww;
  const int mhw = g.Mh * g.Mw;
  const int pt = (int)fdiv((uint32_t)n, g.fmhw);
  const int r2 = n - pt * mhw;
  const int ph = (int)fdiv((uint32_t)r2, g.fMw);
  const int pw = r2 - ph * g.Mw;
  const int rt = wt * g.P + pt, rh = wh * g.Mh + ph, rw = ww * g.Mw + pw;
  int ot = rt + g.st; if (ot >= g.Tp) ot -= g.Tp;
  int oh = rh + g.sh; if (oh >= g.Hp) oh -= g.Hp;
  int ow = rw + g.sw; if (ow >= g.Wp) ow -= g.Wp;
  const bool pad = ot >= g.T || oh >= g.H || ow >= g.W;
  const int lab = 9 * axis_label(rt, g.Tp, g.P, g.st) + 3 * axis_label(rh, g.Hp, g.Mh, g.sh) +
                  axis_label(rw, g.Wp, g.Mw, g.sw);
  label = (pad && !g.pad_visible) ? kPadLabel : lab;
  return pad ? (int64_t)-1 : (((int64_t)b * g.T + ot) * g.H + oh) * g.W + ow;
}

// Source token of window row m (slot order of the geometry) of the whole
// batch of windows, or -1 for a pad slot.
__host__ __device__ inline int64_t row_source(const WinGeo& g, int m, int& label) {
  const int w = (int)fdiv((uint32_t)m, g.fN);
  return slot_source(g, w, m - w * g.N, label);
}

// Window row (slot order of the geometry) that holds token `tok` (flat
// b,t,h,w): the inverse of row_source on real tokens.  The token sits at the
// rolled position (o - s) mod n of each padded axis.
__host__ __device__ inline int token_row(const WinGeo& g, int tok) {
  const int r1 = (int)fdiv((uint32_t)tok, g.fW), ow = tok - r1 * g.W;
  const int r2 = (int)fdiv((uint32_t)r1, g.fH), oh = r1 - r2 * g.H;
  const int b = (int)fdiv((uint32_t)r2, g.fT), ot = r2 - b * g.T;
  int rt = ot - g.st; if (rt < 0) rt += g.Tp;
  int rh = oh - g.sh; if (rh < 0) rh += g.Hp;
  int rw = ow - g.sw; if (rw < 0) rw += g.Wp;
  const int wt = (int)fdiv((uint32_t)rt, g.fP), pt = rt - wt * g.P;
  const int wh = (int)fdiv((uint32_t)rh, g.fMh), ph = rh - wh * g.Mh;
  const int ww = (int)fdiv((uint32_t)rw, g.fMw), pw = rw - ww * g.Mw;
  const int w = b * g.nws + (wt * g.nwh + wh) * g.nww + ww;
  const int k = g.slot_perm ? 4 * (((pt >> 2) * g.Mh + ph) * g.Mw + pw) + (pt & 3) : (pt * g.Mh + ph) * g.Mw + pw;
  return w * g.N + k;
}

// Rolled-grid label of a slot given the window's rolled origin (rt0, rh0, rw0)
// and in-window coordinates; used by the attention kernels, which already know
// the window origin.
__host__ __device__ inline int slot_label_at(const WinGeo& g, int rt, int rh, int rw) {
  int ot = rt + g.st; if (ot >= g.Tp) ot -= g.Tp;
  int oh = rh + g.sh; if (oh >= g.Hp) oh -= g.Hp;
  int ow = rw + g.sw; if (ow >= g.Wp) ow -= g.Wp;
  const bool pad = ot >= g.T || oh >= g.H || ow >= g.W;
  const int lab = 9 * axis_label(rt, g.Tp, g.P, g.st) + 3 * axis_label(rh, g.Hp, g.Mh, g.sh) +
                  axis_label(rw, g.Wp, g.Mw, g.sw);
  return (pad && !g.pad_visible) ? kPadLabel : lab;
}

// Relative-position table geometry (configured window; eq. 2): the row of a
// pair with offset (dt, dh, dw) = query - key is
//   (dt + P0 - 1) * R + (dh + Mh0 - 1) * Rw + (dw + Mw0 - 1),
// R = (2Mh0-1)(2Mw0-1), Rw = 2Mw0-1.  With f(t,h,w) = t*R + h*Rw + w the row
// is f(query) - f(key) + centre, centre = f(P0-1, Mh0-1, Mw0-1).
struct RelTab {
  int rows;     // (2P0-1) * R
  int R, Rw;
  int centre;
};

// The MFMA attention's prepared form of one head's table column: fp32
// 4-tuples (B[r], B[r + Rp], B[r + 2 Rp], B[r + 3 Rp]) * log2(e), entry
// x = dtr * Rp + rem for the offset from the query base (dtr + i, rem / Rw,
// rem % Rw), i = 0..3; Rp >= R is the temporal stride (4 mod 16 for
// conflict-free LDS reads); the last entry TS4 - 1 is a tuple of -inf.
// Scalar form (scalar = 1, windows of more than 512 tokens, whose 4-tuple
// table would not fit in LDS beside one window's K and V^T): the plain fp32
// column S[y] = B(y) * log2(e) for y < TD * Rp (offset y / Rp, y % Rp as
// above), then 3 Rp + 1 entries of -inf; the 4-tuple at y is read as
// S[y], S[y + Rp], S[y + 2 Rp], S[y + 3 Rp], the -inf one at y = TD * Rp.
// TS4 counts 16-byte entries per head in either form (scalar: entry x holds
// S[4x .. 4x + 3]).
struct Tab4Geo {
  int TD, TH, R, Rw, Rp, TS4, heads, scalar;
  FastDiv fdRp, fdRw;
};

#if defined(__HIPCC__)
// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
__device__ __forceinline__ float bflo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bfhi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// round-to-nearest-even float -> bf16 pair (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t f2bf(float a) {
  __bf16 h = (__bf16)a;
  return __builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------------------
// kernel arguments
// ---------------------------------------------------------------------------
// Byte size of a kernel's explicit arguments T... in its argument segment
// (each at its own alignment, the end rounded to 8); the hidden arguments
// (the grid's block counts first) follow.
template <class... T>
constexpr int kArgBytes() {
  int off = 0;
  ((off = (off + (int)alignof(T) - 1) / (int)alignof(T) * (int)alignof(T) + (int)sizeof(T)), ...);
  return (off + 7) / 8 * 8;
}

// Every 64-byte line of the first BYTES bytes of the argument segment
// requested from the scalar cache at once, before any is used: at kernel start
// each line is a miss to memory, and the compiler otherwise issues the loads
// of a large argument block a few at a time as the code needs them, one
// round trip after another.  The loads and their wait are one asm statement,
// so the destination register is never reused while a load is in flight.
template <int BYTES>
__device__ __forceinline__ void kernarg_warm() {
  constexpr int L = (BYTES + 63) / 64;
  static_assert(L >= 1 && L <= 16, "argument block of 1 to 16 lines");
  const auto p = __builtin_amdgcn_kernarg_segment_ptr();
  uint32_t d;
  if constexpr (L == 1)
    asm volatile("s_load_dword %0, %1, 0x0\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 2)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 3)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 4)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 5)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 6)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 7)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 8)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 9)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 10)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 11)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t""s_load_dword %0, %1, 0x280\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 12)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t""s_load_dword %0, %1, 0x280\n\t""s_load_dword %0, %1, 0x2c0\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 13)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t""s_load_dword %0, %1, 0x280\n\t""s_load_dword %0, %1, 0x2c0\n\t""s_load_dword %0, %1, 0x300\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 14)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t""s_load_dword %0, %1, 0x280\n\t""s_load_dword %0, %1, 0x2c0\n\t""s_load_dword %0, %1, 0x300\n\t""s_load_dword %0, %1, 0x340\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 15)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t""s_load_dword %0, %1, 0x280\n\t""s_load_dword %0, %1, 0x2c0\n\t""s_load_dword %0, %1, 0x300\n\t""s_load_dword %0, %1, 0x340\n\t""s_load_dword %0, %1, 0x380\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  if constexpr (L == 16)
    asm volatile("s_load_dword %0, %1, 0x0\n\t""s_load_dword %0, %1, 0x40\n\t""s_load_dword %0, %1, 0x80\n\t""s_load_dword %0, %1, 0xc0\n\t""s_load_dword %0, %1, 0x100\n\t""s_load_dword %0, %1, 0x140\n\t""s_load_dword %0, %1, 0x180\n\t""s_load_dword %0, %1, 0x1c0\n\t""s_load_dword %0, %1, 0x200\n\t""s_load_dword %0, %1, 0x240\n\t""s_load_dword %0, %1, 0x280\n\t""s_load_dword %0, %1, 0x2c0\n\t""s_load_dword %0, %1, 0x300\n\t""s_load_dword %0, %1, 0x340\n\t""s_load_dword %0, %1, 0x380\n\t""s_load_dword %0, %1, 0x3c0\n\t"
                 "s_waitcnt lgkmcnt(0)" : "=&s"(d) : "s"(p) : "memory");
  (void)d;
}

// kernarg_warm over a kernel's explicit arguments (pass them all, in order).
// The segment ends with them unless the kernel reads a hidden argument (its
// grid or workgroup size): warm_args_grid also takes the line of the first
// hidden ones, which then follow.
template <class... T>
__device__ __forceinline__ void warm_args(const T&...) {
  kernarg_warm<kArgBytes<T...>()>();
}
template <class... T>
__device__ __forceinline__ void warm_args_grid(const T&...) {
  kernarg_warm<kArgBytes<T...>() + 8>();
}

// Sum over the 4 lanes of a token row (lanes l, l^16, l^32, l^48) by lane
// swaps in the VALU (v_permlane16_swap / v_permlane32_swap: with both
// operands equal to v, the two results add up to v[l] + v[l ^ 16], resp.
// v[l ^ 32]); the same sums as two xor-shuffle additions.
__device__ __forceinline__ float row4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// entry x of head h's prepared table, from the (rows, heads) bf16 table T:
// offsets outside the table give 0
__device__ __forceinline__ f32x4_t t4_entry(const bf16_t* __restrict__ T, const Tab4Geo& tg, int h, int x) {
  f32x4_t v = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  if (x < tg.TS4 - 1) {
    const int dtr = (int)fdiv((uint32_t)x, tg.fdRp);
    const int rem = x - dtr * tg.Rp;
    const int dhr = (int)fdiv((uint32_t)rem, tg.fdRw);
    const int dwr = rem - dhr * tg.Rw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dt = dtr + i;
      const bool ok = rem < tg.R && dt < tg.TD;
      const int row = ok ? (tg.TD - 1 - dt) * tg.R + (tg.TH - 1 - dhr) * tg.Rw + (tg.Rw - 1 - dwr) : 0;
      v[i] = ok ? bf2f(T[(size_t)row * tg.heads + h]) * 1.4426950408889634f : 0.f;
    }
  }
  return v;
}

// entry x of head h's prepared table in the scalar form: S[4x .. 4x + 3]
__device__ __forceinline__ f32x4_t ts_entry(const bf16_t* __restrict__ T, const Tab4Geo& tg, int h, int x) {
  f32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int y = 4 * x + i;
    float e = -INFINITY;
    if (y < tg.TD * tg.Rp) {
      const int dtr = (int)fdiv((uint32_t)y, tg.fdRp);
      const int rem = y - dtr * tg.Rp;
      const int dhr = (int)fdiv((uint32_t)rem, tg.fdRw);
      const int dwr = rem - dhr * tg.Rw;
      const bool ok = rem < tg.R;
      const int row = ok ? (tg.TD - 1 - dtr) * tg.R + (tg.TH - 1 - dhr) * tg.Rw + (tg.Rw - 1 - dwr) : 0;
      e = ok ? bf2f(T[(size_t)row * tg.heads + h]) * 1.4426950408889634f : 0.f;
    }
    v[i] = e;
  }
  return v;
}

__device__ __forceinline__ f32x4_t tab_entry(const bf16_t* __restrict__ T, const Tab4Geo& tg, int h, int x) {
  return tg.scalar ? ts_entry(T, tg, h, x) : t4_entry(T, tg, h, x);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf2f(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
};

// four consecutive elements (16-byte aligned for float, 8-byte for bf16)
__device__ __forceinline__ void load4(const float* p, int64_t i, float v[4]) {
  const float4 t = *reinterpret_cast<const float4*>(p + i);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, int64_t i, float v[4]) {
  const u32x2_t t = *reinterpret_cast<const u32x2_t*>(p + i);
  v[0] = bflo(t[0]); v[1] = bfhi(t[0]); v[2] = bflo(t[1]); v[3] = bfhi(t[1]);
}
__device__ __forceinline__ void store4(float* p, int64_t i, const float v[4]) {
  *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, int64_t i, const float v[4]) {
  u32x2_t t;
  t[0] = pack_bf16x2(v[0], v[1]);
  t[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2_t*>(p + i) = t;
}
#endif

}  // namespace vswin
