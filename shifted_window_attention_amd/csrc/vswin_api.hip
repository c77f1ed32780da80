// C ABI of libvswin.so: argument validation, the block plan (clamp, padding,
// window counts, workspace layout) and the launch sequence on one stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <map>
#include <mutex>
#include <new>
#include <unordered_map>
#include <utility>

#include "vswin_kernels.h"

namespace vswin {

int device_cu_count() {
  static std::mutex mu;
  static std::unordered_map<int, int> counts;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = counts.find(dev);
  if (it != counts.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  counts[dev] = n;
  return n;
}

hipError_t ensure_dynamic_lds(const void* kern, size_t bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(kern, dev);
  auto it = done.find(key);
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[key] = bytes;
  return e;
}

}  // namespace vswin

using namespace vswin;

namespace {

thread_local char g_err[512] = "";

vswin_status fail(vswin_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
vswin_status fail(vswin_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

vswin_status hip_fail(hipError_t e, const char* where) {
  return fail(VSWIN_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Test hook: VSWIN_FAULT=launch makes every compute call fail as if a launch
// had failed, after validation and before anything is enqueued.
bool fault_injected() {
  const char* f = getenv("VSWIN_FAULT");
  return f && strcmp(f, "launch") == 0;
}

// VSWIN_FUSED=1 runs LN1 + gather + qkv + attention as one kernel where it
// applies (q, k and v stay on chip); by default they are two launches (q, k,
// V^T through the workspace), which measured faster at the Swin-T stage-1
// shape: the one kernel recomputes the keys of windows that two workgroups
// share and builds the bias table in every workgroup.  Both give the same bits.
bool fused_enabled() {
  const char* f = getenv("VSWIN_FUSED");
  return f && strcmp(f, "1") == 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t elem_size(vswin_dtype d) { return d == VSWIN_BF16 ? 2 : 4; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
  WinGeo geo;
  RelTab rel;
  int B, C, heads, d, hid;
  int64_t L, Lp, nW;
  int N;
  bool use_mask;
  bool fast;
  vswin_dtype dt;
  // workspace offsets (bytes)
  size_t off_xw, off_q, off_k, off_v, off_tab, off_zh, off_h, ws_block, ws_msa, ws_attn;
};

AttnArgs attn_args(const Plan& p, const void* q, const void* k, const void* v, const void* table, void* o,
                   uint32_t flags, char* scratch = nullptr) {
  AttnArgs a{};
  a.tab4 = scratch;
  a.q = q; a.k = k; a.v = v; a.table = table; a.o = o;
  a.nW = p.nW; a.heads = p.heads; a.d = p.d; a.C = p.C; a.N = p.N;
  a.rel = p.rel; a.geo = p.geo;
  a.use_mask = p.use_mask ? 1 : 0;
  a.mask_m100 = (flags & VSWIN_F_MASK_M100) ? 1 : 0;
  return a;
}

vswin_status make_plan(const vswin_desc* d, Plan& p, bool compute = true) {
  if (!d) return fail(VSWIN_ERR_INVALID_ARG, "desc is NULL");
  if (d->dtype != VSWIN_FP32 && d->dtype != VSWIN_BF16)
    return fail(VSWIN_ERR_INVALID_ARG, "unknown dtype %d", (int)d->dtype);
  if (d->B < 0 || d->T < 1 || d->H < 1 || d->W < 1 || d->C < 1)
    return fail(VSWIN_ERR_INVALID_ARG, "bad token shape B=%d T=%d H=%d W=%d C=%d", d->B, d->T, d->H, d->W, d->C);
  if (d->heads < 1 || d->C % d->heads != 0)
    return fail(VSWIN_ERR_INVALID_ARG, "C=%d is not a multiple of heads=%d", d->C, d->heads);
  if (d->mlp_hidden < 1) return fail(VSWIN_ERR_INVALID_ARG, "mlp_hidden=%d", d->mlp_hidden);
  if (!(d->ln_eps > 0.f)) return fail(VSWIN_ERR_INVALID_ARG, "ln_eps must be > 0");
  if (d->flags & ~(uint32_t)(VSWIN_F_PAD_VISIBLE | VSWIN_F_CLAMP_STRICT | VSWIN_F_MASK_M100 | VSWIN_F_TABLES_READY))
    return fail(VSWIN_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags);
  const int size[3] = {d->T, d->H, d->W};
  int win[3], sh[3], pad[3];
  for (int i = 0; i < 3; ++i) {
    if (d->window[i] < 1) return fail(VSWIN_ERR_INVALID_ARG, "window[%d]=%d", i, d->window[i]);
    if (d->shift[i] < 0 || d->shift[i] >= d->window[i])
      return fail(VSWIN_ERR_INVALID_ARG, "shift[%d]=%d not in [0, window)", i, d->shift[i]);
    const bool small = (d->flags & VSWIN_F_CLAMP_STRICT) ? size[i] < d->window[i] : size[i] <= d->window[i];
    win[i] = small ? size[i] : d->window[i];
    sh[i] = small ? 0 : d->shift[i];
    pad[i] = (size[i] + win[i] - 1) / win[i] * win[i];
  }
  const int dh = d->C / d->heads;
  const int N = win[0] * win[1] * win[2];
  if (!compute) {
    // permutation-only entry points: 4-channel vectors
    if (d->C % 4) return fail(VSWIN_ERR_UNSUPPORTED, "C=%d not a multiple of 4", d->C);
  } else if (dh > 64) {
    return fail(VSWIN_ERR_UNSUPPORTED, "head_dim %d > 64", dh);
  } else if (dh % 4 != 0) {
    return fail(VSWIN_ERR_UNSUPPORTED, "head_dim %d not a multiple of 4", dh);
  } else if (N > 2048) {
    return fail(VSWIN_ERR_UNSUPPORTED, "window of %d tokens > 2048", N);
  } else if (d->dtype == VSWIN_BF16) {
    if (d->C % 32 || d->mlp_hidden % 32)
      return fail(VSWIN_ERR_UNSUPPORTED, "bf16 path needs C and mlp_hidden multiples of 32 (C=%d hidden=%d)",
                  d->C, d->mlp_hidden);
  } else if (d->C % 4 || d->mlp_hidden % 4) {
    return fail(VSWIN_ERR_UNSUPPORTED, "C and mlp_hidden must be multiples of 4");
  }
  WinGeo& g = p.geo;
  g.T = d->T; g.H = d->H; g.W = d->W;
  g.Tp = pad[0]; g.Hp = pad[1]; g.Wp = pad[2];
  g.P = win[0]; g.Mh = win[1]; g.Mw = win[2];
  g.st = sh[0]; g.sh = sh[1]; g.sw = sh[2];
  g.nwh = pad[1] / win[1]; g.nww = pad[2] / win[2];
  g.N = N;
  g.nws = (pad[0] / win[0]) * g.nwh * g.nww;
  g.pad_visible = (d->flags & VSWIN_F_PAD_VISIBLE) ? 1 : 0;
  geo_divisors(g);
  const int R = (2 * d->window[1] - 1) * (2 * d->window[2] - 1);
  p.rel.R = R;
  p.rel.Rw = 2 * d->window[2] - 1;
  p.rel.rows = (2 * d->window[0] - 1) * R;
  p.rel.centre = (d->window[0] - 1) * R + (d->window[1] - 1) * p.rel.Rw + (d->window[2] - 1);
  p.B = d->B; p.C = d->C; p.heads = d->heads; p.d = dh; p.hid = d->mlp_hidden; p.dt = d->dtype;
  p.N = N;
  p.nW = (int64_t)d->B * g.nws;
  p.Lp = p.nW * N;
  p.L = (int64_t)d->B * d->T * d->H * d->W;
  if (p.Lp >= ((int64_t)1 << 31) - 4096 || p.L * p.C >= ((int64_t)1 << 40))
    return fail(VSWIN_ERR_UNSUPPORTED, "grid of %lld window slots is too large", (long long)p.Lp);
  const bool shifted = sh[0] || sh[1] || sh[2];
  const bool has_pad = pad[0] != d->T || pad[1] != d->H || pad[2] != d->W;
  p.use_mask = shifted || (has_pad && !g.pad_visible);
  p.fast = attention_mfma_supported(p.dt, attn_args(p, nullptr, nullptr, nullptr, nullptr, nullptr, d->flags));
  g.slot_perm = p.fast ? 1 : 0;     // window rows in the MFMA kernel's slot order
  const size_t es = elem_size(d->dtype);
  const size_t act = align256((size_t)p.Lp * p.C * es);
  p.ws_attn = p.fast ? attention_workspace_bytes(p.rel, p.heads, p.N) : 0;
  p.off_xw = 0;
  p.off_q = act;
  p.off_k = 2 * act;
  p.off_v = 3 * act;
  p.off_tab = 4 * act;
  p.ws_msa = 4 * act + p.ws_attn;
  p.off_zh = p.ws_msa;
  p.off_h = p.off_zh + align256((size_t)p.L * p.C * 4);
  p.ws_block = p.off_h + align256((size_t)p.L * p.hid * es);
  return VSWIN_OK;
}

vswin_status check_ptr(const void* ptr, const char* name, bool nullable = false) {
  if (!ptr) return nullable ? VSWIN_OK : fail(VSWIN_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(VSWIN_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return VSWIN_OK;
}

#define CHECK(expr)                     \
  do {                                  \
    const vswin_status s_ = (expr);     \
    if (s_ != VSWIN_OK) return s_;      \
  } while (0)

#define HIPCHECK(expr, where)                          \
  do {                                                 \
    const hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, where);  \
  } while (0)

vswin_status check_msa_weights(const vswin_block_weights* w) {
  if (!w) return fail(VSWIN_ERR_INVALID_ARG, "weights is NULL");
  CHECK(check_ptr(w->qkv_w, "qkv_w"));
  CHECK(check_ptr(w->qkv_b, "qkv_b", true));
  CHECK(check_ptr(w->proj_w, "proj_w"));
  CHECK(check_ptr(w->proj_b, "proj_b", true));
  CHECK(check_ptr(w->rpb_table, "rpb_table"));
  return VSWIN_OK;
}

// Can the block run as qkv (gathering LN1) -> attention -> proj_mlp, the
// projection fused into the MLP kernel?
bool block_proj_fused(const Plan& p) {
  return p.fast && gemm_can_gather(p.dt, p.C) && winproj_supported(p.dt, p.C, p.d, p.N, 1) &&
         proj_mlp_supported(p.dt, p.C, p.hid);
}

// qkv -> attention -> proj (+ scatter).  `ga` (nullable) makes the qkv
// projection gather (and normalise) its rows itself; otherwise `xw` holds the
// gathered window rows.  With `no_proj` (gathering fast path only) it stops
// after the attention, whose output rows are left in `xw`.
vswin_status run_msa(const Plan& p, const vswin_desc* d, const vswin_block_weights* w, char* ws,
                     const void* residual, void* out, bool to_zh, hipStream_t st, const GatherA* ga = nullptr,
                     bool no_proj = false, void* attn_out = nullptr) {
  // the attention output rows (with `no_proj` and `ga`, `attn_out` may take them instead)
  void* xw = attn_out ? attn_out : ws + p.off_xw;
  void* q = ws + p.off_q;
  void* k = ws + p.off_k;
  void* v = ws + p.off_v;
  const int vt = p.fast ? 1 : 0;
  if (ga && fused_enabled()) {
    // LN1 + gather + qkv + attention in one kernel: q, k, v stay on chip
    FusedArgs fa{};
    fa.a = attn_args(p, nullptr, nullptr, nullptr, w->rpb_table, xw, d->flags);
    if (attention_fused_supported(p.dt, fa.a)) {
      fa.x = ga->x;
      fa.ln_g = ga->g;
      fa.ln_b = ga->b;
      fa.eps = ga->eps;
      fa.ln = ga->ln;
      fa.w = w->qkv_w;
      fa.bias = w->qkv_b;
      HIPCHECK(attention_fused(fa, st), "fused qkv + attention");
      if (no_proj) return VSWIN_OK;
      HIPCHECK(out_proj(xw, w->proj_w, w->proj_b, to_zh ? residual : nullptr, out, p.Lp, p.C, p.geo, st),
               "output projection");
      return VSWIN_OK;
    }
  }
  if (ga && winproj_supported(p.dt, p.C, p.d, p.N, vt)) {
    // the MFMA attention takes q pre-multiplied by log2(e) / sqrt(d)
    const float qscale = p.fast ? 1.4426950408889634f / sqrtf((float)p.d) : 1.0f;
    // the MFMA attention's prepared bias tables are written by the qkv launch
    HIPCHECK(qkv_proj(ga->x, ga->g, ga->b, ga->eps, ga->ln, w->qkv_w, w->qkv_b, q, k, v, vt, qscale, p.Lp, p.C,
                      p.heads, p.d, p.geo, p.fast ? w->rpb_table : nullptr, p.fast ? ws + p.off_tab : nullptr,
                      tab4_geo(p.rel, p.heads, p.N), st),
             "qkv projection");
    AttnArgs a = attn_args(p, q, k, v, w->rpb_table, xw, d->flags, ws + p.off_tab);
    a.q_scaled = p.fast ? 1 : 0;
    a.tab_ready = p.fast ? 1 : 0;
    if (p.fast) HIPCHECK(attention_mfma(a, st), "attention (mfma)");
    else HIPCHECK(attention_generic(p.dt, a, st), "attention (generic)");
    if (no_proj) return VSWIN_OK;
    HIPCHECK(out_proj(xw, w->proj_w, w->proj_b, to_zh ? residual : nullptr, out, p.Lp, p.C, p.geo, st),
             "output projection");
    return VSWIN_OK;
  }
  if (no_proj) return fail(VSWIN_ERR_UNSUPPORTED, "internal: fused projection path not available");
  EpiArgs e{};
  e.kind = Epi::kQKV;
  e.bias = w->qkv_b;
  e.out = q; e.out2 = k; e.out3 = v;
  e.C = p.C; e.heads = p.heads; e.d = p.d; e.N = p.N; e.geo = p.geo;
  e.vt = p.fast ? 1 : 0;
  HIPCHECK(gemm(p.dt, xw, w->qkv_w, p.Lp, 3 * p.C, p.C, e, st, ga), "qkv gemm");
  const AttnArgs a = attn_args(p, q, k, v, w->rpb_table, xw, d->flags, ws + p.off_tab);
  if (p.fast) HIPCHECK(attention_mfma(a, st), "attention (mfma)");
  else HIPCHECK(attention_generic(p.dt, a, st), "attention (generic)");
  EpiArgs e2{};
  e2.kind = to_zh ? Epi::kProjRes : Epi::kProjOut;
  e2.bias = w->proj_b;
  e2.out = out;
  e2.res = residual;
  e2.C = p.C; e2.heads = p.heads; e2.d = p.d; e2.N = p.N; e2.geo = p.geo;
  HIPCHECK(gemm(p.dt, xw, w->proj_w, p.Lp, p.C, p.C, e2, st), "proj gemm");
  return VSWIN_OK;
}

// Workspace of the backward entry points (bytes, 256-aligned regions).
struct BwdWs {
  size_t n1w, q, k, v, o, tab, lse;           // forward recompute (window rows)
  size_t zh, n2, a1, h, dh, dzh;              // block only
  size_t dyw, dout, dqkv, dn1w, dn1, attn;
  size_t part;                                 // block only
  size_t pproj, pqkv, pfc2, pfc1, pln2;        // weight-gradient partials (fc, ln2: block only)
  size_t wTqkv, wTproj, wTfc2, wTfc1;          // transposed weights (fc: block only)
  size_t block_bytes, msa_bytes;
};

bool bwd_supported(const Plan& p, const vswin_desc* d) {
  if (p.dt != VSWIN_BF16 || !p.fast || p.d != 32 || p.C > 768 || p.hid % 32) return false;
  return attention_bwd_supported(p.dt, attn_args(p, nullptr, nullptr, nullptr, nullptr, nullptr, d->flags));
}

BwdWs bwd_layout(const Plan& p, const vswin_desc* d) {
  BwdWs w{};
  const size_t act = align256((size_t)p.Lp * p.C * 2);
  const size_t tok = align256((size_t)p.L * p.C * 2), tok32 = align256((size_t)p.L * p.C * 4);
  const size_t hid = align256((size_t)p.L * p.hid * 2);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.n1w = take(act);
  w.q = take(act);
  w.k = take(act);
  w.v = take(act);
  w.o = take(act);
  w.tab = take(p.ws_attn);
  w.lse = take((size_t)p.nW * p.heads * p.N * 4);
  w.dyw = take(act);
  w.dout = take(act);
  w.dqkv = take(3 * act);
  w.dn1w = take(act);
  w.dn1 = take(tok);
  w.wTqkv = take((size_t)3 * p.C * p.C * 2);
  w.wTproj = take((size_t)p.C * p.C * 2);
  w.pproj = take(wgrad_part_bytes(p.Lp, p.C, p.C));
  w.pqkv = take(wgrad_part_bytes(p.Lp, 3 * p.C, p.C));
  w.attn = take(attention_bwd_workspace_bytes(attn_args(p, nullptr, nullptr, nullptr, nullptr, nullptr, d->flags)));
  w.msa_bytes = off;
  w.zh = take(tok32);
  w.n2 = take(tok);
  w.a1 = take(hid);
  w.h = take(hid);
  w.dh = take(hid);
  w.dzh = take(tok32);
  w.wTfc2 = take((size_t)p.hid * p.C * 2);
  w.wTfc1 = take((size_t)p.hid * p.C * 2);
  w.pfc2 = take(wgrad_part_bytes(p.L, p.C, p.hid));
  w.pfc1 = take(wgrad_part_bytes(p.L, p.hid, p.C));
  w.part = take(ln_bwd_part_bytes(p.L, p.C));   // LN1's dγ/dβ partials
  w.pln2 = take(ln_bwd_part_bytes(p.L, p.C));
  w.block_bytes = off;
  return w;
}

// Argument checks of the block forward on a planned descriptor (before
// anything is enqueued).
vswin_status block_fwd_check(const void* x, const vswin_block_weights* w, void* y) {
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(y, "y"));
  if (x == y) return fail(VSWIN_ERR_INVALID_ARG, "x and y must not alias");
  CHECK(check_msa_weights(w));
  CHECK(check_ptr(w->ln1_g, "ln1_g"));
  CHECK(check_ptr(w->ln1_b, "ln1_b"));
  CHECK(check_ptr(w->ln2_g, "ln2_g"));
  CHECK(check_ptr(w->ln2_b, "ln2_b"));
  CHECK(check_ptr(w->fc1_w, "fc1_w"));
  CHECK(check_ptr(w->fc1_b, "fc1_b", true));
  CHECK(check_ptr(w->fc2_w, "fc2_w"));
  CHECK(check_ptr(w->fc2_b, "fc2_b", true));
  return VSWIN_OK;
}

// Can LN1 + gather + qkv + attention run without a separate gather kernel
// (the rows the qkv projection stages are normalised and gathered there)?
bool qkv_attention_supported(const Plan& p) {
  return p.fast && gemm_can_gather(p.dt, p.C) && winproj_supported(p.dt, p.C, p.d, p.N, 1);
}

// Workspace bytes the block's launch sequence touches: the window-MSA regions
// when the projection is fused into the MLP kernel, else the whole block
// layout.
size_t block_ws_needed(const Plan& p) { return block_proj_fused(p) ? p.ws_msa : p.ws_block; }

// One block on a workspace the caller checked (`ws`, at least
// block_ws_needed(p) bytes): the launch sequence shared by vswin_block_fwd
// and vswin_block_fwd_noalloc.
vswin_status block_fwd_run(const Plan& p, const vswin_desc* desc, const void* x, const vswin_block_weights* w,
                           void* y, char* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  // LN1 + pad + roll + partition: fused into the qkv projection when it can
  // stage whole rows, else a separate gather kernel
  if (block_proj_fused(p)) {
    // qkv -> attention -> (proj + residual + LN2 + MLP + residual) in one kernel
    const GatherA ga{x, w->ln1_g, w->ln1_b, desc->ln_eps, 1, p.geo};
    CHECK(run_msa(p, desc, w, ws, x, nullptr, true, st, &ga, true));
    HIPCHECK(proj_mlp(ws + p.off_xw, x, w->proj_w, w->proj_b, w->ln2_g, w->ln2_b, w->fc1_w, w->fc1_b, w->fc2_w,
                      w->fc2_b, y, p.L, p.C, desc->ln_eps, p.geo, st),
             "projection + mlp");
    return VSWIN_OK;
  }
  if (gemm_can_gather(p.dt, p.C)) {
    const GatherA ga{x, w->ln1_g, w->ln1_b, desc->ln_eps, 1, p.geo};
    CHECK(run_msa(p, desc, w, ws, x, ws + p.off_zh, true, st, &ga));
  } else {
    HIPCHECK(ln_gather(p.dt, x, w->ln1_g, w->ln1_b, ws + p.off_xw, p.Lp, p.C, desc->ln_eps, p.geo, 1, st),
             "ln1 gather");
    CHECK(run_msa(p, desc, w, ws, x, ws + p.off_zh, true, st));
  }
  if (mlp_fused_supported(p.dt, p.C, p.hid)) {
    HIPCHECK(mlp_fused((const float*)(ws + p.off_zh), w->ln2_g, w->ln2_b, w->fc1_w, w->fc1_b, w->fc2_w, w->fc2_b,
                       y, p.L, p.C, desc->ln_eps, st),
             "fused mlp");
    return VSWIN_OK;
  }
  // LN2 -> xw region (free after proj)
  HIPCHECK(ln_rows(VSWIN_FP32, p.dt, ws + p.off_zh, w->ln2_g, w->ln2_b, ws + p.off_xw, p.L, p.C, desc->ln_eps,
                   st),
           "ln2");
  EpiArgs e{};
  e.kind = Epi::kGelu;
  e.bias = w->fc1_b;
  e.out = ws + p.off_h;
  e.ld_out = p.hid;
  HIPCHECK(gemm(p.dt, ws + p.off_xw, w->fc1_w, p.L, p.hid, p.C, e, st), "fc1 gemm");
  EpiArgs e2{};
  e2.kind = Epi::kRes;
  e2.bias = w->fc2_b;
  e2.out = y;
  e2.res = ws + p.off_zh;
  e2.ld_out = p.C;
  HIPCHECK(gemm(p.dt, ws + p.off_h, w->fc2_w, p.L, p.C, p.hid, e2, st), "fc2 gemm");
  return VSWIN_OK;
}

// Scratch memory of vswin_block_fwd_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never uses its name
// as an address (on the host it is a stand-in); the device address comes from
// hipGetSymbolAddress once per device, with that device current, and is kept
// per device.
static __device__ __align__(256) unsigned char scratch[VSWIN_NOALLOC_SCRATCH_BYTES];

vswin_status noalloc_scratch(char** out) {
  static std::mutex mu;
  static std::unordered_map<int, char*> ptrs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "noalloc: hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(VSWIN_ERR_HIP, "noalloc: scratch address %p is unusable", ptr);
    it = ptrs.emplace(dev, static_cast<char*>(ptr)).first;
  }
  *out = it->second;
  return VSWIN_OK;
}

}  // namespace

extern "C" {

const char* vswin_last_error(void) { return g_err; }
int32_t vswin_abi_version(void) { return VSWIN_ABI_VERSION; }

const char* vswin_status_string(vswin_status s) {
  switch (s) {
    case VSWIN_OK: return "ok";
    case VSWIN_ERR_INVALID_ARG: return "invalid argument";
    case VSWIN_ERR_UNSUPPORTED: return "unsupported";
    case VSWIN_ERR_WORKSPACE: return "workspace too small";
    case VSWIN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

vswin_status vswin_plan_query(const vswin_desc* desc, vswin_plan* plan) {
  if (!plan) return fail(VSWIN_ERR_INVALID_ARG, "plan is NULL");
  Plan p{};
  CHECK(make_plan(desc, p, false));
  plan->eff_window[0] = p.geo.P; plan->eff_window[1] = p.geo.Mh; plan->eff_window[2] = p.geo.Mw;
  plan->eff_shift[0] = p.geo.st; plan->eff_shift[1] = p.geo.sh; plan->eff_shift[2] = p.geo.sw;
  plan->padded[0] = p.geo.Tp; plan->padded[1] = p.geo.Hp; plan->padded[2] = p.geo.Wp;
  plan->tokens_per_window = p.N;
  plan->num_windows = p.nW;
  plan->tokens = p.L;
  plan->masked = p.use_mask ? 1 : 0;
  plan->fast_attention = p.fast ? 1 : 0;
  plan->workspace_bytes = p.ws_block;
  plan->msa_workspace_bytes = p.ws_msa;
  plan->attention_workspace_bytes = p.ws_attn;
  // geometry is filled in; now the constraints of the compute entry points
  Plan q{};
  return make_plan(desc, q, true);
}

vswin_status vswin_block_fwd(const vswin_desc* desc, const void* x, const vswin_block_weights* w, void* y,
                             void* workspace, size_t workspace_bytes, void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.L == 0) return VSWIN_OK;   // empty batch: nothing to read or write
  CHECK(block_fwd_check(x, w, y));
  if (!workspace || !aligned(workspace, 256))
    return fail(VSWIN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < p.ws_block)
    return fail(VSWIN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, p.ws_block);
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  return block_fwd_run(p, desc, x, w, y, (char*)workspace, stream);
}

vswin_status vswin_block_fwd_noalloc(const vswin_desc* desc, const void* x, const vswin_block_weights* w, void* y,
                                     void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.L == 0) return VSWIN_OK;
  CHECK(block_fwd_check(x, w, y));
  const size_t need = block_ws_needed(p);
  if (need > (size_t)VSWIN_NOALLOC_SCRATCH_BYTES)
    return fail(VSWIN_ERR_WORKSPACE, "this block needs %zu bytes of scratch; the static buffer holds %zu", need,
                (size_t)VSWIN_NOALLOC_SCRATCH_BYTES);
  char* ws = nullptr;
  CHECK(noalloc_scratch(&ws));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  return block_fwd_run(p, desc, x, w, y, ws, stream);
}

vswin_status vswin_window_msa_fwd(const vswin_desc* desc, const void* x_norm, const vswin_block_weights* w,
                                  void* y, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.L == 0) return VSWIN_OK;
  CHECK(check_ptr(x_norm, "x_norm"));
  CHECK(check_ptr(y, "y"));
  if (x_norm == y) return fail(VSWIN_ERR_INVALID_ARG, "x_norm and y must not alias");
  CHECK(check_msa_weights(w));
  if (p.L == 0) return VSWIN_OK;
  if (!workspace || !aligned(workspace, 256))
    return fail(VSWIN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < p.ws_msa)
    return fail(VSWIN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, p.ws_msa);
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (gemm_can_gather(p.dt, p.C)) {
    const GatherA ga{x_norm, nullptr, nullptr, desc->ln_eps, 0, p.geo};
    return run_msa(p, desc, w, ws, nullptr, y, false, st, &ga);
  }
  HIPCHECK(ln_gather(p.dt, x_norm, nullptr, nullptr, ws + p.off_xw, p.Lp, p.C, desc->ln_eps, p.geo, 0, st),
           "partition");
  return run_msa(p, desc, w, ws, nullptr, y, false, st);
}

vswin_status vswin_qkv_attention_fwd(const vswin_desc* desc, const void* x, const vswin_block_weights* w, void* o,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.L == 0) return VSWIN_OK;
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(o, "o"));
  if (x == o) return fail(VSWIN_ERR_INVALID_ARG, "x and o must not alias");
  CHECK(check_msa_weights(w));
  CHECK(check_ptr(w->ln1_g, "ln1_g"));
  CHECK(check_ptr(w->ln1_b, "ln1_b"));
  if (!qkv_attention_supported(p))
    return fail(VSWIN_ERR_UNSUPPORTED, "qkv + attention needs bf16, head_dim 32, C in {96, 128} and the MFMA "
                                       "attention");
  if (!workspace || !aligned(workspace, 256))
    return fail(VSWIN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < p.ws_msa)
    return fail(VSWIN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, p.ws_msa);
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  const GatherA ga{x, w->ln1_g, w->ln1_b, desc->ln_eps, 1, p.geo};
  return run_msa(p, desc, w, (char*)workspace, x, nullptr, false, (hipStream_t)stream, &ga, true, o);
}

vswin_status vswin_attention_fwd(const vswin_desc* desc, const void* q, const void* k, const void* v,
                                 const void* rpb_table, void* o, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.Lp == 0) return VSWIN_OK;
  if (p.ws_attn && (!workspace || !aligned(workspace, 256) || workspace_bytes < p.ws_attn))
    return fail(VSWIN_ERR_WORKSPACE, "attention needs %zu workspace bytes", p.ws_attn);
  CHECK(check_ptr(q, "q"));
  CHECK(check_ptr(k, "k"));
  CHECK(check_ptr(v, "v"));
  CHECK(check_ptr(rpb_table, "rpb_table"));
  CHECK(check_ptr(o, "o"));
  if (p.Lp == 0) return VSWIN_OK;
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  AttnArgs a = attn_args(p, q, k, v, rpb_table, o, desc->flags, (char*)workspace);
  a.tab_ready = (desc->flags & VSWIN_F_TABLES_READY) ? 1 : 0;
  if (p.fast) HIPCHECK(attention_mfma(a, (hipStream_t)stream), "attention (mfma)");
  else HIPCHECK(attention_generic(p.dt, a, (hipStream_t)stream), "attention (generic)");
  return VSWIN_OK;
}

vswin_status vswin_bwd_workspace_query(const vswin_desc* desc, size_t* block_bytes, size_t* msa_bytes) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (!bwd_supported(p, desc))
    return fail(VSWIN_ERR_UNSUPPORTED, "backward needs bf16, head_dim 32, C <= 768 and the MFMA attention (at most "
                                       "1024 tokens per window)");
  const BwdWs w = bwd_layout(p, desc);
  if (block_bytes) *block_bytes = w.block_bytes;
  if (msa_bytes) *msa_bytes = w.msa_bytes;
  return VSWIN_OK;
}

namespace {

// Shared part of the two backward entry points: forward recompute of the
// attention branch from the window rows in w.n1w, then, given the window-row
// gradient of the branch output in w.dyw, the gradients of proj, attention
// (table), qkv and of the window rows (w.dn1w) scattered to token rows dxo.
// The proj and qkv weight gradients are left as partials, their reductions
// appended to `wj` (the caller launches all of them at once).
vswin_status msa_bwd_core(const Plan& p, const vswin_desc* d, const vswin_block_weights* wt,
                          const vswin_block_grads* g, char* ws, const BwdWs& w, void* dxo, hipStream_t st,
                          bool with_mlp, const GatherA& ga, WgradJobs& wj,
                          const std::function<vswin_status()>& mid) {
  const int C = p.C;
  // every weight the input-gradient GEMMs need transposed, in one launch
  // (the block's MLP weights too)
  {
    TransposeJobs tj{};
    tj.job[tj.n++] = TransposeJob{wt->proj_w, ws + w.wTproj, C, C};
    tj.job[tj.n++] = TransposeJob{wt->qkv_w, ws + w.wTqkv, 3 * C, C};
    if (with_mlp) {
      tj.job[tj.n++] = TransposeJob{wt->fc2_w, ws + w.wTfc2, C, p.hid};
      tj.job[tj.n++] = TransposeJob{wt->fc1_w, ws + w.wTfc1, p.hid, C};
    }
    HIPCHECK(transpose_jobs(tj, st), "bwd: weight transposes");
  }
  // qkv (q unscaled, V transposed for the MFMA attention): the fused wave
  // kernel gathers (and normalises) the token rows itself and also writes the
  // attention's prepared bias tables; else a GEMM on the window rows w.n1w
  AttnArgs a = attn_args(p, ws + w.q, ws + w.k, ws + w.v, wt->rpb_table, ws + w.o, d->flags, ws + w.tab);
  if (winproj_supported(p.dt, C, p.d, p.N, 1)) {
    HIPCHECK(qkv_proj(ga.x, ga.g, ga.b, ga.eps, ga.ln, wt->qkv_w, wt->qkv_b, ws + w.q, ws + w.k, ws + w.v, 1, 1.0f,
                      p.Lp, C, p.heads, p.d, p.geo, wt->rpb_table, ws + w.tab, tab4_geo(p.rel, p.heads, p.N), st),
             "bwd: qkv projection");
    a.tab_ready = 1;
  } else {
    EpiArgs e{};
    e.kind = Epi::kQKV;
    e.bias = wt->qkv_b;
    e.out = ws + w.q; e.out2 = ws + w.k; e.out3 = ws + w.v;
    e.C = C; e.heads = p.heads; e.d = p.d; e.N = p.N; e.geo = p.geo;
    e.vt = 1;
    HIPCHECK(gemm(p.dt, ws + w.n1w, wt->qkv_w, p.Lp, 3 * C, C, e, st), "bwd: qkv gemm");
  }
  a.lse = (float*)(ws + w.lse);
  HIPCHECK(attention_mfma(a, st), "bwd: attention forward");
  // the caller's middle part: everything between the attention output and
  // the window-row gradient of the branch output (w.dyw)
  CHECK(mid());
  // projection
  HIPCHECK(wgrad_partials(ws + w.dyw, ws + w.o, g->proj_w, g->proj_b, (float*)(ws + w.pproj), p.Lp, C, C,
                          wj.job[wj.n++], st),
           "bwd: proj weight gradient");
  EpiArgs eb{};
  eb.kind = Epi::kBias;
  eb.out = ws + w.dout;
  eb.ld_out = C;
  HIPCHECK(gemm(p.dt, ws + w.dyw, ws + w.wTproj, p.Lp, C, C, eb, st), "bwd: proj input gradient");
  // attention
  AttnBwdArgs b{};
  b.a = a;
  b.dout = ws + w.dout;
  b.lse = (const float*)(ws + w.lse);
  b.dqkv = (bf16_t*)(ws + w.dqkv);
  b.dtable = g->rpb_table;
  b.work = ws + w.attn;
  HIPCHECK(attention_bwd(b, st), "bwd: attention");
  // qkv
  HIPCHECK(wgrad_partials(ws + w.dqkv, ws + w.n1w, g->qkv_w, g->qkv_b, (float*)(ws + w.pqkv), p.Lp, 3 * C, C,
                          wj.job[wj.n++], st),
           "bwd: qkv weight gradient");
  eb.out = ws + w.dn1w;
  HIPCHECK(gemm(p.dt, ws + w.dqkv, ws + w.wTqkv, p.Lp, C, 3 * C, eb, st), "bwd: qkv input gradient");
  HIPCHECK(reverse_scatter(p.dt, ws + w.dn1w, nullptr, dxo, p.Lp, C, p.geo, st), "bwd: window rows to tokens");
  return VSWIN_OK;
}

// an empty batch: every gradient the caller passed is zero
vswin_status zero_grads(const Plan& p, const vswin_block_grads* g, hipStream_t st) {
  if (!g) return VSWIN_OK;
  const int64_t C = p.C, H = p.hid;
  const std::pair<float*, int64_t> z[] = {
      {g->ln1_g, C}, {g->ln1_b, C}, {g->qkv_w, 3 * C * C}, {g->qkv_b, 3 * C}, {g->proj_w, C * C},
      {g->proj_b, C}, {g->rpb_table, (int64_t)p.rel.rows * p.heads}, {g->ln2_g, C}, {g->ln2_b, C},
      {g->fc1_w, H * C}, {g->fc1_b, H}, {g->fc2_w, C * H}, {g->fc2_b, C}};
  for (const auto& e : z) HIPCHECK(zero_f32(e.first, e.second, st), "bwd: zero gradients");
  return VSWIN_OK;
}

vswin_status check_bwd_args(const Plan& p, const vswin_desc* desc, const void* x, const vswin_block_weights* w,
                            const void* dy, const void* dx, const vswin_block_grads* g, const void* workspace,
                            size_t workspace_bytes, size_t need) {
  if (!bwd_supported(p, desc))
    return fail(VSWIN_ERR_UNSUPPORTED, "backward needs bf16, head_dim 32, C <= 768 and the MFMA attention (at most "
                                       "1024 tokens per window)");
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(dy, "dy"));
  CHECK(check_ptr(dx, "dx"));
  if (dx == x || dx == dy) return fail(VSWIN_ERR_INVALID_ARG, "dx must not alias x or dy");
  CHECK(check_msa_weights(w));
  if (!g) return fail(VSWIN_ERR_INVALID_ARG, "grads is NULL");
  CHECK(check_ptr(g->qkv_w, "g.qkv_w"));
  CHECK(check_ptr(g->qkv_b, "g.qkv_b", true));
  CHECK(check_ptr(g->proj_w, "g.proj_w"));
  CHECK(check_ptr(g->proj_b, "g.proj_b", true));
  CHECK(check_ptr(g->rpb_table, "g.rpb_table"));
  if (!workspace || !aligned(workspace, 256))
    return fail(VSWIN_ERR_WORKSPACE, "workspace is NULL or not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(VSWIN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  return VSWIN_OK;
}

}  // namespace

vswin_status vswin_window_msa_bwd(const vswin_desc* desc, const void* x_norm, const vswin_block_weights* w,
                                  const void* dy, void* dx_norm, const vswin_block_grads* g, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.L == 0) {   // empty batch: the gradients the caller passed are zero
    vswin_block_grads gm{};
    if (g) {
      gm.qkv_w = g->qkv_w; gm.qkv_b = g->qkv_b; gm.proj_w = g->proj_w; gm.proj_b = g->proj_b;
      gm.rpb_table = g->rpb_table;
    }
    return zero_grads(p, g ? &gm : nullptr, (hipStream_t)stream);
  }
  const BwdWs L = bwd_layout(p, desc);
  CHECK(check_bwd_args(p, desc, x_norm, w, dy, dx_norm, g, workspace, workspace_bytes, L.msa_bytes));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  HIPCHECK(ln_gather(p.dt, x_norm, nullptr, nullptr, ws + L.n1w, p.Lp, p.C, desc->ln_eps, p.geo, 0, st),
           "bwd: partition");
  const GatherA ga{x_norm, nullptr, nullptr, desc->ln_eps, 0, p.geo};
  WgradJobs wj{};
  CHECK(msa_bwd_core(p, desc, w, g, ws, L, dx_norm, st, false, ga, wj, [&]() -> vswin_status {
    HIPCHECK(ln_gather(p.dt, dy, nullptr, nullptr, ws + L.dyw, p.Lp, p.C, desc->ln_eps, p.geo, 0, st),
             "bwd: partition of dy");
    return VSWIN_OK;
  }));
  HIPCHECK(wgrad_reduce(wj, st), "bwd: weight gradient reduction");
  return VSWIN_OK;
}

vswin_status vswin_block_bwd(const vswin_desc* desc, const void* x, const vswin_block_weights* w, const void* dy,
                             void* dx, const vswin_block_grads* g, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p));
  if (p.L == 0) return zero_grads(p, g, (hipStream_t)stream);   // empty batch: zero gradients
  const BwdWs L = bwd_layout(p, desc);
  CHECK(check_bwd_args(p, desc, x, w, dy, dx, g, workspace, workspace_bytes, L.block_bytes));
  CHECK(check_ptr(w->ln1_g, "ln1_g"));
  CHECK(check_ptr(w->ln1_b, "ln1_b"));
  CHECK(check_ptr(w->ln2_g, "ln2_g"));
  CHECK(check_ptr(w->ln2_b, "ln2_b"));
  CHECK(check_ptr(w->fc1_w, "fc1_w"));
  CHECK(check_ptr(w->fc1_b, "fc1_b", true));
  CHECK(check_ptr(w->fc2_w, "fc2_w"));
  CHECK(check_ptr(w->fc2_b, "fc2_b", true));
  const float* req[] = {g->ln1_g, g->ln1_b, g->ln2_g, g->ln2_b, g->fc1_w, g->fc2_w};
  const char* names[] = {"g.ln1_g", "g.ln1_b", "g.ln2_g", "g.ln2_b", "g.fc1_w", "g.fc2_w"};
  for (int i = 0; i < 6; ++i) CHECK(check_ptr(req[i], names[i]));
  CHECK(check_ptr(g->fc1_b, "g.fc1_b", true));
  CHECK(check_ptr(g->fc2_b, "g.fc2_b", true));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int C = p.C, hid = p.hid;
  float* part = (float*)(ws + L.part);
  WgradJobs wj{};
  LnReds lr{};
  lr.n = 2;
  // LN1 + pad + roll + partition of x
  HIPCHECK(ln_gather(p.dt, x, w->ln1_g, w->ln1_b, ws + L.n1w, p.Lp, C, desc->ln_eps, p.geo, 1, st),
           "bwd: ln1 gather");
  auto mid = [&]() -> vswin_status {
    // forward: z^ = x + proj(o) (fp32 token rows), LN2, fc1, GELU
    EpiArgs e2{};
    e2.kind = Epi::kProjRes;
    e2.bias = w->proj_b;
    e2.out = ws + L.zh;
    e2.res = x;
    e2.C = C; e2.heads = p.heads; e2.d = p.d; e2.N = p.N; e2.geo = p.geo;
    HIPCHECK(gemm(p.dt, ws + L.o, w->proj_w, p.Lp, C, C, e2, st), "bwd: proj forward");
    HIPCHECK(ln_rows(VSWIN_FP32, p.dt, ws + L.zh, w->ln2_g, w->ln2_b, ws + L.n2, p.L, C, desc->ln_eps, st),
             "bwd: ln2 forward");
    EpiArgs e{};
    e.kind = Epi::kBias;
    e.bias = w->fc1_b;
    e.out = ws + L.a1;
    e.ld_out = hid;
    HIPCHECK(gemm(p.dt, ws + L.n2, w->fc1_w, p.L, hid, C, e, st), "bwd: fc1 forward");
    HIPCHECK(gelu_apply(ws + L.a1, ws + L.h, p.L * hid, 0, st), "bwd: gelu forward");
    // fc2
    HIPCHECK(wgrad_partials(dy, ws + L.h, g->fc2_w, g->fc2_b, (float*)(ws + L.pfc2), p.L, C, hid, wj.job[wj.n++],
                            st),
             "bwd: fc2 weight gradient");
    EpiArgs eb{};
    eb.kind = Epi::kBias;
    eb.out = ws + L.dh;
    eb.ld_out = hid;
    HIPCHECK(gemm(p.dt, dy, ws + L.wTfc2, p.L, hid, C, eb, st), "bwd: fc2 input gradient");
    HIPCHECK(gelu_apply(ws + L.a1, ws + L.dh, p.L * hid, 1, st), "bwd: gelu backward");
    // fc1
    HIPCHECK(wgrad_partials(ws + L.dh, ws + L.n2, g->fc1_w, g->fc1_b, (float*)(ws + L.pfc1), p.L, hid, C,
                            wj.job[wj.n++], st),
             "bwd: fc1 weight gradient");
    eb.out = ws + L.dn1;   // dLN2 output, token rows (the buffer is reused for dLN1 later)
    eb.ld_out = C;
    HIPCHECK(gemm(p.dt, ws + L.dh, ws + L.wTfc1, p.L, C, hid, eb, st), "bwd: fc1 input gradient");
    // LN2 (+ the residual path of y = z^ + ...)
    HIPCHECK(ln_bwd(1, ws + L.zh, w->ln2_g, ws + L.dn1, 0, dy, 1, ws + L.dzh, (float*)(ws + L.pln2), g->ln2_g,
                    g->ln2_b, p.L, C, desc->ln_eps, lr.job[1], st),
             "bwd: ln2 backward");
    HIPCHECK(gather_f32_bf16((const float*)(ws + L.dzh), ws + L.dyw, p.Lp, C, p.geo, st), "bwd: gather dz");
    return VSWIN_OK;
  };
  const GatherA ga{x, w->ln1_g, w->ln1_b, desc->ln_eps, 1, p.geo};
  CHECK(msa_bwd_core(p, desc, w, g, ws, L, ws + L.dn1, st, true, ga, wj, mid));
  // the four weight gradients from their partials, one launch
  HIPCHECK(wgrad_reduce(wj, st), "bwd: weight gradient reduction");
  // LN1 (+ the residual path of z^ = x + ...)
  HIPCHECK(ln_bwd(0, x, w->ln1_g, ws + L.dn1, 1, ws + L.dzh, 0, dx, part, g->ln1_g, g->ln1_b, p.L, C, desc->ln_eps,
                  lr.job[0], st),
           "bwd: ln1 backward");
  // dγ, dβ of both LayerNorms from their partials, one launch
  HIPCHECK(ln_reduce(lr, st), "bwd: layernorm gradient reduction");
  return VSWIN_OK;
}

vswin_status vswin_mfma_rate_probe(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (blocks < 1 || iters < 1) return fail(VSWIN_ERR_INVALID_ARG, "blocks=%d iters=%d", blocks, iters);
  CHECK(check_ptr(out, "out"));
  HIPCHECK(mfma_rate(out, blocks, iters, (hipStream_t)stream), "mfma rate probe");
  return VSWIN_OK;
}

vswin_status vswin_issue_probe(float* out, int32_t blocks, int32_t iters, int32_t mode, void* stream) {
  if (blocks < 1 || iters < 1 || mode < 0 || mode > 3)
    return fail(VSWIN_ERR_INVALID_ARG, "blocks=%d iters=%d mode=%d", blocks, iters, mode);
  CHECK(check_ptr(out, "out"));
  HIPCHECK(issue_probe(out, blocks, iters, mode, (hipStream_t)stream), "issue probe");
  return VSWIN_OK;
}

vswin_status vswin_index_map(const vswin_desc* desc, int32_t* map, uint8_t* region, void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p, false));
  if (p.Lp == 0) return VSWIN_OK;
  if (!map) return fail(VSWIN_ERR_INVALID_ARG, "map is NULL");
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  WinGeo g = p.geo;
  g.slot_perm = 0;   // the export reports natural (pt, ph, pw) order
  HIPCHECK(index_map(map, region, p.Lp, g, (hipStream_t)stream), "index map");
  return VSWIN_OK;
}

vswin_status vswin_partition_fwd(const vswin_desc* desc, const void* x, void* windows, void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p, false));
  if (p.Lp == 0) return VSWIN_OK;
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(windows, "windows"));
  if (p.Lp == 0) return VSWIN_OK;
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  WinGeo g = p.geo;
  g.slot_perm = 0;
  HIPCHECK(ln_gather(p.dt, x, nullptr, nullptr, windows, p.Lp, p.C, desc->ln_eps, g, 0, (hipStream_t)stream),
           "partition");
  return VSWIN_OK;
}

vswin_status vswin_reverse_fwd(const vswin_desc* desc, const void* windows, const void* residual, void* y,
                               void* stream) {
  Plan p{};
  CHECK(make_plan(desc, p, false));
  if (p.Lp == 0) return VSWIN_OK;
  CHECK(check_ptr(windows, "windows"));
  CHECK(check_ptr(residual, "residual", true));
  CHECK(check_ptr(y, "y"));
  if (p.Lp == 0) return VSWIN_OK;
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  WinGeo g = p.geo;
  g.slot_perm = 0;
  HIPCHECK(reverse_scatter(p.dt, windows, residual, y, p.Lp, p.C, g, (hipStream_t)stream), "reverse");
  return VSWIN_OK;
}

vswin_status vswin_layernorm_fwd(int64_t rows, int32_t C, vswin_dtype in_dtype, vswin_dtype out_dtype,
                                 const void* x, const void* g, const void* b, float eps, void* y, void* stream) {
  if (rows < 0 || C < 2 || C % 2 || C > 4096) return fail(VSWIN_ERR_INVALID_ARG, "rows=%lld C=%d", (long long)rows, C);
  if ((in_dtype != VSWIN_FP32 && in_dtype != VSWIN_BF16) || (out_dtype != VSWIN_FP32 && out_dtype != VSWIN_BF16))
    return fail(VSWIN_ERR_INVALID_ARG, "bad dtype");
  if (!(eps > 0.f)) return fail(VSWIN_ERR_INVALID_ARG, "eps must be > 0");
  if (rows == 0) return VSWIN_OK;
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(g, "g"));
  CHECK(check_ptr(b, "b"));
  CHECK(check_ptr(y, "y"));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  HIPCHECK(ln_rows(in_dtype, out_dtype, x, g, b, y, rows, C, eps, (hipStream_t)stream), "layernorm");
  return VSWIN_OK;
}

size_t vswin_patch_embed_workspace(int32_t B, int32_t Cin, int32_t T, int32_t H, int32_t W, const int32_t patch[3],
                                   vswin_dtype dtype) {
  if (!patch || patch[0] < 1 || patch[1] < 1 || patch[2] < 1 || B < 0 || Cin < 1) return 0;
  const int64_t rows = (int64_t)B * ((T + patch[0] - 1) / patch[0]) * ((H + patch[1] - 1) / patch[1]) *
                       ((W + patch[2] - 1) / patch[2]);
  return align256((size_t)rows * Cin * patch[0] * patch[1] * patch[2] * elem_size(dtype));
}

vswin_status vswin_patch_embed_fwd(int32_t B, int32_t Cin, int32_t T, int32_t H, int32_t W, const int32_t patch[3],
                                   int32_t C, vswin_dtype dtype, const void* video, const void* w, const void* b,
                                   void* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (!patch || patch[0] < 1 || patch[1] < 1 || patch[2] < 1)
    return fail(VSWIN_ERR_INVALID_ARG, "bad patch size");
  if (B < 0 || Cin < 1 || T < 1 || H < 1 || W < 1 || C < 1)
    return fail(VSWIN_ERR_INVALID_ARG, "bad video shape");
  if (dtype != VSWIN_FP32 && dtype != VSWIN_BF16) return fail(VSWIN_ERR_INVALID_ARG, "bad dtype");
  const int K = Cin * patch[0] * patch[1] * patch[2];
  if (dtype == VSWIN_BF16 && (K % 32 || C % 32))
    return fail(VSWIN_ERR_UNSUPPORTED, "bf16 patch embed needs Cin*patch and C multiples of 32");
  if (dtype == VSWIN_FP32 && C % 4) return fail(VSWIN_ERR_UNSUPPORTED, "C must be a multiple of 4");
  if (B == 0) return VSWIN_OK;
  CHECK(check_ptr(video, "video"));
  CHECK(check_ptr(w, "w"));
  CHECK(check_ptr(b, "b", true));
  CHECK(check_ptr(y, "y"));
  const size_t need = vswin_patch_embed_workspace(B, Cin, T, H, W, patch, dtype);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(VSWIN_ERR_WORKSPACE, "patch embed needs %zu workspace bytes", need);
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  hipStream_t st = (hipStream_t)stream;
  HIPCHECK(patch_gather(dtype, video, workspace, B, Cin, T, H, W, patch[0], patch[1], patch[2], st), "patch gather");
  const int64_t rows = (int64_t)B * ((T + patch[0] - 1) / patch[0]) * ((H + patch[1] - 1) / patch[1]) *
                       ((W + patch[2] - 1) / patch[2]);
  EpiArgs e{};
  e.kind = Epi::kBias;
  e.bias = b;
  e.out = y;
  e.ld_out = C;
  HIPCHECK(gemm(dtype, workspace, w, rows, C, K, e, st), "patch embed gemm");
  return VSWIN_OK;
}

size_t vswin_patch_merge_workspace(int32_t B, int32_t T, int32_t H, int32_t W, int32_t C, vswin_dtype dtype) {
  if (B < 0 || T < 1 || H < 1 || W < 1 || C < 1) return 0;
  const int64_t rows = (int64_t)B * T * ((H + 1) / 2) * ((W + 1) / 2);
  return 2 * align256((size_t)rows * 4 * C * elem_size(dtype));
}

vswin_status vswin_patch_merge_fwd(int32_t B, int32_t T, int32_t H, int32_t W, int32_t C, int32_t Cout,
                                   vswin_dtype dtype, const void* x, const void* ln_g, const void* ln_b,
                                   const void* w, const void* b, float eps, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 1 || H < 1 || W < 1 || C < 1 || Cout < 1) return fail(VSWIN_ERR_INVALID_ARG, "bad shape");
  if (dtype != VSWIN_FP32 && dtype != VSWIN_BF16) return fail(VSWIN_ERR_INVALID_ARG, "bad dtype");
  if (!(eps > 0.f)) return fail(VSWIN_ERR_INVALID_ARG, "eps must be > 0");
  if (C % 8) return fail(VSWIN_ERR_UNSUPPORTED, "C must be a multiple of 8");
  if (4 * C > 4096) return fail(VSWIN_ERR_UNSUPPORTED, "4C > 4096");
  if (dtype == VSWIN_BF16 && Cout % 32) return fail(VSWIN_ERR_UNSUPPORTED, "bf16 merge needs Cout %% 32 == 0");
  if (dtype == VSWIN_FP32 && Cout % 4) return fail(VSWIN_ERR_UNSUPPORTED, "Cout must be a multiple of 4");
  if (B == 0) return VSWIN_OK;
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(ln_g, "ln_g"));
  CHECK(check_ptr(ln_b, "ln_b"));
  CHECK(check_ptr(w, "w"));
  CHECK(check_ptr(b, "b", true));
  CHECK(check_ptr(y, "y"));
  const size_t need = vswin_patch_merge_workspace(B, T, H, W, C, dtype);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(VSWIN_ERR_WORKSPACE, "patch merge needs %zu workspace bytes", need);
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  hipStream_t st = (hipStream_t)stream;
  const int64_t rows = (int64_t)B * T * ((H + 1) / 2) * ((W + 1) / 2);
  char* g4 = (char*)workspace;
  char* n4 = g4 + need / 2;
  HIPCHECK(merge_gather(dtype, x, g4, B, T, H, W, C, st), "merge gather");
  HIPCHECK(ln_rows(dtype, dtype, g4, ln_g, ln_b, n4, rows, 4 * C, eps, st), "merge layernorm");
  EpiArgs e{};
  e.kind = Epi::kBias;
  e.bias = b;
  e.out = y;
  e.ld_out = Cout;
  HIPCHECK(gemm(dtype, n4, w, rows, Cout, 4 * C, e, st), "merge gemm");
  return VSWIN_OK;
}


size_t vswin_head_workspace(int32_t B, int64_t L, int32_t C) {
  if (B < 0 || L < 1 || C < 1) return 0;
  return align256(head_workspace_floats(B, L, C) * sizeof(float));
}

vswin_status vswin_head_fwd(int32_t B, int64_t L, int32_t C, int32_t K, vswin_dtype dtype, const void* x,
                            const void* w, const void* b, float* logits, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (B < 0 || L < 1 || K < 0 || C < 4 || C % 4 || C > 4096)
    return fail(VSWIN_ERR_INVALID_ARG, "head: B=%d L=%lld C=%d K=%d", B, (long long)L, C, K);
  if (dtype != VSWIN_FP32 && dtype != VSWIN_BF16) return fail(VSWIN_ERR_INVALID_ARG, "bad dtype");
  if (B == 0 || K == 0) return VSWIN_OK;
  CHECK(check_ptr(x, "x"));
  CHECK(check_ptr(w, "w"));
  CHECK(check_ptr(b, "b", true));
  CHECK(check_ptr(logits, "logits"));
  const size_t need = vswin_head_workspace(B, L, C);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(VSWIN_ERR_WORKSPACE, "head needs %zu workspace bytes", need);
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  HIPCHECK(head_fwd(dtype, x, w, b, logits, (float*)workspace, B, L, C, K, (hipStream_t)stream), "head");
  return VSWIN_OK;
}

vswin_status vswin_multiview_average(int32_t B, int32_t V, int32_t K, const float* logits, float* probs,
                                     void* stream) {
  if (B < 0 || V < 1 || V > view_avg_max_views() || K < 1)
    return fail(VSWIN_ERR_INVALID_ARG, "multiview: B=%d V=%d K=%d (V <= %d)", B, V, K, view_avg_max_views());
  if (B == 0) return VSWIN_OK;
  CHECK(check_ptr(logits, "logits"));
  CHECK(check_ptr(probs, "probs"));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  HIPCHECK(view_avg(logits, probs, B, V, K, (hipStream_t)stream), "multiview average");
  return VSWIN_OK;
}

vswin_status vswin_inflate_patch_embed(int32_t C, int32_t Cin, int32_t pt, int32_t ph, int32_t pw,
                                       vswin_dtype dtype, const void* w2, void* w3, void* stream) {
  if (C < 1 || Cin < 1 || pt < 1 || ph < 1 || pw < 1)
    return fail(VSWIN_ERR_INVALID_ARG, "inflate patch: C=%d Cin=%d patch=(%d,%d,%d)", C, Cin, pt, ph, pw);
  if (dtype != VSWIN_FP32 && dtype != VSWIN_BF16) return fail(VSWIN_ERR_INVALID_ARG, "bad dtype");
  CHECK(check_ptr(w2, "w2"));
  CHECK(check_ptr(w3, "w3"));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  HIPCHECK(inflate_patch(dtype, w2, w3, (int64_t)C * Cin, pt, ph, pw, (hipStream_t)stream), "inflate patch");
  return VSWIN_OK;
}

vswin_status vswin_inflate_bias_table(int32_t rows2d, int32_t heads, int32_t P, vswin_dtype dtype, const void* t2,
                                      void* t3, void* stream) {
  if (rows2d < 1 || heads < 1 || P < 1)
    return fail(VSWIN_ERR_INVALID_ARG, "inflate table: rows=%d heads=%d P=%d", rows2d, heads, P);
  if (dtype != VSWIN_FP32 && dtype != VSWIN_BF16) return fail(VSWIN_ERR_INVALID_ARG, "bad dtype");
  CHECK(check_ptr(t2, "t2"));
  CHECK(check_ptr(t3, "t3"));
  if (fault_injected()) return fail(VSWIN_ERR_HIP, "injected launch failure (VSWIN_FAULT=launch)");
  const int64_t halves = (int64_t)rows2d * heads * (dtype == VSWIN_FP32 ? 2 : 1);
  HIPCHECK(inflate_table(t2, t3, halves, 2 * P - 1, (hipStream_t)stream), "inflate table");
  return VSWIN_OK;
}

}  // extern "C"
