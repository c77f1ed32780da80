// Host-side launchers of the vswin kernels (internal to libvswin.so).
#pragma once

#include "vswin_common.h"

namespace vswin {

// --- launch helpers (vswin_api.hip) ---------------------------------------
// compute units of the current device (queried once per device)
int device_cu_count();
// raise `kern`'s dynamic LDS limit to `bytes` once per (kernel, device, size)
hipError_t ensure_dynamic_lds(const void* kern, size_t bytes);

// --- permutation / normalisation (k_layout.hip) ---------------------------
hipError_t ln_gather(vswin_dtype dt, const void* x, const void* g, const void* b, void* y, int64_t slots,
                     int C, float eps, const WinGeo& geo, int apply_ln, hipStream_t st);
hipError_t ln_rows(vswin_dtype in_dt, vswin_dtype out_dt, const void* x, const void* g, const void* b,
                   void* y, int64_t rows, int C, float eps, hipStream_t st);
hipError_t reverse_scatter(vswin_dtype dt, const void* win, const void* res, void* y, int64_t slots, int C,
                           const WinGeo& geo, hipStream_t st);
hipError_t index_map(int32_t* map, uint8_t* region, int64_t slots, const WinGeo& geo, hipStream_t st);

// --- GEMMs (k_gemm.hip): out = A (M x K) * W^T (W: N x K) + epilogue -------
enum class Epi : int {
  kBias = 0,     // out[m, n] = acc + bias                      (out: dtype)
  kQKV = 1,      // acc + bias scattered to q/k/v (nW, heads, N, d)
  kProjRes = 2,  // zh[src(m), n] = x[src(m), n] + acc + bias   (zh fp32)
  kProjOut = 3,  // y[src(m), n] = acc + bias                   (y: dtype)
  kGelu = 4,     // out[m, n] = gelu(acc + bias)                (out: dtype)
  kRes = 5,      // out[m, n] = res32[m, n] + acc + bias        (out: dtype)
};

struct EpiArgs {
  Epi kind;
  const void* bias;   // (N) of dtype, nullable
  void* out;          // primary output
  void* out2;         // kQKV: k, out3: v
  void* out3;
  const void* res;    // kProjRes: x (dtype); kRes: zh (fp32)
  int64_t ld_out;     // row pitch of out (elements) for kBias/kGelu/kRes
  // kQKV / kProj*: geometry
  int C, heads, d, N;
  WinGeo geo;
  int vt;             // kQKV: write v transposed (item, d, N) (MFMA attention layout)
};

// Optional A-row gather: row m of A = token row src(m) of x (zeros for pad
// slots), layer-normalised with g, b when `ln` (bf16, K in {96, 128} only).
struct GatherA {
  const void* x;
  const void* g;
  const void* b;
  float eps;
  int ln;
  WinGeo geo;
};
hipError_t gemm(vswin_dtype dt, const void* A, const void* W, int64_t M, int N, int K, const EpiArgs& e,
                hipStream_t st, const GatherA* ga = nullptr);
bool gemm_can_gather(vswin_dtype dt, int K);

// --- window projections for C in {96, 128}, bf16 (k_winproj.hip) ----------
// qkv: gather (+ LN1 when ln) window rows of x, project, split by head into
// q, k (nW*heads, N, d) and v (same, or transposed (nW*heads, d, N) when vt).
// out: o rows * W^T + bias scattered to token rows; with `res` the output is
// fp32 z = res + ..., else bf16.
bool winproj_supported(vswin_dtype dt, int C, int d, int N, int vt);
// q is multiplied by qscale after the bias (1 for plain q).  With tab4
// non-null, extra workgroups also write the attention's prepared tables
// (tg) of `table` there.
hipError_t qkv_proj(const void* x, const void* ln_g, const void* ln_b, float eps, int ln, const void* W,
                    const void* bias, void* q, void* k, void* v, int vt, float qscale, int64_t M, int C, int heads,
                    int d, const WinGeo& geo, const void* table, void* tab4, const Tab4Geo& tg, hipStream_t st);
hipError_t out_proj(const void* o, const void* W, const void* bias, const void* res, void* out, int64_t M, int C,
                    const WinGeo& geo, hipStream_t st);

// --- attention (k_attention.hip: generic; k_attn_mfma.hip: MFMA) -----------
struct AttnArgs {
  const void *q, *k, *v;   // (nW, heads, N, d) of dtype; MFMA path: v is (nW, heads, d, N)
  const void* table;       // (rows, heads) of dtype
  void* o;                 // (nW, N, C) of dtype
  int64_t nW;
  int heads, d, C, N;
  RelTab rel;
  WinGeo geo;
  int use_mask;            // some window may need the region mask
  int mask_m100;           // additive -100 instead of exclusion
  int force_max;           // MFMA kernel: always take the exact row-max pass
  int q_scaled;            // MFMA kernel: q already multiplied by log2(e) / sqrt(d)
  void* tab4;              // MFMA kernel: workspace of attention_workspace_bytes for the prepared tables
  int tab_ready;           // MFMA kernel: tab4 already holds this call's tables
  float* lse;              // MFMA kernel, nullable: (nW*heads, N) log2 of each query row's sum of
                           // exp2 of its log2-domain logits (the backward's normaliser)
};
// bytes of workspace the MFMA kernel needs for its prepared bias tables
// (heads * TS4 fp32 4-tuples) and their extents
size_t attention_workspace_bytes(const RelTab& rel, int heads, int N);
Tab4Geo tab4_geo(const RelTab& rel, int heads, int N);
// the attention for shapes the bf16 MFMA kernel does not serve: fp32 on the
// matrix cores where attention_f32_mfma_supported, else the SIMT kernel
hipError_t attention_generic(vswin_dtype dt, const AttnArgs& a, hipStream_t st);
// fp32, head_dim 16, 32 or 64, K, V and the bias column within 160 KB of LDS
bool attention_f32_mfma_supported(vswin_dtype dt, const AttnArgs& a);
hipError_t attention_f32_mfma(const AttnArgs& a, hipStream_t st);
hipError_t attention_mfma(const AttnArgs& a, hipStream_t st);
// shapes the MFMA kernel serves (bf16, d = 32, temporal window % 4 == 0 with
// group-uniform temporal labels, no additive -100 mask): N <= kMfmaMaxN with
// the 4-tuple bias table, or up to kMfmaBigN with the scalar table and the
// 7 x 7 spatial window
constexpr int kMfmaMaxN = 512;
constexpr int kMfmaBigN = 1024;
bool attention_mfma_supported(vswin_dtype dt, const AttnArgs& a);

// LN1 + gather + qkv projection + MFMA attention in one kernel (bf16, C in
// {96, 128}, head_dim 32, the MFMA kernel's 4-tuple-table forms with group
// labels and the exclusion mask): o (a.o, window rows in slot order) from the
// token rows x; a.table is the (rows, heads) bf16 table; a.q, a.k, a.v and
// a.tab4 are not used.  With ln == 0 the rows are taken as they are.
struct FusedArgs {
  AttnArgs a;
  const void* x;        // token rows (B*T*H*W, C)
  const void* ln_g;     // LN1 gamma, beta (C)
  const void* ln_b;
  float eps;
  int ln;
  const void* w;        // (3C, C)
  const void* bias;     // (3C) or NULL
};
bool attention_fused_supported(vswin_dtype dt, const AttnArgs& a);
hipError_t attention_fused(const FusedArgs& f, hipStream_t st);

// Backward of the MFMA attention (bf16, d = 32, group-uniform region labels,
// exclusion mask).  In: a.q (q * log2(e) / sqrt(d)), a.k, a.v (V^T), a.o,
// a.table as the forward had them, dout (window rows), lse (the forward's
// a.lse output).  Out: dqkv rows (nW*N, 3C) = [dq | dk | dv] for the
// unscaled q, k, v; dtable (rows, heads) fp32.  work: attention_bwd_workspace_bytes.
struct AttnBwdArgs {
  AttnArgs a;
  const void* dout;
  const float* lse;
  bf16_t* dqkv;
  float* dtable;
  void* work;
  // set by attention_bwd inside `work`
  bf16_t *qr, *kr, *vr, *dor;   // padded rows (items, NPAD, 32)
  bf16_t *qt, *kt, *dot;        // transposes (items, 32, NPAD), pair order per 32-row block
  float* D;                     // (items, NPAD) row sums of dout * o
  float* dgrp;                  // per (item, query group, key group): 7 temporal-diagonal sums of dS
  float dq_scale, dk_scale;
};
bool attention_bwd_supported(vswin_dtype dt, const AttnArgs& a);
size_t attention_bwd_workspace_bytes(const AttnArgs& a);
hipError_t attention_bwd(const AttnBwdArgs& b, hipStream_t st);

// --- fused LN2 -> fc1 -> GELU -> fc2 -> residual (k_mlp.hip) --------------
// proj_mlp (bf16, C = 96 or 128, hid = 4C): the output projection in front as well,
// y = z^ + MLP(LN2(z^)), z^ = x + o Wp^T + bp with o the attention output in
// window-row space (gathered per token) and z^ kept in fp32 registers.
bool proj_mlp_supported(vswin_dtype dt, int C, int hid);
hipError_t proj_mlp(const void* o, const void* x, const void* wp, const void* bp, const void* g2, const void* b2ln,
                    const void* W1, const void* b1, const void* W2, const void* bo, void* y, int64_t L, int C,
                    float eps, const WinGeo& geo, hipStream_t st);
bool mlp_fused_supported(vswin_dtype dt, int C, int hid);
hipError_t mlp_fused(const float* zh, const void* g2, const void* b2ln, const void* W1, const void* b1,
                     const void* W2, const void* bo, void* y, int64_t L, int C, float eps, hipStream_t st);

// --- backward pieces (k_backward.hip) --------------------------------------
// dst (C x R) = src (R x C)^T, bf16
// bwd = 0: io = GELU(a); bwd = 1: io = io * GELU'(a)  (bf16, n % 8 == 0)
hipError_t gelu_apply(const void* a, void* io, int64_t n, int bwd, hipStream_t st);
// dst (C, R) = src (R, C)^T for up to 4 bf16 matrices in one launch
struct TransposeJob {
  const void* src;
  void* dst;
  int R, C;
};
struct TransposeJobs {
  TransposeJob job[4];
  int n;
};
hipError_t transpose_jobs(const TransposeJobs& jobs, hipStream_t st);
// bf16 window rows of an fp32 token-row tensor, zeros for pad slots
hipError_t gather_f32_bf16(const float* in, void* out, int64_t slots, int C, const WinGeo& geo, hipStream_t st);
// LayerNorm backward over rows of C (<= 768): out = dLN(x; g)/dx applied to dy, plus res (nullable);
// dg, db (fp32, C) from per-wave partials in part (ln_bwd_part_bytes)
size_t ln_bwd_part_bytes(int64_t rows, int C);
// the reduction of one LayerNorm backward's dg / db partials (np of them,
// 2C floats each); several run as one ln_reduce launch
struct LnRed {
  const float* part;
  float* dg;
  float* db;
  int np, C;
};
struct LnReds {
  LnRed job[2];
  int n;
};
hipError_t ln_reduce(const LnReds& jobs, hipStream_t st);
hipError_t ln_bwd(int x_fp32, const void* x, const void* g, const void* dy, int res_fp32, const void* res,
                  int out_fp32, void* out, float* part, float* dg, float* db, int64_t rows, int C, float eps,
                  LnRed& red, hipStream_t st);
// p[0 .. n) = 0 (a kernel, so that it may sit inside a captured graph); p nullable
hipError_t zero_f32(float* p, int64_t n, hipStream_t st);
// dW (NO x KI) = A^T B and db (NO, nullable) = column sums of A over M token rows,
// A (M x NO), B (M x KI) bf16; fp32 outputs; part: wgrad_part_bytes
size_t wgrad_part_bytes(int64_t M, int NO, int KI);
// One weight gradient's reduction: dW (n1 floats) and db (n - n1, or none)
// from np partial rows of `stride` floats.
struct WgradJob {
  const float* part;
  float* dW;
  float* db;
  int np;
  int64_t n, n1, stride;
};
struct WgradJobs {
  WgradJob job[4];
  int n;
};
// the partial rows of dW = A^T B (and db = column sums of A) into `part`,
// and the job that reduces them (wgrad_reduce, several jobs in one launch)
hipError_t wgrad_partials(const void* A, const void* B, float* dW, float* db, float* part, int64_t M, int NO, int KI,
                          WgradJob& job, hipStream_t st);
hipError_t wgrad_reduce(const WgradJobs& jobs, hipStream_t st);

// --- measurement helper (k_probe.hip) --------------------------------------
// blocks x 512 threads of v_mfma_f32_16x16x32_bf16 chains: 8 per wave per
// round, `iters` rounds; out holds blocks * 512 floats
hipError_t issue_probe(float* out, int blocks, int iters, int mode, hipStream_t st);
hipError_t mfma_rate(float* out, int blocks, int iters, hipStream_t st);

// --- patch embedding / merging gathers (k_patch.hip) ----------------------
hipError_t patch_gather(vswin_dtype dt, const void* video, void* out, int B, int Cin, int T, int H, int W,
                        int pt, int ph, int pw, hipStream_t st);
hipError_t merge_gather(vswin_dtype dt, const void* x, void* out, int B, int T, int H, int W, int C,
                        hipStream_t st);

// --- classification head, view average, inflation (k_head.hip) -------------
// token-row splits of the head's pooling; its fp32 workspace (partial sums,
// then the pooled vectors)
int head_splits(int B, int64_t L);
size_t head_workspace_floats(int B, int64_t L, int C);
hipError_t head_fwd(vswin_dtype dt, const void* x, const void* w, const void* b, float* logits, float* work,
                    int B, int64_t L, int C, int K, hipStream_t st);
int view_avg_max_views();
hipError_t view_avg(const float* logits, float* probs, int B, int V, int K, hipStream_t st);
hipError_t inflate_patch(vswin_dtype dt, const void* w2, void* w3, int64_t C_Cin, int pt, int ph, int pw,
                         hipStream_t st);
// t3 = reps copies of t2 (n2_halves 2-byte units; fp32 tables pass 2x the count)
hipError_t inflate_table(const void* t2, void* t3, int64_t n2_halves, int reps, hipStream_t st);

}  // namespace vswin
