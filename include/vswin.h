/*
 * vswin.h -- C ABI of the MI355X (gfx950) Video Swin 3D (shifted-)window
 * attention block library (libvswin.so).
 *
 * Every entry point takes plain pointers and sizes.  Device pointers point to
 * HIP device memory owned by the caller; the library never allocates, frees
 * or keeps a reference to caller memory.  Work is enqueued asynchronously on
 * the given HIP stream (`stream` is a hipStream_t; NULL = the null stream).
 *
 * Errors: argument errors are detected on the host before anything is
 * enqueued and leave every output untouched.  A call on an empty input
 * (B = 0, or zero rows) is a no-op that succeeds without looking at its
 * pointers.  Launch failures come back as
 * VSWIN_ERR_HIP.  No C++ exception crosses this boundary.  vswin_last_error()
 * returns a thread-local description of the last failing call on the calling
 * thread.  Calls keep no state between invocations and may be made from
 * several threads at once (with distinct output and workspace buffers).
 *
 * Method (Video Swin Transformer pages):
 *   block      = pre-norm block of eq. 1 (§3.1): z^ = x + MSA(LN1(x)),
 *                y = z^ + MLP(LN2(z^));
 *   MSA        = 3D window multi-head self-attention of §3.2 / eq. 2:
 *                pad -> roll(-shift) -> partition into P x Mh x Mw windows
 *                -> qkv Linear -> softmax(q k^T / sqrt(d) + B + mask) v
 *                -> proj Linear -> reverse partition -> roll(+shift) -> crop;
 *   B          = relative position bias read from a (2P-1)(2Mh-1)(2Mw-1) x
 *                heads table (§3.2, eq. 2);
 *   mask       = pairs of tokens that were not neighbours before the roll
 *                (§3.2, fig. 3) are excluded.
 * Conventions for points the pages leave open are stated at each entry point.
 */
#ifndef VSWIN_H_
#define VSWIN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VSWIN_ABI_VERSION 1

typedef enum {
  VSWIN_OK = 0,
  VSWIN_ERR_INVALID_ARG = -1,   /* bad descriptor, null or misaligned pointer    */
  VSWIN_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. head_dim > 64) */
  VSWIN_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required    */
  VSWIN_ERR_HIP = -4            /* a HIP call or kernel launch failed            */
} vswin_status;

typedef enum { VSWIN_FP32 = 0, VSWIN_BF16 = 1 } vswin_dtype;

/* Descriptor flags: readings of points the pages leave open.              */
enum {
  /* Pad tokens keep the region label of their grid position instead of
   * forming a region of their own (the published code's behaviour: pads are
   * visible in regular blocks).  Default off: pads are masked.            */
  VSWIN_F_PAD_VISIBLE = 1u,
  /* Clamp an axis's window to its size only when size < window (the pages'
   * literal "smaller").  Default: clamp when size <= window, shift 0.       */
  VSWIN_F_CLAMP_STRICT = 2u,
  /* Add -100 to masked scores (the published code's value) instead of
   * excluding the pair.  Default off: masked pairs get weight exactly 0.   */
  VSWIN_F_MASK_M100 = 4u,
  /* vswin_attention_fwd only (other entry points ignore it): the workspace
   * already holds the prepared bias tables of this rpb_table and geometry,
   * left there by an earlier vswin_attention_fwd call on the same workspace,
   * so they are not rebuilt.  For repeated calls with fixed weights; the
   * result is undefined if the table or the workspace changed since.      */
  VSWIN_F_TABLES_READY = 8u
};

/* One block's geometry.  Tokens are (B, T, H, W, C), contiguous, channels
 * last.  window/shift are the requested values (P, Mh, Mw) and (sP, sMh, sMw)
 * with 0 <= shift < window; the library applies the clamp itself and reports
 * the effective values through vswin_plan_query.  The relative-position
 * table is sized by the requested window.                                  */
typedef struct {
  int32_t B, T, H, W, C;
  int32_t heads;          /* C % heads == 0; head_dim = C / heads            */
  int32_t window[3];      /* requested window (P, Mh, Mw), all >= 1          */
  int32_t shift[3];       /* requested shift, 0 <= shift[i] < window[i]      */
  int32_t mlp_hidden;     /* MLP hidden width (4 * C for the pages' ratio)   */
  vswin_dtype dtype;      /* storage type of tokens, weights and outputs     */
  float ln_eps;           /* LayerNorm epsilon (1e-5)                        */
  uint32_t flags;         /* VSWIN_F_* bits                                  */
} vswin_desc;

/* Block weights: device pointers, element type = desc.dtype, PyTorch layouts
 * (Linear weight = (out, in), row-major).  All must be 16-byte aligned.
 * qkv output rows are [q | k | v], channel = head * head_dim + e.
 * rpb_table is (rows, heads) row-major, rows = (2P-1)(2Mh-1)(2Mw-1); the row
 * of a (query, key) pair with in-window offset (dt, dh, dw) = query - key is
 * (dt+P-1)(2Mh-1)(2Mw-1) + (dh+Mh-1)(2Mw-1) + (dw+Mw-1) (temporal outermost,
 * so that the §3.4 inflation tiling makes the bias frame independent).      */
typedef struct {
  const void *ln1_g, *ln1_b;     /* (C), (C)                                  */
  const void *qkv_w, *qkv_b;     /* (3C, C), (3C); qkv_b may be NULL          */
  const void *proj_w, *proj_b;   /* (C, C), (C); proj_b may be NULL           */
  const void *rpb_table;         /* (rows, heads)                             */
  const void *ln2_g, *ln2_b;     /* (C), (C)                                  */
  const void *fc1_w, *fc1_b;     /* (hidden, C), (hidden); fc1_b may be NULL  */
  const void *fc2_w, *fc2_b;     /* (C, hidden), (C); fc2_b may be NULL       */
} vswin_block_weights;

/* Result of planning one block.                                            */
typedef struct {
  int32_t eff_window[3];   /* window after the clamp                          */
  int32_t eff_shift[3];    /* shift after the clamp                           */
  int32_t padded[3];       /* (Tp, Hp, Wp): sizes rounded up to the window    */
  int32_t tokens_per_window; /* N = P * Mh * Mw                               */
  int64_t num_windows;     /* B * prod(padded / window)                      */
  int64_t tokens;          /* B * T * H * W                                  */
  int32_t masked;          /* 1 if any window needs the region mask          */
  int32_t fast_attention;  /* 1 if the MFMA attention kernel serves it       */
  size_t workspace_bytes;  /* device workspace needed by vswin_block_fwd     */
  size_t msa_workspace_bytes; /* ... and by vswin_window_msa_fwd             */
  size_t attention_workspace_bytes; /* ... and by vswin_attention_fwd        */
} vswin_plan;

/* Validate `desc` and report the clamped geometry and workspace sizes.
 * Host only: makes no HIP call.  Returns VSWIN_ERR_INVALID_ARG for a bad
 * descriptor (plan untouched), VSWIN_ERR_UNSUPPORTED when the geometry is
 * valid but vswin_block_fwd / vswin_window_msa_fwd cannot serve it (plan is
 * still filled in: the permutation entry points accept such descriptors).  Window/shift clamp (pages: Pitfalls and the
 * paper-vs-code notes): an axis whose size is <= its window (< with
 * VSWIN_F_CLAMP_STRICT) takes window = size and shift = 0.                  */
vswin_status vswin_plan_query(const vswin_desc* desc, vswin_plan* plan);

/* One Video Swin block (eq. 1):  y = z^ + MLP(LN2(z^)),
 * z^ = x + MSA(LN1(x)).  x, y: (B,T,H,W,C) of desc.dtype, must not alias.
 * MSA as in vswin_window_msa_fwd; MLP = Linear(C, hidden) -> erf GELU
 * -> Linear(hidden, C); LayerNorm with biased variance and desc.ln_eps.
 * In the bf16 path z^ is kept in fp32 (in registers of the fused projection +
 * MLP kernel at C = 96 and 128, else in the workspace), and the fused MLP
 * kernels take GELU from a piecewise linear table of the erf form (absolute
 * error below 2.5e-5 before the bf16 rounding of the hidden activations);
 * softmax runs in fp32 and the attention weights are rounded to bf16 for the
 * AV product.
 * A regular/shifted pair (eq. 1) is two calls: shift 0, then window // 2.
 * workspace: >= plan.workspace_bytes bytes of device memory, 256-byte
 * aligned, used as scratch for the duration of the call on `stream`.        */
vswin_status vswin_block_fwd(const vswin_desc* desc, const void* x,
                             const vswin_block_weights* w, void* y,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* vswin_block_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and result, with the scratch taken from a
 * static device array of VSWIN_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU the library runs on, held until the process ends) instead of
 * a caller workspace.  The call allocates and frees nothing.  A block whose
 * scratch need exceeds the array (at most plan.workspace_bytes; the Swin-T
 * stage-1 to stage-4 blocks at B = 1 and the stage-1 block at B = 2 fit)
 * returns VSWIN_ERR_WORKSPACE before anything is enqueued.  Every call on a
 * GPU shares that GPU's array and leaves its own contents there: calls that
 * overlap on one GPU (other streams, other host threads) race, so serialise
 * them.  Other arguments and errors as vswin_block_fwd.                    */
#define VSWIN_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)
vswin_status vswin_block_fwd_noalloc(const vswin_desc* desc, const void* x,
                                     const vswin_block_weights* w, void* y,
                                     void* stream);

/* The window attention branch alone (the pages' window_msa, §3.2 / eq. 2):
 * x_norm (B,T,H,W,C) is the LayerNorm output; y (same shape) receives the
 * projected attention output with no residual.  Zero padding is appended at
 * the end of each axis, then the padded grid is rolled by -shift; masked
 * pairs are those whose tokens carry different region labels, where along
 * every shifted axis of padded length n the rolled positions [0, n-w),
 * [n-w, n-s) and [n-s, n) form separate regions and pad tokens form their
 * own region (see VSWIN_F_PAD_VISIBLE).  The ln1_*, ln2_* and fc* fields of
 * `w` are ignored.  workspace >= plan.msa_workspace_bytes.                          */
vswin_status vswin_window_msa_fwd(const vswin_desc* desc, const void* x_norm,
                                  const vswin_block_weights* w, void* y,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* The attention core alone (eq. 2) on projected windows, in the layout
 * vswin_block_fwd keeps internally:
 *   q, k: [((w * heads + h) * N + s) * head_dim + e], o: [(w * N + s) * C +
 *   h * head_dim + e]; v: as q when plan.fast_attention == 0, else transposed
 *   [((w * heads + h) * head_dim + e) * N + s].
 * s is the row of a window slot: natural (pt, ph, pw) order when
 * plan.fast_attention == 0; otherwise the MFMA slot order s = 4 m + i for
 * the token (pt = 4 a + i, ph, pw), m = (a * Mh + ph) * Mw + pw.
 * o receives softmax(q k^T / sqrt(head_dim) + B + mask) v per window and head
 * (rows of pad slots are unspecified).  rpb_table as in vswin_block_weights.
 * workspace >= plan.attention_workspace_bytes (may be NULL when 0); when
 * plan.fast_attention == 1 it receives the fp32 prepared form of rpb_table
 * (heads x about 2.7K 16-byte 4-tuples for a (8,7,7) window) that the
 * kernel stages in LDS; see VSWIN_F_TABLES_READY.                          */
vswin_status vswin_attention_fwd(const vswin_desc* desc, const void* q, const void* k,
                                 const void* v, const void* rpb_table, void* o,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* LN1, pad + roll + partition, the qkv projection and the attention core of
 * one block (§3.2 / eq. 2: the (S)W-MSA branch of eq. 1 up to, not
 * including, its output projection), from the block input x (B,T,H,W,C):
 * o receives the heads' concatenated attention outputs in the window-row
 * layout of vswin_attention_fwd's o, [(w * N + s) * C + h * head_dim + e]
 * with s in the MFMA slot order (rows of pad slots unspecified).  Reads
 * w->ln1_g, ln1_b, qkv_w, qkv_b (may be NULL) and rpb_table; the other
 * fields are ignored.  Two launches (the qkv projection, which normalises
 * and gathers its rows, then the attention kernel; q, k and V^T pass
 * through the workspace); with the environment variable VSWIN_FUSED=1, and
 * where the geometry allows (at most 512 tokens per window, key groups of
 * uniform region), one kernel in which q, k and v never leave the chip,
 * with the same bits (vswin_block_fwd and vswin_window_msa_fwd follow the
 * same switch).  Needs bf16, head_dim 32, C in {96, 128} and
 * plan.fast_attention == 1, else VSWIN_ERR_UNSUPPORTED.
 * x and o must not alias; workspace >= plan.msa_workspace_bytes, 256-byte
 * aligned.                                                                   */
vswin_status vswin_qkv_attention_fwd(const vswin_desc* desc, const void* x, const vswin_block_weights* w,
                                     void* o, void* workspace, size_t workspace_bytes, void* stream);

/* Gradients of one block's weights (training): fp32 device buffers of the
 * weights' shapes (vswin_block_weights), each overwritten (not accumulated).
 * Bias gradients may be NULL (not computed); weight, table and LayerNorm
 * gradients are required by vswin_block_bwd, and vswin_window_msa_bwd uses
 * only qkv_w, qkv_b, proj_w, proj_b and rpb_table.                          */
typedef struct {
  float *ln1_g, *ln1_b;
  float *qkv_w, *qkv_b;
  float *proj_w, *proj_b;
  float *rpb_table;
  float *ln2_g, *ln2_b;
  float *fc1_w, *fc1_b;
  float *fc2_w, *fc2_b;
} vswin_block_grads;

/* Workspace bytes of vswin_block_bwd and vswin_window_msa_bwd for `desc`.
 * Host only.  VSWIN_ERR_UNSUPPORTED when the backward cannot serve the
 * descriptor: it needs bf16, head_dim 32, C <= 768 and the MFMA attention
 * (temporal window a multiple of 4, at most 1024 tokens per window; the -100
 * mask and key-by-key region labels as in the forward).                    */
vswin_status vswin_bwd_workspace_query(const vswin_desc* desc, size_t* block_bytes, size_t* msa_bytes);

/* Backward of vswin_block_fwd (eq. 1 differentiated; the backbone is
 * fine-tuned on video, §4.1): given dy = dL/dy, writes dx = dL/dx (desc.dtype, same shape as
 * x) and the weight gradients `g`.  The forward is recomputed inside the
 * call (x and the weights are the forward's inputs; nothing is saved
 * between calls).  Arithmetic: bf16 operands, fp32 accumulation; the
 * attention probabilities are recomputed in fp32 from the forward's
 * log-sum-exp; dS = P (dP - rowsum(dO * O)); the relative-position table
 * gradient sums dS over the pairs of every offset (deterministic: no
 * atomics on the path).  An empty batch (B = 0) sets every gradient passed
 * to zero.  dx must not alias x or dy.
 * workspace >= block_bytes of vswin_bwd_workspace_query, 256-byte aligned.  */
vswin_status vswin_block_bwd(const vswin_desc* desc, const void* x, const vswin_block_weights* w,
                             const void* dy, void* dx, const vswin_block_grads* g,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward of vswin_window_msa_fwd: given dy = dL/dy of the branch output,
 * writes dx_norm = dL/dx_norm and the qkv, proj and table gradients of `g`.
 * workspace >= msa_bytes of vswin_bwd_workspace_query.                     */
vswin_status vswin_window_msa_bwd(const vswin_desc* desc, const void* x_norm, const vswin_block_weights* w,
                                  const void* dy, void* dx_norm, const vswin_block_grads* g,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Index map of the pad + roll + partition permutation (§3.2):
 * map[w * N + n] = flat source token index b*T*H*W + (t*H + h)*W + w of
 * window slot n of window w (windows ordered (b, wt, wh, ww), slots
 * (pt, ph, pw), row-major), or -1 for a pad slot.  region (nullable) gets the
 * slot's region label 9*lt + 3*lh + lw, or 255 for a pad that forms its own
 * region.  map, region: device buffers of num_windows * N entries.           */
vswin_status vswin_index_map(const vswin_desc* desc, int32_t* map, uint8_t* region,
                             void* stream);

/* Pad + roll(-shift) + partition of x (B,T,H,W,C) into windows
 * (num_windows, N, C), pad slots zero (Video Swin Transformer, §3.2 and its
 * pseudo-code for window_msa: roll by the negated shift, pad to window
 * multiples, partition; the pad-before-roll order and end-of-axis zeros follow
 * the paper-vs-code notes, "Mask value and padding").  Windows are ordered
 * (b, wt, wh, ww) and slots (pt, ph, pw), both row-major.  x and windows are
 * device buffers of desc->dtype; windows holds num_windows * N * C elements
 * (vswin_plan_query).  Bit-exact permutation: no arithmetic on the values.
 * Argument errors (bad descriptor, null pointers) return
 * VSWIN_ERR_INVALID_ARG before anything is enqueued.                       */
vswin_status vswin_partition_fwd(const vswin_desc* desc, const void* x, void* windows,
                                 void* stream);

/* Inverse: reverse partition + roll(+shift) + crop of windows
 * (num_windows, N, C) into y (B,T,H,W,C) (Video Swin Transformer, §3.2
 * pseudo-code for window_msa: merge the windows back, roll by +shift, crop the
 * padding); with residual != NULL, y = residual + unpartitioned windows in
 * desc->dtype arithmetic rounded once (the first residual of eq. 1).  Pad
 * slots are dropped.  All pointers are device buffers of desc->dtype;
 * residual and y hold B*T*H*W*C elements.  Without a residual the result is
 * a bit-exact permutation.  Argument errors return VSWIN_ERR_INVALID_ARG
 * before anything is enqueued.                                               */
vswin_status vswin_reverse_fwd(const vswin_desc* desc, const void* windows,
                               const void* residual, void* y, void* stream);

/* LayerNorm over the last axis of `rows` rows of width C (biased variance):
 * y = (x - mean) / sqrt(var + eps) * g + b.  It is the LN of eq. 1 (Video
 * Swin Transformer, §3.1, Method step 3: pre-norm before the MSA and the
 * MLP), of patch merging (CSDN walk-through, PatchMerging: LN over the 4C
 * concatenation) and the backbone's final norm.  Statistics in fp32.  x
 * (rows * C of in_dtype), g and b (C of out_dtype), y (rows * C of out_dtype)
 * are device buffers.  rows = 0 is a no-op; C odd or outside 2..4096, eps <= 0,
 * a bad dtype or null pointers return VSWIN_ERR_INVALID_ARG before anything
 * is enqueued.                                                               */
vswin_status vswin_layernorm_fwd(int64_t rows, int32_t C, vswin_dtype in_dtype,
                                 vswin_dtype out_dtype, const void* x, const void* g,
                                 const void* b, float eps, void* y, void* stream);

/* 3D patch embedding (§3.1 step 1; the Conv3d of the mmaction2 code with
 * kernel = stride = patch):  video (B, Cin, T, H, W) -> tokens
 * (B, ceil(T/pt), ceil(H/ph), ceil(W/pw), C); each patch's values in
 * (c, kt, kh, kw) order (zero beyond the video's end) times w^T + b.
 * w is (C, Cin, pt, ph, pw), b (C) nullable.  Needs a workspace of
 * vswin_patch_embed_workspace() bytes.                                       */
size_t vswin_patch_embed_workspace(int32_t B, int32_t Cin, int32_t T, int32_t H, int32_t W,
                                   const int32_t patch[3], vswin_dtype dtype);
vswin_status vswin_patch_embed_fwd(int32_t B, int32_t Cin, int32_t T, int32_t H, int32_t W,
                                   const int32_t patch[3], int32_t C, vswin_dtype dtype,
                                   const void* video, const void* w, const void* b,
                                   void* y, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Patch merging between stages (§3.1 step 2): x (B,T,H,W,C) ->
 * y (B, T, ceil(H/2), ceil(W/2), Cout): the 2x2 spatial group concatenated in
 * (h, w) offset order (0,0), (1,0), (0,1), (1,1) (zero beyond the grid),
 * LayerNorm over 4C (g, b of 4C), then Linear(4C -> Cout) with w (Cout, 4C)
 * and b (Cout) nullable.  Workspace: vswin_patch_merge_workspace() bytes.     */
size_t vswin_patch_merge_workspace(int32_t B, int32_t T, int32_t H, int32_t W, int32_t C,
                                   vswin_dtype dtype);
vswin_status vswin_patch_merge_fwd(int32_t B, int32_t T, int32_t H, int32_t W, int32_t C,
                                   int32_t Cout, vswin_dtype dtype, const void* x,
                                   const void* ln_g, const void* ln_b, const void* w,
                                   const void* b, float eps, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Classification head (the 2D Swin page's global average pooling and linear
 * classifier, taken over the 3D grid of final tokens): logits (B, K) fp32 =
 * (mean over the L tokens of x (B, L, C), L = T' H' W', any token order)
 * times w^T + b, with w (K, C) and b (K, nullable) in `dtype` like x (bf16 or
 * fp32).  fp32 accumulation in a fixed order: repeated calls give identical
 * bits.  C a multiple of 4 (<= 4096); pointers 16-byte aligned.  Needs a
 * workspace of vswin_head_workspace() bytes (256-byte aligned).  Errors:
 * VSWIN_ERR_INVALID_ARG (sizes, dtype, NULL or misaligned pointers),
 * VSWIN_ERR_WORKSPACE (too small), VSWIN_ERR_HIP (launch).  B == 0 or
 * K == 0 does nothing.                                                       */
size_t vswin_head_workspace(int32_t B, int64_t L, int32_t C);
vswin_status vswin_head_fwd(int32_t B, int64_t L, int32_t C, int32_t K, vswin_dtype dtype,
                            const void* x, const void* w, const void* b, float* logits,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Scores of several views of each video (temporal clips x spatial crops,
 * Table 1 of the Video Swin Transformer page): probs (B, K) = the mean over
 * the V views of softmax(logits[b, v, :]); logits (B, V, K) fp32 with the
 * views of one video adjacent (a batch of B * V clips in video-major order).
 * 1 <= V <= 4096.  Errors: VSWIN_ERR_INVALID_ARG, VSWIN_ERR_HIP.              */
vswin_status vswin_multiview_average(int32_t B, int32_t V, int32_t K, const float* logits,
                                     float* probs, void* stream);

/* 2D -> 3D inflation of an image model (§3.4, initialisation from an image
 * model).  Patch kernel: w3 (C, Cin, pt, ph, pw) = the 2D kernel w2
 * (C, Cin, ph, pw) in each of the pt temporal slots, divided by pt (0.5 for
 * the pages' pt = 2; fp32 division, bf16 rounded to nearest even).  Bias
 * table: t3 ((2P-1) rows2d, heads) = the 2D table t2 (rows2d, heads),
 * rows2d = (2Mh-1)(2Mw-1), repeated once per temporal offset with the
 * temporal offset outermost, the row order of the block's own table, so every
 * frame pair gets the 2D bias (a plain copy).  Caller-owned device buffers,
 * 16-byte aligned.  Errors: VSWIN_ERR_INVALID_ARG, VSWIN_ERR_HIP.              */
vswin_status vswin_inflate_patch_embed(int32_t C, int32_t Cin, int32_t pt, int32_t ph, int32_t pw,
                                       vswin_dtype dtype, const void* w2, void* w3, void* stream);
vswin_status vswin_inflate_bias_table(int32_t rows2d, int32_t heads, int32_t P, vswin_dtype dtype,
                                      const void* t2, void* t3, void* stream);

/* Measurement helper, not part of the block: launches `blocks` workgroups of
 * 512 threads that each issue `iters` rounds of 8 independent
 * v_mfma_f32_16x16x32_bf16 per wave (16384 FLOP each), so a caller timing it
 * on `stream` gets the MFMA rate the device sustains (FLOP = blocks * 8 waves
 * * 8 * iters * 16384).  out: device buffer of blocks * 512 floats (written,
 * values meaningless).  Errors: VSWIN_ERR_INVALID_ARG for blocks < 1,
 * iters < 1 or a NULL / unaligned out; VSWIN_ERR_HIP for a launch failure.    */
vswin_status vswin_mfma_rate_probe(float* out, int32_t blocks, int32_t iters, void* stream);

/* Measurement helper, not part of the block: whether MFMA and VALU work
 * overlap on a SIMD.  `blocks` workgroups of 512 threads run `iters` rounds;
 * per round a wave issues 8 independent v_mfma_f32_16x16x32_bf16 (mode 0),
 * 8 independent v_exp_f32 + v_fma_f32 pairs (mode 1), one of the two by wave
 * parity (mode 2), or both (mode 3).  The caller times the launches: with
 * concurrent units mode 3 would take max(t0, t1), run back to back t0 + t1.
 * out: device buffer of blocks * 512 floats (values meaningless).  Errors:
 * VSWIN_ERR_INVALID_ARG (blocks, iters < 1, mode outside 0..3, NULL or
 * unaligned out), VSWIN_ERR_HIP.                                              */
vswin_status vswin_issue_probe(float* out, int32_t blocks, int32_t iters, int32_t mode, void* stream);

const char* vswin_status_string(vswin_status s);
const char* vswin_last_error(void);
int32_t vswin_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSWIN_H_ */
