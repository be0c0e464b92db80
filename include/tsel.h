/*
 * tsel.h -- attention-score visual-token selection on AMD Instinct MI355X (gfx950).
 *
 * The selection step scores every vision token by the softmax attention it
 * receives in one attention layer, keeps a global top-k of those scores over
 * all images of a request, and compacts the kept tokens.  Four calls make up
 * the path:
 *
 *   tsel_lse          per-row softmax log-sum-exp over all visible keys
 *   tsel_colscore     tile-by-tile recomputation of P = exp(s - LSE), reduced
 *                     down the candidate columns, averaged over heads and rows
 *   tsel_budget_topk  one top-k per request pool, k = floor(r * N + 1e-6)
 *   tsel_compact      stable compaction and gather of the kept tokens
 *
 * tsel_budget_mass replaces the fixed ratio of tsel_budget_topk with a budget
 * read from the scores themselves, and two calls sit on either side of the
 * path:
 *
 *   tsel_attention_fwd    the layer's attention forward, which yields the LSE
 *                         the selection can reuse instead of tsel_lse
 *   tsel_mrope_positions  rotary positions of the compacted sequence
 *
 * Sources: LiteVLM (arXiv 2506.07416) review, section 3.2 (token selection
 * module) and its formula section (score of a vision token = the attention it
 * receives; softmax(QK^T / sqrt(d))); REDtech "vision token compression + SERE"
 * article, sections 3.1-3.2 (dominant tokens found by the average attention a
 * token receives at a chosen layer, one global candidate pool per request,
 * reuse of FlashAttention's softmax LSE, column-wise reduction without
 * materialising the attention matrix, updated lengths / image boundaries /
 * original spatial indices after pruning).
 *
 * Conventions for every call
 * --------------------------
 * - Pointers without an _h suffix are DEVICE pointers; _h pointers are HOST
 *   pointers read synchronously during the call.  The caller owns every
 *   buffer; the library allocates no device memory.  Scratch space comes from
 *   a caller workspace whose size tsel_workspace_size() reports.
 * - Every call validates its host-side arguments first.  On failure it
 *   returns a negative TSEL_E* code before enqueuing anything, and
 *   tsel_last_error() (thread-local) describes the problem.  On success it
 *   returns TSEL_OK after enqueuing its kernels on `stream` (a hipStream_t;
 *   NULL is the null stream).  No call synchronises the device or copies
 *   device memory to the host; calls enqueue kernel launches only (no
 *   allocation, copy or memset), so a caller may capture them in a HIP graph
 *   and replay it while the layout, sizes and buffers stay the same.
 * - Device array contents are trusted to equal their host mirrors; with
 *   TSEL_DEBUG=1 in the environment every call first checks that they do
 *   (a synchronous device-to-host copy, for debugging) and returns
 *   TSEL_EINVAL when they differ.
 * - Results are deterministic: no floating-point atomics; every reduction
 *   runs in a fixed order.
 */
#ifndef TSEL_H_
#define TSEL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSEL_VERSION 4

#define TSEL_OK 0
#define TSEL_EINVAL (-1)      /* bad pointer, size, offset, ratio or layout        */
#define TSEL_EUNSUPPORTED (-2) /* dtype or head_dim outside what is built          */
#define TSEL_EWORKSPACE (-3)  /* workspace missing or smaller than required        */
#define TSEL_EHIP (-4)        /* a HIP launch reported an error                    */

/* Q/K element types.  TSEL_FP8_E4M3 is the OCP 8-bit float with 4 exponent
 * bits (bias 7), 3 mantissa bits, subnormals, no infinities and NaN =
 * S.1111.111 (largest finite 448); the low-precision Q/K scoring LiteVLM
 * deploys (LiteVLM review, sections 3.2 and 5).  Per-tensor dequantisation
 * factors of q and k are folded into softmax_scale by the caller. */
typedef enum { TSEL_F32 = 0, TSEL_F16 = 1, TSEL_BF16 = 2, TSEL_FP8_E4M3 = 3 } tsel_dtype_t;

/* Which keys a row sees (the LiteVLM first decoder layer is causal; the
 * REDtech ViT-layer statistics use per-image bidirectional attention):
 *   FULL       every token of the same request,
 *   CAUSAL     tokens j <= i of the same request (diagonal included),
 *   BLOCKDIAG  tokens of the same image; every token must belong to an image. */
typedef enum { TSEL_MASK_FULL = 0, TSEL_MASK_CAUSAL = 1, TSEL_MASK_BLOCKDIAG = 2 } tsel_mask_t;

/* Token layout of one batch.  Requests are packed back to back.  Images are
 * disjoint token ranges [img_start[s], img_start[s] + rows*cols), sorted by
 * start, each inside its request; request b owns images
 * cu_images[b] .. cu_images[b+1]-1.  Candidates (the vision tokens that
 * compete for the budget) are numbered in token order: image s holds
 * candidates cu_cands[s] .. cu_cands[s+1]-1, cu_cands[s+1]-cu_cands[s] =
 * rows*cols.  Every array is given twice: on the device and on the host. */
typedef struct {
  int32_t num_reqs;               /* B >= 1                                         */
  int32_t num_images;             /* S >= 0                                         */
  int32_t total_tokens;           /* T = cu_seqlens[B]                              */
  int32_t max_seqlen;             /* longest request, max_b (cu_seqlens[b+1] -
                                     cu_seqlens[b]); checked against the host mirror
                                     when nonzero (TSEL_EINVAL if it differs);
                                     0 = not given                                  */
  const int32_t *cu_seqlens;      /* [B+1] device                                   */
  const int32_t *cu_images;       /* [B+1] device                                   */
  const int32_t *img_start;       /* [S]   device                                   */
  const int32_t *img_hw;          /* [2S]  device, (rows, cols) per image           */
  const int32_t *cu_cands;        /* [S+1] device                                   */
  const int32_t *cu_seqlens_h;    /* host mirrors of the five arrays above          */
  const int32_t *cu_images_h;
  const int32_t *img_start_h;
  const int32_t *img_hw_h;
  const int32_t *cu_cands_h;
} tsel_layout_t;

/* One attention layer's queries and keys.  q is [T, Hq, head_dim] and k is
 * [T, Hkv, head_dim] with arbitrary token and head strides (in ELEMENTS) and a
 * contiguous last dimension.  Query head h reads KV head h / (Hq / Hkv).
 * Requirements: Hq % Hkv == 0; head_dim in {64, 72, 80, 96, 128} ({64, 128}
 * for TSEL_FP8_E4M3; 72 runs as 80 with zero padding); q and k 16-byte
 * aligned; both strides multiples of 16 bytes.  softmax_scale <= 0 selects
 * 1/sqrt(head_dim) (LiteVLM review, formula section). */
typedef struct {
  tsel_dtype_t dtype;
  int32_t num_heads_q;
  int32_t num_heads_kv;
  int32_t head_dim;
  const void *q;
  int64_t q_stride_tok, q_stride_head;
  const void *k;
  int64_t k_stride_tok, k_stride_head;
  tsel_mask_t mask;
  float softmax_scale;
} tsel_attn_t;

/* Workspace queries (op codes for tsel_workspace_size). */
#define TSEL_OP_LSE 0
#define TSEL_OP_COLSCORE 1
#define TSEL_OP_TOPK 2
#define TSEL_OP_COMPACT 3
#define TSEL_OP_MROPE 4

/* Bytes of workspace `op` needs for this problem (0 if none; the caller may
 * then pass NULL).  `attn` may be NULL for TSEL_OP_TOPK / TSEL_OP_COMPACT /
 * TSEL_OP_MROPE.
 * Returns (size_t)-1 when the arguments fail validation. */
size_t tsel_workspace_size(int op, const tsel_attn_t *attn, const tsel_layout_t *layout);

/* Per-row softmax normaliser (natural log) over every key the row sees, text
 * keys included -- the LSE a FlashAttention forward returns (REDtech article,
 * section 3.2):  lse[h*T + i] = log sum_{j visible(i)} exp(scale * q_{i,h} . k_{j,g(h)}).
 * Output: lse, fp32 [Hq, T] contiguous, every entry written.  Arithmetic:
 * MFMA products in fp32, exp2/log2 in fp32.  Non-finite inputs give a
 * non-finite LSE for the rows that see them.
 * Workspace: tsel_workspace_size(TSEL_OP_LSE) bytes, 4-byte aligned.  It is 0
 * for grids that fill the GPU; a small grid (a short causal request, few
 * heads) splits each row's keys into ranges whose partial log-sum-exps the
 * workspace holds until a merge pass combines them in a fixed order. */
int tsel_lse(const tsel_attn_t *attn, const tsel_layout_t *layout, float *lse, void *workspace,
             size_t workspace_bytes, void *stream);

/* Importance score of every candidate (LiteVLM review, formula section: the
 * attention a vision token receives; REDtech article, section 3.2: the
 * average attention it receives, computed tile by tile from the reused LSE
 * without writing the attention matrix out):
 *   score[c] = 1/(Hq * n_b) * sum_h sum_{i in request b, i sees c} exp(scale * q_{i,h}.k_{c,g(h)} - lse[h*T+i])
 * where n_b is the length of c's request (all rows of the request count,
 * masked pairs contribute zero).  lse: fp32 [Hq, T], either from tsel_lse or
 * supplied by the caller (e.g. a FlashAttention forward).  Output: score,
 * fp32 [N], N = cu_cands[S].  Workspace: tsel_workspace_size(TSEL_OP_COLSCORE). */
int tsel_colscore(const tsel_attn_t *attn, const tsel_layout_t *layout, const float *lse,
                  float *score, void *workspace, size_t workspace_bytes, void *stream);

/* tsel_colscore for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, with the column-score partials in a
 * static device buffer of the library (16 MiB, one per GPU, held until the
 * process ends) instead of a caller workspace.  The call allocates and frees
 * nothing.  Problems whose partials need more than 16 MiB
 * (tsel_workspace_size(TSEL_OP_COLSCORE) > 16 MiB) return TSEL_EWORKSPACE
 * before enqueuing anything.  Every call on one GPU shares that GPU's buffer:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * give wrong scores; calls ordered on one stream are safe.  Arguments, output
 * and errors otherwise as tsel_colscore. */
int tsel_colscore_noalloc(const tsel_attn_t *attn, const tsel_layout_t *layout, const float *lse,
                          float *score, void *stream);

/* Global budget per request (REDtech article, sections 3.1-3.2: all images of
 * a request compete in one pool; LiteVLM review, section 3.2 / section 5 table:
 * keep ratio r).  For pool b with N_b candidates,
 *   k_b = clamp(floor(clamp(r_b, 0, 1) * N_b + 1e-6), 0, N_b)      (binary64)
 * and the k_b candidates with the largest scores are kept; equal scores go to
 * the lower candidate index; NaN and +-inf scores rank as -inf.
 * keep_ratio_h: host [B]; NaN is TSEL_EINVAL.  k_h: host [B], written
 * synchronously.  keep: device uint8 [N], 1 = kept.
 * Workspace: tsel_workspace_size(TSEL_OP_TOPK) bytes, 4-byte aligned (0 when
 * every pool fits one workgroup's registers). */
int tsel_budget_topk(const tsel_layout_t *layout, const float *score, const double *keep_ratio_h,
                     int32_t *k_h, uint8_t *keep, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Input-dependent budget (the REDtech article, section 6.2, names choosing
 * the compression rate from the input as the next step and gives no rule;
 * section 5.2 prunes less on detail-dense inputs, and section 3.1's premise is
 * that a few dominant tokens gather most of the attention; this call is this
 * library's reading).  Scores are read as attention mass, in integer units of
 * 2^-32: m = floor(min(s, 1) * 2^32) for a finite s > 0, else 0.  For pool b
 * with total mass M_b (exact 64-bit sum),
 *   target = min(M_b, ceil((tau_b * M_b) * (1 - 1e-12)))         (binary64)
 *   k*_b   = fewest candidates, taken in the tsel_budget_topk order, whose
 *            mass reaches target (0 when target is 0)
 *   k_b    = clamp(k*_b, floor(r_min_b * N_b + 1e-6), floor(r_max_b * N_b + 1e-6))
 * and the k_b candidates are kept exactly as tsel_budget_topk keeps them.  A
 * pool whose attention concentrates on a few tokens keeps few; a diffuse one
 * keeps many.  tau_h, r_min_h, r_max_h: host [B], clamped to [0, 1]; NaN or
 * r_min > r_max is TSEL_EINVAL.  k: device int32 [B], written on `stream`
 * (tsel_compact needs the kept counts only through `keep`; copy k to the host
 * to size its outputs exactly).  keep: device uint8 [N].  No workspace. */
int tsel_budget_mass(const tsel_layout_t *layout, const float *score, const double *tau_h,
                     const double *r_min_h, const double *r_max_h, int32_t *k, uint8_t *keep,
                     void *stream);

/* Stable compaction of every request (REDtech article, section 3.2: new
 * multimodal lengths, image boundaries and original spatial indices).  A
 * token stays iff it is not a candidate (text always stays) or its keep flag
 * is set; order is preserved.  With T_out = sum_b (n_b - N_b + k_b):
 *   out_token_idx  int32 [T_out]     original packed token index
 *   out_spatial    int32 [T_out, 3]  (image, row, col), (-1, -1, -1) for text
 *   out_cu_seqlens int32 [B+1]       new packed offsets
 *   out_img_counts int32 [S]         kept candidates per image
 *   out_emb        [T_out] rows of emb_row_bytes bytes, copied bit-exact from
 *                  emb (row t at emb + t*emb_stride bytes) to out_emb (row p at
 *                  out_emb + p*out_emb_stride bytes); emb may be NULL to skip.
 * out_capacity is the number of rows the output arrays hold; rows past it are
 * not written (pass T_out computed from k_h).  Any output pointer but
 * out_token_idx may be NULL.  Workspace: tsel_workspace_size(TSEL_OP_COMPACT). */
int tsel_compact(const tsel_layout_t *layout, const uint8_t *keep, const void *emb,
                 int64_t emb_stride, int64_t emb_row_bytes, int32_t out_capacity, void *out_emb,
                 int64_t out_emb_stride, int32_t *out_token_idx, int32_t *out_spatial,
                 int32_t *out_cu_seqlens, int32_t *out_img_counts, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Attention forward of the layer whose softmax normaliser the selection
 * reuses (REDtech article, section 3.2: the FlashAttention pass already
 * produces the LSE): for every query head h and row i,
 *   out[i, h, :] = sum_j softmax_j(scale * q_{i,h} . k_{j,g(h)}) v[j, g(h), :]
 * over the row's visible keys (the masks and segments of tsel_lse), and
 * lse[h, i] exactly as tsel_lse computes it.  bf16 or f16 inputs only
 * (TSEL_EUNSUPPORTED otherwise); v is [T, Hkv, head_dim] in the same type,
 * 16-byte aligned, strides (elements) multiples of 16 bytes; the token strides
 * of k and v must be at least head_dim (rows that do not overlap in memory;
 * TSEL_EUNSUPPORTED otherwise); out is
 * [T, Hq, head_dim] in the same type, 8-byte aligned, strides multiples of
 * 8 bytes; lse fp32 [Hq, T].  No workspace. */
int tsel_attention_fwd(const tsel_attn_t *attn, const tsel_layout_t *layout, const void *v,
                       int64_t v_stride_tok, int64_t v_stride_head, void *out, int64_t out_stride_tok,
                       int64_t out_stride_head, float *lse, void *stream);

/* Rotary position ids of the compacted sequence, for a prefill that takes it
 * (REDtech article, section 3.2: the mRoPE positions are updated together
 * with lengths, image boundaries and spatial indices so the shorter sequence
 * enters prefill unchanged otherwise).  The pages name the update but not the
 * rule; the reading taken is that every kept token keeps the position it had
 * in its full request under the multimodal rotary scheme of the Qwen-VL
 * models the article serves: a running index starts at 0 in every request,
 * a text token gets (i, i, i) and advances it by 1, an image of rows x cols
 * whose first token meets index i gives token (row, col) the position
 * (i, i + row, i + col) and advances the index by max(rows, cols).
 *   out_token_idx, out_spatial: tsel_compact's outputs for this layout (the
 *                  first n_out rows are read);
 *   out_pos        int32 [n_out, 3] (t, h, w); a row whose token index is
 *                  outside [0, T) gets (-1, -1, -1).
 * Workspace: tsel_workspace_size(TSEL_OP_MROPE) bytes (one int32 per image). */
int tsel_mrope_positions(const tsel_layout_t *layout, const int32_t *out_token_idx,
                         const int32_t *out_spatial, int32_t n_out, int32_t *out_pos,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Description of the last error on this thread ("" if none). */
const char *tsel_last_error(void);

/* TSEL_VERSION of the built library. */
int tsel_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TSEL_H_ */
