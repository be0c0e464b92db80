/*
 * A plain C99 program that uses libtsel through include/tsel.h and the HIP
 * runtime's C API only (no C++, no torch): the proof that the boundary is a
 * C ABI.
 *
 *   tsel_consumer check            host-side checks, no GPU needed: version,
 *                                  validation error codes and messages
 *   tsel_consumer run IN OUT       the whole selection path on the GPU for the
 *                                  problem in file IN, results to file OUT
 *
 * File IN (little-endian): int32 magic 0x31435354 ("TSC1"), T, B, S, Hq, Hkv,
 * d, dtype, mask, emb_row_bytes; int32 cu_seqlens[B+1], cu_images[B+1],
 * img_start[S], img_hw[2S], cu_cands[S+1]; float64 keep_ratio[B]; then the
 * bytes of q [T, Hq, d], k [T, Hkv, d] (contiguous, in dtype) and the
 * embedding rows [T, emb_row_bytes].
 *
 * File OUT: float32 lse[Hq*T], float32 score[N], int32 k[B], uint8 keep[N],
 * int32 T_out, int32 token_idx[T_out], int32 spatial[3*T_out],
 * int32 cu_seqlens_out[B+1], int32 img_counts[S], int32 positions[3*T_out],
 * then the gathered embedding rows [T_out, emb_row_bytes].
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tsel.h"

#define CHECK_HIP(x)                                                           \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(3);                                                                 \
    }                                                                          \
  } while (0)

#define CHECK_TSEL(x)                                                          \
  do {                                                                         \
    int rc_ = (x);                                                             \
    if (rc_ != TSEL_OK) {                                                      \
      fprintf(stderr, "%s:%d: rc %d: %s\n", __FILE__, __LINE__, rc_, tsel_last_error()); \
      exit(4);                                                                 \
    }                                                                          \
  } while (0)

static int fail(const char *what) {
  fprintf(stderr, "check failed: %s\n", what);
  return 1;
}

/* Host-side contract: every call validates before touching the device. */
static int check(void) {
  static const int32_t cu_seqlens[3] = {0, 19, 28}, cu_images[3] = {0, 1, 2}, img_start[2] = {0, 21};
  static const int32_t img_hw[4] = {4, 4, 2, 3}, cu_cands[3] = {0, 16, 22};
  const void *fake = (const void *)(uintptr_t)4096; /* never dereferenced by validation */
  tsel_layout_t lay;
  tsel_attn_t a;
  double ratios[2] = {0.5, 0.5};
  int32_t k_h[2];
  if (tsel_version() != TSEL_VERSION) return fail("version");
  memset(&lay, 0, sizeof lay);
  lay.num_reqs = 2;
  lay.num_images = 2;
  lay.total_tokens = 28;
  lay.cu_seqlens = lay.cu_seqlens_h = cu_seqlens;
  lay.cu_images = lay.cu_images_h = cu_images;
  lay.img_start = lay.img_start_h = img_start;
  lay.img_hw = lay.img_hw_h = img_hw;
  lay.cu_cands = lay.cu_cands_h = cu_cands;
  memset(&a, 0, sizeof a);
  a.dtype = TSEL_BF16;
  a.num_heads_q = 8;
  a.num_heads_kv = 2;
  a.head_dim = 112; /* not built */
  a.q = a.k = fake;
  a.q_stride_tok = 8 * 112;
  a.q_stride_head = 112;
  a.k_stride_tok = 2 * 112;
  a.k_stride_head = 112;
  a.mask = TSEL_MASK_CAUSAL;
  if (tsel_lse(&a, &lay, (float *)(uintptr_t)4096, NULL, 0, NULL) != TSEL_EUNSUPPORTED) return fail("head_dim");
  if (strstr(tsel_last_error(), "head_dim") == NULL) return fail("head_dim message");
  if (tsel_lse(NULL, &lay, NULL, NULL, 0, NULL) != TSEL_EINVAL) return fail("null attn");
  ratios[1] = NAN;
  if (tsel_budget_topk(&lay, (const float *)fake, ratios, k_h, (uint8_t *)(uintptr_t)4096, NULL, 0, NULL) !=
      TSEL_EINVAL)
    return fail("NaN ratio");
  ratios[1] = 0.5;
  lay.max_seqlen = 18; /* the longest request has 19 tokens */
  if (tsel_budget_topk(&lay, (const float *)fake, ratios, k_h, (uint8_t *)(uintptr_t)4096, NULL, 0, NULL) !=
      TSEL_EINVAL)
    return fail("max_seqlen");
  lay.max_seqlen = 19;
  if (tsel_workspace_size(TSEL_OP_COMPACT, NULL, &lay) == (size_t)-1) return fail("compact workspace size");
  lay.cu_seqlens_h = NULL;
  if (tsel_workspace_size(TSEL_OP_COMPACT, NULL, &lay) != (size_t)-1) return fail("missing host mirror");
  printf("check ok: tsel version %d\n", tsel_version());
  return 0;
}

static void *read_exact(FILE *f, size_t n) {
  void *p = malloc(n ? n : 1);
  if (p == NULL || fread(p, 1, n, f) != n) {
    fprintf(stderr, "input file truncated\n");
    exit(2);
  }
  return p;
}

static void *to_device(const void *h, size_t n) {
  void *d = NULL;
  CHECK_HIP(hipMalloc(&d, n ? n : 16));
  if (n) CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
  return d;
}

static void write_back(FILE *f, const void *d, size_t n) {
  void *h = malloc(n ? n : 1);
  if (h == NULL) exit(2);
  if (n) CHECK_HIP(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, n, f) != n) exit(2);
  free(h);
}

static int run(const char *in_path, const char *out_path) {
  FILE *f = fopen(in_path, "rb");
  int32_t hdr[10];
  int32_t T, B, S, hq, hkv, d, dtype, mask, row_bytes, N, b, t_out;
  size_t es, ws_bytes, ws_lse, ws_col, ws_topk, ws_cmp, ws_rope;
  int32_t *cu_seqlens, *cu_images, *img_start, *img_hw, *cu_cands, *k_h;
  double *ratios;
  void *q_h, *k_hbuf, *emb_h;
  tsel_layout_t lay;
  tsel_attn_t a;
  float *lse, *score;
  uint8_t *keep;
  void *q, *k, *emb, *ws, *out_emb;
  int32_t *tok, *spatial, *cu_out, *img_counts, *pos;
  hipStream_t stream;
  FILE *o;

  if (f == NULL) return fail("open input");
  if (fread(hdr, sizeof(int32_t), 10, f) != 10 || hdr[0] != 0x31435354) return fail("input header");
  T = hdr[1], B = hdr[2], S = hdr[3], hq = hdr[4], hkv = hdr[5], d = hdr[6];
  dtype = hdr[7], mask = hdr[8], row_bytes = hdr[9];
  es = dtype == TSEL_F32 ? 4 : dtype == TSEL_FP8_E4M3 ? 1 : 2;
  cu_seqlens = read_exact(f, sizeof(int32_t) * (B + 1));
  cu_images = read_exact(f, sizeof(int32_t) * (B + 1));
  img_start = read_exact(f, sizeof(int32_t) * S);
  img_hw = read_exact(f, sizeof(int32_t) * 2 * S);
  cu_cands = read_exact(f, sizeof(int32_t) * (S + 1));
  ratios = read_exact(f, sizeof(double) * B);
  q_h = read_exact(f, (size_t)T * hq * d * es);
  k_hbuf = read_exact(f, (size_t)T * hkv * d * es);
  emb_h = read_exact(f, (size_t)T * row_bytes);
  fclose(f);
  N = cu_cands[S];

  CHECK_HIP(hipStreamCreate(&stream));
  memset(&lay, 0, sizeof lay);
  lay.num_reqs = B;
  lay.num_images = S;
  lay.total_tokens = T;
  for (b = 0; b < B; ++b)
    if (cu_seqlens[b + 1] - cu_seqlens[b] > lay.max_seqlen) lay.max_seqlen = cu_seqlens[b + 1] - cu_seqlens[b];
  lay.cu_seqlens = to_device(cu_seqlens, sizeof(int32_t) * (B + 1));
  lay.cu_images = to_device(cu_images, sizeof(int32_t) * (B + 1));
  lay.img_start = to_device(img_start, sizeof(int32_t) * S);
  lay.img_hw = to_device(img_hw, sizeof(int32_t) * 2 * S);
  lay.cu_cands = to_device(cu_cands, sizeof(int32_t) * (S + 1));
  lay.cu_seqlens_h = cu_seqlens;
  lay.cu_images_h = cu_images;
  lay.img_start_h = img_start;
  lay.img_hw_h = img_hw;
  lay.cu_cands_h = cu_cands;

  q = to_device(q_h, (size_t)T * hq * d * es);
  k = to_device(k_hbuf, (size_t)T * hkv * d * es);
  emb = to_device(emb_h, (size_t)T * row_bytes);
  memset(&a, 0, sizeof a);
  a.dtype = (tsel_dtype_t)dtype;
  a.num_heads_q = hq;
  a.num_heads_kv = hkv;
  a.head_dim = d;
  a.q = q;
  a.q_stride_tok = (int64_t)hq * d;
  a.q_stride_head = d;
  a.k = k;
  a.k_stride_tok = (int64_t)hkv * d;
  a.k_stride_head = d;
  a.mask = (tsel_mask_t)mask;
  a.softmax_scale = 0.0f;

  ws_lse = tsel_workspace_size(TSEL_OP_LSE, &a, &lay);
  ws_col = tsel_workspace_size(TSEL_OP_COLSCORE, &a, &lay);
  ws_topk = tsel_workspace_size(TSEL_OP_TOPK, NULL, &lay);
  ws_cmp = tsel_workspace_size(TSEL_OP_COMPACT, NULL, &lay);
  ws_rope = tsel_workspace_size(TSEL_OP_MROPE, NULL, &lay);
  if (ws_lse == (size_t)-1 || ws_col == (size_t)-1 || ws_topk == (size_t)-1 || ws_cmp == (size_t)-1 ||
      ws_rope == (size_t)-1)
    return fail(tsel_last_error());
  /* One buffer serves every call: the calls run one after another on one stream. */
  ws_bytes = ws_col > ws_cmp ? ws_col : ws_cmp;
  ws_bytes = ws_bytes > ws_rope ? ws_bytes : ws_rope;
  ws_bytes = ws_bytes > ws_lse ? ws_bytes : ws_lse;
  ws_bytes = ws_bytes > ws_topk ? ws_bytes : ws_topk;
  CHECK_HIP(hipMalloc(&ws, ws_bytes ? ws_bytes : 16));
  CHECK_HIP(hipMalloc((void **)&lse, sizeof(float) * (size_t)hq * T + 16));
  CHECK_HIP(hipMalloc((void **)&score, sizeof(float) * (size_t)N + 16));
  CHECK_HIP(hipMalloc((void **)&keep, (size_t)N + 16));

  /* The path: LSE -> column score -> budget -> compaction -> rotary positions. */
  CHECK_TSEL(tsel_lse(&a, &lay, lse, ws, ws_bytes, stream));
  CHECK_TSEL(tsel_colscore(&a, &lay, lse, score, ws, ws_bytes, stream));
  k_h = malloc(sizeof(int32_t) * B);
  CHECK_TSEL(tsel_budget_topk(&lay, score, ratios, k_h, keep, ws, ws_bytes, stream));
  t_out = 0;
  for (b = 0; b < B; ++b)
    t_out += (cu_seqlens[b + 1] - cu_seqlens[b]) - (cu_cands[cu_images[b + 1]] - cu_cands[cu_images[b]]) + k_h[b];
  CHECK_HIP(hipMalloc((void **)&tok, sizeof(int32_t) * (size_t)t_out + 16));
  CHECK_HIP(hipMalloc((void **)&spatial, sizeof(int32_t) * 3 * (size_t)t_out + 16));
  CHECK_HIP(hipMalloc((void **)&cu_out, sizeof(int32_t) * (size_t)(B + 1)));
  CHECK_HIP(hipMalloc((void **)&img_counts, sizeof(int32_t) * (size_t)S + 16));
  CHECK_HIP(hipMalloc((void **)&pos, sizeof(int32_t) * 3 * (size_t)t_out + 16));
  CHECK_HIP(hipMalloc(&out_emb, (size_t)t_out * row_bytes + 16));
  CHECK_TSEL(tsel_compact(&lay, keep, emb, row_bytes, row_bytes, t_out, out_emb, row_bytes, tok, spatial, cu_out,
                          img_counts, ws, ws_bytes, stream));
  CHECK_TSEL(tsel_mrope_positions(&lay, tok, spatial, t_out, pos, ws, ws_bytes, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  o = fopen(out_path, "wb");
  if (o == NULL) return fail("open output");
  write_back(o, lse, sizeof(float) * (size_t)hq * T);
  write_back(o, score, sizeof(float) * (size_t)N);
  if (fwrite(k_h, sizeof(int32_t), (size_t)B, o) != (size_t)B) return fail("write");
  write_back(o, keep, (size_t)N);
  if (fwrite(&t_out, sizeof(int32_t), 1, o) != 1) return fail("write");
  write_back(o, tok, sizeof(int32_t) * (size_t)t_out);
  write_back(o, spatial, sizeof(int32_t) * 3 * (size_t)t_out);
  write_back(o, cu_out, sizeof(int32_t) * (size_t)(B + 1));
  write_back(o, img_counts, sizeof(int32_t) * (size_t)S);
  write_back(o, pos, sizeof(int32_t) * 3 * (size_t)t_out);
  write_back(o, out_emb, (size_t)t_out * row_bytes);
  fclose(o);
  printf("run ok: T=%d N=%d kept=%d T_out=%d\n", T, N, t_out - (T - N), t_out);
  return 0;
}

int main(int argc, char **argv) {
  if (argc == 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc == 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
  fprintf(stderr, "usage: %s check | run IN OUT\n", argv[0]);
  return 2;
}
