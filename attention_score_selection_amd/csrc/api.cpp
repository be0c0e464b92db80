// C-ABI entry points: host-side validation, launch planning and dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "internal.h"

namespace tsel {

static thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

void clear_error() { g_err.clear(); }

static int elem_size(int dt) { return dt == TSEL_F32 ? 4 : dt == TSEL_FP8_E4M3 ? 1 : 2; }

// The ABI's enum fields hold whatever int the caller stored; reading them as
// the enum type is undefined for values outside the enumerators, so they are
// read as integers.
static int dtype_of(const tsel_attn_t *a) {
  int32_t v;
  static_assert(sizeof(a->dtype) == sizeof(v), "enum fields are 32-bit");
  memcpy(&v, &a->dtype, sizeof v);
  return v;
}
static int mask_of(const tsel_attn_t *a) {
  int32_t v;
  static_assert(sizeof(a->mask) == sizeof(v), "enum fields are 32-bit");
  memcpy(&v, &a->mask, sizeof v);
  return v;
}

// With TSEL_DEBUG=1 in the environment, every call also checks that the
// device layout arrays equal their host mirrors, through a synchronous
// device-to-host copy (debugging only: otherwise the device arrays are
// trusted and no call reads device memory back).
static int check_device_mirrors(const tsel_layout_t *l) {
  const char *dbg = getenv("TSEL_DEBUG");
  if (dbg == nullptr || dbg[0] != '1') return TSEL_OK;
  const size_t B = (size_t)l->num_reqs, S = (size_t)l->num_images;
  const struct {
    const int32_t *d, *h;
    size_t n;
    const char *name;
  } arr[] = {{l->cu_seqlens, l->cu_seqlens_h, B + 1, "cu_seqlens"},
             {l->cu_images, l->cu_images_h, B + 1, "cu_images"},
             {l->img_start, l->img_start_h, S, "img_start"},
             {l->img_hw, l->img_hw_h, 2 * S, "img_hw"},
             {l->cu_cands, l->cu_cands_h, S + 1, "cu_cands"}};
  std::vector<int32_t> tmp;
  for (const auto &x : arr) {
    if (x.n == 0) continue;
    tmp.resize(x.n);
    const hipError_t e = hipMemcpy(tmp.data(), x.d, x.n * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(TSEL_EHIP, "TSEL_DEBUG: reading device %s: %s", x.name, hipGetErrorString(e));
    for (size_t i = 0; i < x.n; ++i)
      if (tmp[i] != x.h[i])
        return fail(TSEL_EINVAL, "TSEL_DEBUG: device %s[%zu] = %d differs from its host mirror (%d)", x.name, i,
                    tmp[i], x.h[i]);
  }
  return TSEL_OK;
}

static int check_layout(const tsel_layout_t *l) {
  if (l == nullptr) return fail(TSEL_EINVAL, "layout is NULL");
  const int B = l->num_reqs, S = l->num_images, T = l->total_tokens;
  if (B < 1) return fail(TSEL_EINVAL, "num_reqs must be >= 1 (got %d)", B);
  if (S < 0 || T < 0) return fail(TSEL_EINVAL, "num_images and total_tokens must be >= 0");
  if (!l->cu_seqlens_h || !l->cu_images_h || !l->cu_cands_h)
    return fail(TSEL_EINVAL, "host layout arrays cu_seqlens_h/cu_images_h/cu_cands_h are required");
  if (!l->cu_seqlens || !l->cu_images || !l->cu_cands)
    return fail(TSEL_EINVAL, "device layout arrays cu_seqlens/cu_images/cu_cands are required");
  if (S > 0 && (!l->img_start_h || !l->img_hw_h || !l->img_start || !l->img_hw))
    return fail(TSEL_EINVAL, "img_start/img_hw (host and device) are required when num_images > 0");
  const int32_t *cu = l->cu_seqlens_h, *ci = l->cu_images_h, *cc = l->cu_cands_h;
  if (cu[0] != 0 || cu[B] != T) return fail(TSEL_EINVAL, "cu_seqlens must run from 0 to total_tokens");
  if (l->max_seqlen != 0) {
    int32_t longest = 0;
    for (int b = 0; b < B; ++b) longest = std::max(longest, cu[b + 1] - cu[b]);
    if (l->max_seqlen != longest)
      return fail(TSEL_EINVAL, "max_seqlen is %d but the longest request has %d tokens", l->max_seqlen, longest);
  }
  if (ci[0] != 0 || ci[B] != S) return fail(TSEL_EINVAL, "cu_images must run from 0 to num_images");
  if (cc[0] != 0) return fail(TSEL_EINVAL, "cu_cands[0] must be 0");
  for (int b = 0; b < B; ++b) {
    if (cu[b + 1] < cu[b]) return fail(TSEL_EINVAL, "cu_seqlens decreases at request %d", b);
    if (ci[b + 1] < ci[b]) return fail(TSEL_EINVAL, "cu_images decreases at request %d", b);
    int prev_end = cu[b];
    for (int s = ci[b]; s < ci[b + 1]; ++s) {
      const long long h = l->img_hw_h[2 * s], w = l->img_hw_h[2 * s + 1];
      if (h <= 0 || w <= 0) return fail(TSEL_EINVAL, "image %d has an empty grid", s);
      const long long start = l->img_start_h[s], end = start + h * w;
      if (start < prev_end || end > cu[b + 1])
        return fail(TSEL_EINVAL, "image %d is not sorted, disjoint and inside request %d", s, b);
      if ((long long)cc[s + 1] - cc[s] != h * w)
        return fail(TSEL_EINVAL, "cu_cands[%d+1]-cu_cands[%d] != rows*cols", s, s);
      prev_end = (int)end;
    }
  }
  return check_device_mirrors(l);
}

static int check_attn(const tsel_attn_t *a, const tsel_layout_t *l) {
  if (a == nullptr) return fail(TSEL_EINVAL, "attn is NULL");
  if (dtype_of(a) != TSEL_F32 && dtype_of(a) != TSEL_F16 && dtype_of(a) != TSEL_BF16 &&
      dtype_of(a) != TSEL_FP8_E4M3)
    return fail(TSEL_EUNSUPPORTED, "dtype %d is not supported", dtype_of(a));
  if (a->head_dim != 64 && a->head_dim != 72 && a->head_dim != 80 && a->head_dim != 96 && a->head_dim != 128)
    return fail(TSEL_EUNSUPPORTED, "head_dim %d is not one of 64, 72, 80, 96, 128", a->head_dim);
  if (dtype_of(a) == TSEL_FP8_E4M3 && a->head_dim != 64 && a->head_dim != 128)
    return fail(TSEL_EUNSUPPORTED, "fp8 inputs need head_dim 64 or 128 (got %d)", a->head_dim);
  if (a->num_heads_q < 1 || a->num_heads_kv < 1 || a->num_heads_q % a->num_heads_kv != 0)
    return fail(TSEL_EINVAL, "num_heads_q (%d) must be a positive multiple of num_heads_kv (%d)",
                a->num_heads_q, a->num_heads_kv);
  if (mask_of(a) != TSEL_MASK_FULL && mask_of(a) != TSEL_MASK_CAUSAL && mask_of(a) != TSEL_MASK_BLOCKDIAG)
    return fail(TSEL_EINVAL, "mask %d is not valid", mask_of(a));
  if (!isfinite(a->softmax_scale)) return fail(TSEL_EINVAL, "softmax_scale is not finite");
  const int es = elem_size(dtype_of(a));
  if (l->total_tokens > 0) {
    if (a->q == nullptr || a->k == nullptr) return fail(TSEL_EINVAL, "q and k are required");
    if (((uintptr_t)a->q | (uintptr_t)a->k) & 15) return fail(TSEL_EINVAL, "q and k must be 16-byte aligned");
  }
  const long long st[4] = {a->q_stride_tok, a->q_stride_head, a->k_stride_tok, a->k_stride_head};
  for (long long s : st)
    if (s <= 0 || (s * es) % 16 != 0)
      return fail(TSEL_EINVAL, "q/k strides must be positive and multiples of 16 bytes");
  if (mask_of(a) == TSEL_MASK_BLOCKDIAG) {
    const long long n = l->cu_cands_h[l->num_images];
    if (n != l->total_tokens)
      return fail(TSEL_EINVAL, "BLOCKDIAG needs every token inside an image (%lld of %d are)", n,
                  l->total_tokens);
  }
  return TSEL_OK;
}

// The kernels address each streamed 32-row tile (and a tile's LSE values)
// with 32-bit byte offsets from a per-tile base; those offsets must stay below
// kBufferLimit.
static int check_offsets(const tsel_attn_t *a, const tsel_layout_t *l, int F) {
  const long long es = elem_size(dtype_of(a));
  const long long k_span = 32LL * a->k_stride_tok * es;
  const long long q_span = ((32LL / F) * a->q_stride_tok + (long long)F * a->q_stride_head) * es;
  const long long l_span = ((long long)F * l->total_tokens + 32) * 4;
  if (k_span >= kBufferLimit || q_span >= kBufferLimit || l_span >= kBufferLimit)
    return fail(TSEL_EUNSUPPORTED, "strides too large: a 32-row tile spans 2 GiB or more");
  return TSEL_OK;
}

static void plan_common(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p) {
  const int hg = a->num_heads_q / a->num_heads_kv;
  int F = 1;
  while (F < 16 && hg % (F * 2) == 0) F *= 2;
  p->dtype = dtype_of(a);
  p->D = a->head_dim;
  p->F = F;
  p->nhb = a->num_heads_q / F;
  p->segkind = (mask_of(a) == TSEL_MASK_BLOCKDIAG) ? SEG_IMG : SEG_REQ;
  p->nseg = (p->segkind == SEG_IMG) ? l->num_images : l->num_reqs;
}

static void seg_sizes(const tsel_layout_t *l, int kind, int a, long long &n, long long &nc) {
  if (kind == SEG_REQ) {
    n = l->cu_seqlens_h[a + 1] - l->cu_seqlens_h[a];
    nc = l->cu_cands_h[l->cu_images_h[a + 1]] - l->cu_cands_h[l->cu_images_h[a]];
  } else {
    n = (long long)l->img_hw_h[2 * a] * l->img_hw_h[2 * a + 1];
    nc = n;
  }
}

// Row blocks of 4 waves x NG resident 32-row groups.  A grid of at least 512
// jobs (two workgroups per CU) runs as it is.  A smaller one (a short causal
// request, a few heads) takes one group per wave and splits every row
// block's keys into ranges of KS keys whose partial log-sum-exps a merge pass
// combines: the largest KS in 2048 .. 256 that gives 1024 jobs with keys
// (measured on the 3214-token, 16-head layer: 47 us with 512-key splits,
// 53-62 us with 256 or 1024, 63 us unsplit, 111 us unsplit with three groups
// per wave).  The partials take Hq * T * (splits of the longest segment)
// floats of workspace.
int plan_lse(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p) {
  plan_common(a, l, p);
  if (int rc = check_offsets(a, l, p->F)) return rc;
  const bool causal = mask_of(a) == TSEL_MASK_CAUSAL;
  // all: jobs launched; real: jobs that see at least one key.
  auto count = [&](int ng, int KS, long long &all, long long &real, long long &nmax) {
    const int TB = 4 * ng * 32 / p->F;
    all = real = nmax = 0;
    for (int s = 0; s < p->nseg; ++s) {
      long long n, nc;
      seg_sizes(l, p->segkind, s, n, nc);
      nmax = std::max(nmax, n);
      const long long nrb = (n + TB - 1) / TB, nks = KS ? (n + KS - 1) / KS : 1;
      all += nrb * nks;
      if (KS && causal) {
        for (long long rb = 0; rb < nrb; ++rb) real += (std::min((rb + 1) * TB, n) + KS - 1) / KS;
      } else {
        real += nrb * nks;
      }
    }
    all *= p->nhb;
    real *= p->nhb;
  };
  auto choose = [&](int ng, int KS) {
    long long all, real, nmax;
    count(ng, KS, all, real, nmax);
    p->NT = ng;
    p->TB = 4 * ng * 32 / p->F;
    p->KS = KS;
    p->ksmax = KS ? (int)((nmax + KS - 1) / KS) : 0;
    p->total_jobs = all;
    p->jobs_per_hb = all / p->nhb;
  };
  const int ng_max = lse_groups(dtype_of(a), a->head_dim);
  long long all, real, nmax;
  count(ng_max, 0, all, real, nmax);
  if (all >= 512) {
    choose(ng_max, 0);
  } else {
    // One group per wave (short jobs, more waves resident to cover latency)
    // and the largest split that gives 1024 jobs with keys; failing that, the
    // split with the most such jobs (no split when none divides a segment).
    const int splits[4] = {2048, 1024, 512, 256};
    int pick = 0;
    long long best = -1;
    for (int KS : splits) {
      count(1, KS, all, real, nmax);
      if (real >= 1024) {
        pick = KS;
        break;
      }
      if (real > best) {
        best = real;
        pick = KS;
      }
    }
    count(1, pick, all, real, nmax);
    choose(1, nmax > pick ? pick : 0);
  }
  p->KB = p->RC = p->RCF = p->RCmax = 0;
  p->partial_bytes = p->KS ? (size_t)a->num_heads_q * l->total_tokens * p->ksmax * sizeof(float) : 0;
  if (p->total_jobs > (1LL << 30)) return fail(TSEL_EINVAL, "problem too large");
  return TSEL_OK;
}

// Attention forward: row blocks of 4 waves x one resident 32-row group.
int plan_fwd(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p) {
  plan_common(a, l, p);
  if (int rc = check_offsets(a, l, p->F)) return rc;
  p->NT = 1;
  p->TB = 4 * 32 / p->F;
  long long R = 0;
  for (int s = 0; s < p->nseg; ++s) {
    long long n, nc;
    seg_sizes(l, p->segkind, s, n, nc);
    R += (n + p->TB - 1) / p->TB;
  }
  p->jobs_per_hb = R;
  p->total_jobs = R * p->nhb;
  p->KB = p->RC = p->RCF = p->RCmax = 0;
  p->KS = p->ksmax = 0;
  p->partial_bytes = 0;
  if (p->total_jobs > (1LL << 30)) return fail(TSEL_EINVAL, "problem too large");
  return TSEL_OK;
}

// Key blocks of 4 waves x NG resident 32-key groups; row chunks of ~8192
// streamed rows, halved while the grid has fewer jobs than two workgroups
// per CU (halving further measured slower: more per-job setup).  One
// partial per (head block, row chunk, candidate).
int plan_colscore(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p) {
  plan_common(a, l, p);
  if (int rc = check_offsets(a, l, p->F)) return rc;
  long long maxn = 0;
  for (int s = 0; s < p->nseg; ++s) {
    long long n, nc;
    seg_sizes(l, p->segkind, s, n, nc);
    maxn = std::max(maxn, n);
  }
  const int ng_max = colscore_groups(dtype_of(a), a->head_dim);
  auto plan_jobs = [&](int rc, int rcf) {
    long long J = 0;
    for (int s = 0; s < p->nseg; ++s) {
      long long n, nc;
      seg_sizes(l, p->segkind, s, n, nc);
      J += ((nc + p->KB - 1) / p->KB) * chunk_count((int)n, rc, rcf);
    }
    p->RC = rc;
    p->RCF = rcf;
    p->jobs_per_hb = J;
    p->total_jobs = J * p->nhb;
  };
  // Row chunks of 8192 query rows (RC tokens x F heads); halved while the
  // grid has fewer than 512 jobs (two workgroups per CU).
  const int rc_full = std::max(32, kChunkRows / p->F);
  for (int ng = ng_max;; ng = 1) {
    p->NT = ng;
    p->KB = 4 * ng * 32;
    int rc = rc_full;
    for (;;) {
      plan_jobs(rc, rc);
      if (p->total_jobs >= 512 || rc < 64) break;
      rc = (rc / 2 + 31) / 32 * 32;
    }
    if (p->total_jobs >= 512 || ng == 1) break;
  }
  // Full-size chunks and a segment longer than one: the launch runs several
  // rounds of long jobs, and the last round decides its length.  Cutting each
  // segment's last chunk in four makes that round short jobs.  On the
  // 16384-token GQA layer this measured 3% faster with fp8 inputs and 0.5%
  // with bf16, where the clock rises as the tail leaves CUs idle (pieces of
  // 2 and 8 measured between).
  if (p->RC == rc_full && maxn > rc_full) plan_jobs(rc_full, rc_full / 4);
  p->TB = 0;
  p->KS = p->ksmax = 0;
  p->RCmax = 1;
  for (int s = 0; s < p->nseg; ++s) {
    long long n, nc;
    seg_sizes(l, p->segkind, s, n, nc);
    p->RCmax = std::max(p->RCmax, chunk_count((int)n, p->RC, p->RCF));
  }
  // The kernel reads a chunk's query tiles through one buffer resource at
  // 32-bit byte offsets from the chunk's first row.
  const long long es = elem_size(dtype_of(a));
  if (((long long)p->RC + 32) * a->q_stride_tok * es + (long long)p->F * a->q_stride_head * es >= kBufferLimit)
    return fail(TSEL_EUNSUPPORTED, "q strides too large: a row chunk of %d tokens spans 2 GiB or more", p->RC);
  const long long N = l->cu_cands_h[l->num_images];
  p->partial_bytes = (size_t)p->nhb * p->RCmax * N * sizeof(float);
  if (p->total_jobs > (1LL << 30)) return fail(TSEL_EINVAL, "problem too large");
  return TSEL_OK;
}

static DevLayout dev_layout(const tsel_layout_t *l) {
  DevLayout L;
  L.B = l->num_reqs;
  L.S = l->num_images;
  L.T = l->total_tokens;
  L.cu_seqlens = l->cu_seqlens;
  L.cu_images = l->cu_images;
  L.img_start = l->img_start;
  L.img_hw = l->img_hw;
  L.cu_cands = l->cu_cands;
  return L;
}

// Work of each job of one head block, in 32-row tiles streamed, in the
// kernels' enumeration (segment by segment).  Row-block jobs (LSE, forward):
// a causal segment's row blocks are enumerated last first and see keys up to
// their last token; otherwise every row block sees the whole segment.
// Key-block jobs (column score, row chunk rc x key block kb): the rows of the
// chunk from the first one that sees the block's first key.  One tile more
// per job stands for its setup.
static void job_weights(const tsel_attn_t *a, const tsel_layout_t *l, const AttnPlan &p, bool keyblocks,
                        std::vector<int> &w) {
  const bool causal = mask_of(a) == TSEL_MASK_CAUSAL;
  w.clear();
  for (int s = 0; s < p.nseg; ++s) {
    long long lo, hi, sl, sh;
    if (p.segkind == SEG_REQ) {
      lo = l->cu_seqlens_h[s];
      hi = l->cu_seqlens_h[s + 1];
      sl = l->cu_images_h[s];
      sh = l->cu_images_h[s + 1];
    } else {
      lo = l->img_start_h[s];
      hi = lo + (long long)l->img_hw_h[2 * s] * l->img_hw_h[2 * s + 1];
      sl = s;
      sh = s + 1;
    }
    if (!keyblocks) {
      const long long nrb = (hi - lo + p.TB - 1) / p.TB;
      for (long long loc = 0; loc < nrb; ++loc) {
        const long long rb = causal ? nrb - 1 - loc : loc;
        const long long keys = causal ? std::min((rb + 1) * p.TB, hi - lo) : hi - lo;
        w.push_back((int)((keys + 31) / 32 + 1));
      }
      continue;
    }
    const long long cl = l->cu_cands_h[sl], ch = l->cu_cands_h[sh];
    const long long nkb = (ch - cl + p.KB - 1) / p.KB;
    const int nrc = chunk_count((int)(hi - lo), p.RC, p.RCF);
    const long long tpt = 32 / p.F;
    for (int rc = 0; rc < nrc; ++rc)
      for (long long kb = 0; kb < nkb; ++kb) {
        int r0, r1;
        chunk_range(rc, (int)(hi - lo), p.RC, p.RCF, r0, r1);
        const long long c_lo = lo + r0, c_hi = lo + r1;
        long long r_lo = c_lo;
        if (causal) {
          const long long c = cl + kb * p.KB;
          long long img = sl;
          while (img + 1 < sh && l->cu_cands_h[img + 1] <= c) ++img;
          r_lo = std::max(c_lo, (long long)l->img_start_h[img] + (c - l->cu_cands_h[img]));
        }
        w.push_back((int)(std::max(0LL, (c_hi - r_lo + tpt - 1) / tpt) + 1));
      }
  }
}

// Heaviest-first job order for launches over several segments (varlen
// batches): jobs are enumerated segment by segment, so without it the light
// jobs of one request run before the heavy jobs of the next and the tail of
// the launch grows.  The column score of one causal segment is reordered too:
// its row chunks are enumerated first to last, each with its key blocks in
// order, so the half-visible diagonal jobs and the empty ones (a chunk before
// the block) are spread through the launch; heaviest first (empty jobs last),
// the 16384-token GQA layer's column score measured 1.8% faster, 5% with fp8
// inputs.  Left in enumeration order when the weights already do not increase
// (one causal segment of row blocks, equal segments) or there are too many
// jobs per head block for the permutation to travel in the arguments (row-block
// launches keep a limit of 512).  The column score runs an XCD's jobs rank by
// rank across its head blocks, the LSE head block by head block.  The forward
// keeps enumeration order: its jobs also stream V, and mixing requests within
// an XCD costs it more L2 reuse than the order wins (measured on an 8-request
// varlen batch).
static void set_order(AttnArgs &x, JobPerm &perm, const tsel_attn_t *a, const tsel_layout_t *l,
                      const AttnPlan &p, bool keyblocks, int mode) {
  x.order = kOrderPlain;
  memset(perm.w, 0, sizeof(perm.w));
  const long long cap = keyblocks ? kOrderMaxJobs : 512;
  if (mode == kOrderPlain || (p.nseg < 2 && !keyblocks) || p.jobs_per_hb > cap || p.KS > 0) return;
  std::vector<int> w;
  job_weights(a, l, p, keyblocks, w);
  if ((long long)w.size() != p.jobs_per_hb) return;
  bool sorted = true;
  for (size_t i = 1; i < w.size() && sorted; ++i) sorted = w[i] <= w[i - 1];
  if (sorted) return;
  std::vector<int> idx(w.size());
  for (size_t i = 0; i < idx.size(); ++i) idx[i] = (int)i;
  std::stable_sort(idx.begin(), idx.end(), [&](int i, int j) { return w[i] > w[j]; });
  for (size_t i = 0; i < idx.size(); ++i)
    perm.w[i >> 1] |= (unsigned)idx[i] << (16 * (i & 1));
  x.order = (mode == kOrderRankMajor && p.nhb % 8 == 0) ? kOrderRankMajor : kOrderSorted;
}

static AttnArgs attn_args(const tsel_attn_t *a, const tsel_layout_t *l, const AttnPlan &p) {
  AttnArgs x{};
  x.L = dev_layout(l);
  x.q = a->q;
  x.q_st = a->q_stride_tok;
  x.q_sh = a->q_stride_head;
  x.k = a->k;
  x.k_st = a->k_stride_tok;
  x.k_sh = a->k_stride_head;
  x.hq = a->num_heads_q;
  x.hg = a->num_heads_q / a->num_heads_kv;
  x.F = p.F;
  x.nhb = p.nhb;
  x.causal = (mask_of(a) == TSEL_MASK_CAUSAL) ? 1 : 0;
  x.segkind = p.segkind;
  x.nseg = p.nseg;
  const double scale = a->softmax_scale > 0.0f ? (double)a->softmax_scale : 1.0 / sqrt((double)a->head_dim);
  x.c1 = (float)(scale * 1.4426950408889634074);
  x.jobs_per_hb = (int)p.jobs_per_hb;
  x.total_jobs = (int)p.total_jobs;
  x.order = kOrderPlain;
  x.TB = p.TB;
  x.KS = p.KS;
  x.ksmax = p.ksmax;
  x.N = l->cu_cands_h[l->num_images];
  x.RC = p.RC;
  x.RCF = p.RCF;
  x.RCmax = p.RCmax;
  x.KB = p.KB;
  return x;
}

// Pools of more than kTopkRegLimit candidates, in launches of up to
// kTopkLargeChunk pools; the workspace holds one launch's state.
static void topk_large_launches(const tsel_layout_t *l, std::vector<TopkLarge> *out, long long *max_blocks) {
  *max_blocks = 0;
  TopkLarge cur{};
  auto flush = [&]() {
    if (cur.np == 0) return;
    *max_blocks = std::max(*max_blocks, (long long)cur.blk[cur.np]);
    if (out) out->push_back(cur);
    cur = TopkLarge{};
  };
  for (int b = 0; b < l->num_reqs; ++b) {
    const long long nb = l->cu_cands_h[l->cu_images_h[b + 1]] - l->cu_cands_h[l->cu_images_h[b]];
    if (nb <= kTopkRegLimit) continue;
    cur.pool[cur.np] = b;
    cur.blk[cur.np + 1] = cur.blk[cur.np] + (int)((nb + kTopkSplit - 1) / kTopkSplit);
    ++cur.np;
    if (cur.np == kTopkLargeChunk) flush();
  }
  flush();
}

static size_t topk_ws(const tsel_layout_t *l) {
  long long mb;
  topk_large_launches(l, nullptr, &mb);
  return mb > 0 ? topk_large_ws_bytes(mb) : 0;
}

static size_t compact_ws(const tsel_layout_t *l) {
  const long long nblk = (l->total_tokens + kCompactBlock - 1) / kCompactBlock;
  return (size_t)((2 * nblk + 1) * sizeof(int) + 255) / 256 * 256;
}

}  // namespace tsel

using namespace tsel;

extern "C" {

int tsel_version(void) { return TSEL_VERSION; }

const char *tsel_last_error(void) { return g_err.c_str(); }

size_t tsel_workspace_size(int op, const tsel_attn_t *attn, const tsel_layout_t *layout) {
  clear_error();
  if (check_layout(layout) != TSEL_OK) return (size_t)-1;
  switch (op) {
    case TSEL_OP_LSE: {
      if (check_attn(attn, layout) != TSEL_OK) return (size_t)-1;
      AttnPlan p;
      if (plan_lse(attn, layout, &p) != TSEL_OK) return (size_t)-1;
      return p.partial_bytes;
    }
    case TSEL_OP_COLSCORE: {
      if (check_attn(attn, layout) != TSEL_OK) return (size_t)-1;
      AttnPlan p;
      if (plan_colscore(attn, layout, &p) != TSEL_OK) return (size_t)-1;
      return p.partial_bytes;
    }
    case TSEL_OP_TOPK:
      return topk_ws(layout);
    case TSEL_OP_COMPACT:
      return compact_ws(layout);
    case TSEL_OP_MROPE:
      return (size_t)layout->num_images * sizeof(int32_t);
    default:
      fail(TSEL_EINVAL, "unknown op %d", op);
      return (size_t)-1;
  }
}

int tsel_lse(const tsel_attn_t *attn, const tsel_layout_t *layout, float *lse, void *workspace,
             size_t workspace_bytes, void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc == TSEL_OK) rc = check_attn(attn, layout);
  if (rc != TSEL_OK) return rc;
  if (layout->total_tokens > 0 && lse == nullptr) return fail(TSEL_EINVAL, "lse is NULL");
  if ((uintptr_t)lse & 3) return fail(TSEL_EINVAL, "lse must be 4-byte aligned");
  AttnPlan p;
  if ((rc = plan_lse(attn, layout, &p)) != TSEL_OK) return rc;
  if (p.partial_bytes > 0 && (workspace == nullptr || workspace_bytes < p.partial_bytes))
    return fail(TSEL_EWORKSPACE, "tsel_lse needs %zu workspace bytes (got %zu)", p.partial_bytes, workspace_bytes);
  if ((uintptr_t)workspace & 3) return fail(TSEL_EINVAL, "workspace must be 4-byte aligned");
  AttnArgs a = attn_args(attn, layout, p);
  JobPerm perm;
  set_order(a, perm, attn, layout, p, false, kOrderSorted);
  a.lse_out = lse;
  a.lse_part = reinterpret_cast<float *>(workspace);
  const hipError_t e = launch_lse(p, a, a.order != kOrderPlain ? &perm : nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_lse launch: %s", hipGetErrorString(e));
  return TSEL_OK;
}

}  // extern "C"

namespace tsel {

// tsel_colscore and tsel_colscore_noalloc: validation and planning, then the
// same kernels with the partials either in the caller's workspace or (noalloc)
// in the library's static device scratch.
static int colscore_call(const tsel_attn_t *attn, const tsel_layout_t *layout, const float *lse,
                         float *score, void *workspace, size_t workspace_bytes, bool noalloc,
                         void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc == TSEL_OK) rc = check_attn(attn, layout);
  if (rc != TSEL_OK) return rc;
  const int N = layout->cu_cands_h[layout->num_images];
  if (N == 0) return TSEL_OK;
  if (lse == nullptr || score == nullptr) return fail(TSEL_EINVAL, "lse and score are required");
  if (((uintptr_t)lse | (uintptr_t)score) & 3) return fail(TSEL_EINVAL, "lse/score must be 4-byte aligned");
  AttnPlan p;
  if ((rc = plan_colscore(attn, layout, &p)) != TSEL_OK) return rc;
  if (noalloc) {
    if (p.partial_bytes > kStaticScratchBytes)
      return fail(TSEL_EWORKSPACE,
                  "tsel_colscore_noalloc: this problem needs %zu bytes of column-score scratch, more than the "
                  "library's static %zu bytes; call tsel_colscore with a workspace instead",
                  p.partial_bytes, kStaticScratchBytes);
    const hipError_t e = static_scratch(&workspace);
    if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_colscore_noalloc: scratch address: %s", hipGetErrorString(e));
    workspace_bytes = kStaticScratchBytes;
  }
  if (p.partial_bytes > 0 && (workspace == nullptr || workspace_bytes < p.partial_bytes))
    return fail(TSEL_EWORKSPACE, "tsel_colscore needs %zu workspace bytes (got %zu)", p.partial_bytes,
                workspace_bytes);
  if ((uintptr_t)workspace & 15) return fail(TSEL_EINVAL, "workspace must be 16-byte aligned");
  AttnArgs a = attn_args(attn, layout, p);
  JobPerm perm;
  set_order(a, perm, attn, layout, p, true, kOrderRankMajor);
  a.lse_in = lse;
  a.partial = reinterpret_cast<float *>(workspace);
  const hipError_t e =
      launch_colscore(p, a, a.order != kOrderPlain ? &perm : nullptr, score, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_colscore launch: %s", hipGetErrorString(e));
  return TSEL_OK;
}

}  // namespace tsel

extern "C" {

int tsel_colscore(const tsel_attn_t *attn, const tsel_layout_t *layout, const float *lse,
                  float *score, void *workspace, size_t workspace_bytes, void *stream) {
  return colscore_call(attn, layout, lse, score, workspace, workspace_bytes, false, stream);
}

int tsel_colscore_noalloc(const tsel_attn_t *attn, const tsel_layout_t *layout, const float *lse,
                          float *score, void *stream) {
  return colscore_call(attn, layout, lse, score, nullptr, 0, true, stream);
}

int tsel_budget_topk(const tsel_layout_t *layout, const float *score, const double *keep_ratio_h,
                     int32_t *k_h, uint8_t *keep, void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc != TSEL_OK) return rc;
  const int B = layout->num_reqs;
  if (keep_ratio_h == nullptr || k_h == nullptr) return fail(TSEL_EINVAL, "keep_ratio_h and k_h are required");
  for (int b = 0; b < B; ++b)
    if (isnan(keep_ratio_h[b])) return fail(TSEL_EINVAL, "keep_ratio_h[%d] is NaN", b);
  const int N = layout->cu_cands_h[layout->num_images];
  if (N > 0 && (score == nullptr || keep == nullptr)) return fail(TSEL_EINVAL, "score and keep are required");
  for (int b = 0; b < B; ++b) {
    const long long nb = layout->cu_cands_h[layout->cu_images_h[b + 1]] -
                         layout->cu_cands_h[layout->cu_images_h[b]];
    const double r = std::min(1.0, std::max(0.0, keep_ratio_h[b]));
    const long long k = (long long)floor(r * (double)nb + 1e-6);
    k_h[b] = (int32_t)std::min(nb, std::max(0LL, k));
  }
  if (N == 0) return TSEL_OK;
  std::vector<TopkLarge> large;
  long long max_blocks;
  topk_large_launches(layout, &large, &max_blocks);
  const size_t need = max_blocks > 0 ? topk_large_ws_bytes(max_blocks) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(TSEL_EWORKSPACE, "tsel_budget_topk needs %zu workspace bytes (got %zu)", need, workspace_bytes);
  if ((uintptr_t)workspace & 3) return fail(TSEL_EINVAL, "workspace must be 4-byte aligned");
  const DevLayout L = dev_layout(layout);
  for (int b0 = 0; b0 < B; b0 += 256) {
    TopkChunk ch;
    ch.b0 = b0;
    const int np = std::min(256, B - b0);
    for (int i = 0; i < 256; ++i) ch.k[i] = (i < np) ? k_h[b0 + i] : 0;
    const hipError_t e = launch_topk(L, score, ch, np, keep, (hipStream_t)stream);
    if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_budget_topk launch: %s", hipGetErrorString(e));
  }
  int *ws = reinterpret_cast<int *>(workspace);
  const TopkLargeWs lw{ws, ws + kTopkLargeChunk * 4, ws + kTopkLargeChunk * 4 + kTopkLargeChunk * 256};
  for (TopkLarge &tl : large) {
    for (int i = 0; i < tl.np; ++i) tl.k[i] = k_h[tl.pool[i]];
    const hipError_t e = launch_topk_large(L, score, tl, lw, keep, (hipStream_t)stream);
    if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_budget_topk launch: %s", hipGetErrorString(e));
  }
  return TSEL_OK;
}

int tsel_budget_mass(const tsel_layout_t *layout, const float *score, const double *tau_h,
                     const double *r_min_h, const double *r_max_h, int32_t *k, uint8_t *keep,
                     void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc != TSEL_OK) return rc;
  const int B = layout->num_reqs;
  if (tau_h == nullptr || r_min_h == nullptr || r_max_h == nullptr)
    return fail(TSEL_EINVAL, "tau_h, r_min_h and r_max_h are required");
  if (k == nullptr || ((uintptr_t)k & 3)) return fail(TSEL_EINVAL, "k must be a 4-byte aligned device array");
  const int N = layout->cu_cands_h[layout->num_images];
  if (N > 0 && (score == nullptr || keep == nullptr)) return fail(TSEL_EINVAL, "score and keep are required");
  auto clamp01 = [](double v) { return std::min(1.0, std::max(0.0, v)); };
  for (int b = 0; b < B; ++b) {
    if (isnan(tau_h[b]) || isnan(r_min_h[b]) || isnan(r_max_h[b]))
      return fail(TSEL_EINVAL, "tau/r_min/r_max of pool %d is NaN", b);
    if (clamp01(r_min_h[b]) > clamp01(r_max_h[b])) return fail(TSEL_EINVAL, "r_min > r_max in pool %d", b);
  }
  const DevLayout L = dev_layout(layout);
  for (int b0 = 0; b0 < B; b0 += kMassChunk) {
    MassChunk mc{};
    mc.b0 = b0;
    const int np = std::min(kMassChunk, B - b0);
    for (int i = 0; i < np; ++i) {
      const int b = b0 + i;
      const long long nb = layout->cu_cands_h[layout->cu_images_h[b + 1]] -
                           layout->cu_cands_h[layout->cu_images_h[b]];
      auto bound = [&](double r) {
        return (int)std::min(nb, std::max(0LL, (long long)floor(clamp01(r) * (double)nb + 1e-6)));
      };
      mc.kmin[i] = bound(r_min_h[b]);
      mc.kmax[i] = bound(r_max_h[b]);
      mc.tau[i] = clamp01(tau_h[b]);
    }
    const hipError_t e = launch_mass_budget(L, score, mc, np, k, keep, (hipStream_t)stream);
    if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_budget_mass launch: %s", hipGetErrorString(e));
  }
  return TSEL_OK;
}

int tsel_compact(const tsel_layout_t *layout, const uint8_t *keep, const void *emb,
                 int64_t emb_stride, int64_t emb_row_bytes, int32_t out_capacity, void *out_emb,
                 int64_t out_emb_stride, int32_t *out_token_idx, int32_t *out_spatial,
                 int32_t *out_cu_seqlens, int32_t *out_img_counts, void *workspace,
                 size_t workspace_bytes, void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc != TSEL_OK) return rc;
  const int N = layout->cu_cands_h[layout->num_images];
  if (N > 0 && keep == nullptr) return fail(TSEL_EINVAL, "keep is required");
  if (out_capacity < 0) return fail(TSEL_EINVAL, "out_capacity must be >= 0");
  if (out_capacity > 0 && out_token_idx == nullptr) return fail(TSEL_EINVAL, "out_token_idx is required");
  if (emb != nullptr) {
    if (out_emb == nullptr) return fail(TSEL_EINVAL, "out_emb is required when emb is given");
    if (emb_row_bytes <= 0 || emb_stride < emb_row_bytes || out_emb_stride < emb_row_bytes)
      return fail(TSEL_EINVAL, "embedding row bytes/strides are inconsistent");
  }
  const size_t need = compact_ws(layout);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(TSEL_EWORKSPACE, "tsel_compact needs %zu workspace bytes (got %zu)", need, workspace_bytes);
  if ((uintptr_t)workspace & 3) return fail(TSEL_EINVAL, "workspace must be 4-byte aligned");
  CompactArgs c{};
  c.L = dev_layout(layout);
  c.keep = keep;
  c.N = N;
  c.nblk = (layout->total_tokens + kCompactBlock - 1) / kCompactBlock;
  int *ws = reinterpret_cast<int *>(workspace);
  c.blk_cnt = ws;
  c.blk_off = ws + c.nblk;
  c.total = ws + 2 * c.nblk;
  c.cap = out_capacity;
  c.out_token_idx = out_token_idx;
  c.out_spatial = out_spatial;
  c.out_cu_seqlens = out_cu_seqlens;
  c.out_img_counts = out_img_counts;
  hipError_t e = launch_compact(c, (hipStream_t)stream);
  if (e == hipSuccess && emb != nullptr)
    e = launch_gather(emb, emb_stride, emb_row_bytes, out_emb, out_emb_stride, out_token_idx, c.total,
                      out_capacity, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_compact launch: %s", hipGetErrorString(e));
  return TSEL_OK;
}

int tsel_attention_fwd(const tsel_attn_t *attn, const tsel_layout_t *layout, const void *v,
                       int64_t v_stride_tok, int64_t v_stride_head, void *out, int64_t out_stride_tok,
                       int64_t out_stride_head, float *lse, void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc == TSEL_OK) rc = check_attn(attn, layout);
  if (rc != TSEL_OK) return rc;
  if (dtype_of(attn) != TSEL_BF16 && dtype_of(attn) != TSEL_F16)
    return fail(TSEL_EUNSUPPORTED, "the attention forward takes bf16 or f16 inputs");
  const long long es = elem_size(dtype_of(attn));
  if (layout->total_tokens > 0) {
    if (v == nullptr || out == nullptr || lse == nullptr)
      return fail(TSEL_EINVAL, "v, out and lse are required");
    if ((uintptr_t)v & 15) return fail(TSEL_EINVAL, "v must be 16-byte aligned");
    if ((uintptr_t)out & 7) return fail(TSEL_EINVAL, "out must be 8-byte aligned");
    if ((uintptr_t)lse & 3) return fail(TSEL_EINVAL, "lse must be 4-byte aligned");
  }
  if (v_stride_tok <= 0 || v_stride_head <= 0 || (v_stride_tok * es) % 16 || (v_stride_head * es) % 16)
    return fail(TSEL_EINVAL, "v strides must be positive and multiples of 16 bytes");
  if (out_stride_tok <= 0 || out_stride_head <= 0 || (out_stride_tok * es) % 8 ||
      (out_stride_head * es) % 8)
    return fail(TSEL_EINVAL, "out strides must be positive and multiples of 8 bytes");
  if (32LL * v_stride_tok * es >= kBufferLimit)
    return fail(TSEL_EUNSUPPORTED, "strides too large: a 32-row tile spans 2 GiB or more");
  // The kernel zeroes the key and value rows past a tile's valid range by
  // ending that tile's buffer range after its last valid row, which needs
  // rows that do not overlap in memory.
  if (attn->k_stride_tok < attn->head_dim || v_stride_tok < attn->head_dim)
    return fail(TSEL_EUNSUPPORTED, "the attention forward needs k and v token strides of at least head_dim");
  AttnPlan p;
  if ((rc = plan_fwd(attn, layout, &p)) != TSEL_OK) return rc;
  FwdArgs x{};
  x.at = attn_args(attn, layout, p);
  x.at.lse_out = lse;
  x.v = v;
  x.v_st = v_stride_tok;
  x.v_sh = v_stride_head;
  x.out = out;
  x.o_st = out_stride_tok;
  x.o_sh = out_stride_head;
  hipError_t e = launch_fwd(p, x, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_attention_fwd launch: %s", hipGetErrorString(e));
  return TSEL_OK;
}

int tsel_mrope_positions(const tsel_layout_t *layout, const int32_t *out_token_idx,
                         const int32_t *out_spatial, int32_t n_out, int32_t *out_pos,
                         void *workspace, size_t workspace_bytes, void *stream) {
  clear_error();
  int rc = check_layout(layout);
  if (rc != TSEL_OK) return rc;
  if (n_out < 0) return fail(TSEL_EINVAL, "n_out must be >= 0");
  if (n_out > 0 && (out_token_idx == nullptr || out_spatial == nullptr || out_pos == nullptr))
    return fail(TSEL_EINVAL, "out_token_idx, out_spatial and out_pos are required");
  const size_t need = (size_t)layout->num_images * sizeof(int32_t);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(TSEL_EWORKSPACE, "tsel_mrope_positions needs %zu workspace bytes (got %zu)", need,
                workspace_bytes);
  if ((uintptr_t)workspace & 3) return fail(TSEL_EINVAL, "workspace must be 4-byte aligned");
  hipError_t e = launch_mrope(dev_layout(layout), reinterpret_cast<int *>(workspace), out_token_idx,
                              out_spatial, n_out, out_pos, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TSEL_EHIP, "tsel_mrope_positions launch: %s", hipGetErrorString(e));
  return TSEL_OK;
}

}  // extern "C"
