// Softmax LSE and column-score kernels for gfx950.
//
// Both kernels share one shape: a RESIDENT operand held in VGPRs for the whole
// workgroup (the B operand of v_mfma_f32_32x32x16_{bf16,f16}, or of eight
// v_mfma_f32_32x32x2_f32 for fp32), and a STREAMED operand that the workgroup
// stages through LDS in tiles of 32 rows (the A operand).  The 32x32
// accumulator then holds, per lane, one column of the resident side
// (lane % 32) and sixteen rows of the streamed side, so every reduction the
// method needs along the streamed side happens inside the lane; the two lane
// halves are combined once at the very end.  The 32x32x16 shape is used
// because on gfx950 it lets the VALU work (exp2, FMA, adds) overlap the matrix
// pipe far better than 16x16x32 does.
//
//  * LSE (per-row softmax normaliser; the REDtech article, section 3.2,
//    reuses it): resident = query rows, streamed = key tiles.  Rows reduce
//    in-lane.
//  * Column score (attention a vision token receives: LiteVLM review,
//    formula section; a column-wise reduction that never materialises the
//    attention matrix: REDtech article, section 3.2): resident = candidate
//    keys, streamed = query-row tiles; each tile's accumulation chains start
//    from its rows' -LSE/scale, held in LDS for the job.  Columns reduce
//    in-lane; nothing of P leaves the registers.
//
// Query heads that share a KV head are folded into the row dimension (F heads
// per token in each 32-row group), so one key fragment serves F query heads.
//
// Streamed tiles reach LDS through the LDS-direct form of the buffer load (no
// staging registers), one tile ahead, with per-lane offsets fixed for the
// whole job.
#include "tiles.h"

namespace tsel {

// ---------------------------------------------------------------------------
// LSE kernel.
// Job = (head block hb, segment a, row block rb): TB tokens x F heads of one
// segment; each of the 4 waves owns NG*32 of those rows.  Keys stream in
// tiles of 32 over [seg_lo, key_hi).
// ---------------------------------------------------------------------------

// One pass over the job's key tiles [0, nt): tile it holds keys key_lo + 32*it
// .. +31 (those from key_hi on read as zero).  Tiles [0, full_end) are
// visible to every row of this wave, tiles [full_end, seen_end) to some of
// them (masked per lane), tiles from seen_end on to none (skipped; the wave
// still stages them and joins every barrier).  MAXMODE: acc = running max of
// the raw logit over this lane's keys.  Otherwise acc = running sum of
// exp2(c1*s - m) over this lane's keys; with FIRSTM, m is first set from
// tile 0 (its row max in log2 units plus 32) before that tile's terms.
template <int DT, int D, int NG, bool MAXMODE, bool FIRSTM = false>
__device__ __forceinline__ void lse_pass(char *smem, const AttnArgs &a, StageDirect<DT, D> &st,
                                         const char *kbase, int tile_bytes, int key_lo, int key_hi, int nt,
                                         int full_end, int seen_end,
                                         const Chunk<DT> (&qf)[NG][kch(DT, D)],
                                         const int (&qtok)[NG], float (&m)[NG],
                                         float (&acc)[NG]) {
  using G = Geom<DT, D>;
#pragma unroll
  for (int n = 0; n < NG; ++n) acc[n] = MAXMODE ? kNegInf : 0.0f;
  // Key tile it from its first row on (one scalar base per tile, so the
  // key range of a job is not limited by the 32-bit buffer offsets).
  auto load = [&](int it) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(kbase + (long long)it * tile_bytes);
    const int nv = key_hi - (key_lo + kRows * it);
    char *b = smem + (it & 1) * G::TILE;
    if (nv >= kRows) st.template load_at<false>(b, rs, 0, kRows);
    else st.template load_at<true>(b, rs, 0, nv);
  };
  load(0);
  __syncthreads();

  // One tile (MODE 0: skipped, 1: masked, 2: visible to every row; FIRST:
  // tile 0 of a FIRSTM pass).
  auto step = [&](int it, auto mode, auto first) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool FIRST = decltype(first)::value;
    Chunk<DT> af[G::KCH];
    if (MODE != 0) read_frag<DT, D>(af, smem + (it & 1) * G::TILE);
    if (it + 1 < nt) load(it + 1);
    if (FIRST && MODE == 0) {
#pragma unroll
      for (int n = 0; n < NG; ++n) m[n] = kNegInf;  // no row of this wave sees tile 0
    }
    if (MODE != 0) {
      const int k0 = key_lo + kRows * it;
      f32x16 s[NG];
      tile_mma<DT, D, NG>(af, qf, s);
#pragma unroll
      for (int n = 0; n < NG; ++n) {
        // Key of register v is k0 + acc_row_c(v) + 4*(lane/32): visible while
        // below key_hi and (causal) not past the row's token qtok[n].
        const int lim = MODE == 1 ? min(key_hi - 1, a.causal ? qtok[n] : key_hi - 1) -
                                        (k0 + 4 * (lane_id() >> 5))
                                  : 0;
        if (FIRST) {
          float t = kNegInf;
#pragma unroll
          for (int v = 0; v < 16; ++v) t = fmaxf(t, (MODE == 2 || acc_row_c(v) <= lim) ? s[n][v] : kNegInf);
          m[n] = fmaxf(t, __shfl_xor(t, 32, 64)) * a.c1 + 32.0f;
        }
        float p[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const bool vis = MODE == 2 || acc_row_c(v) <= lim;
          if (MAXMODE) p[v] = vis ? s[n][v] : kNegInf;
          else p[v] = vis ? fast_exp2(fmaf(s[n][v], a.c1, -m[n])) : 0.0f;
        }
        if (MAXMODE) {
          float t = p[0];
#pragma unroll
          for (int v = 1; v < 16; ++v) t = fmaxf(t, p[v]);
          acc[n] = fmaxf(acc[n], t);
        } else {
          acc[n] += tree16(p);
        }
      }
    }
    // Keep the barrier after this tile's MFMAs and epilogue (the scheduler
    // would otherwise hoist it above them in the branch-free runs).
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  int it = 0;
  if (FIRSTM && nt > 0) {
    if (0 < full_end) step(0, std::integral_constant<int, 2>{}, std::true_type{});
    else if (0 < seen_end) step(0, std::integral_constant<int, 1>{}, std::true_type{});
    else step(0, std::integral_constant<int, 0>{}, std::true_type{});
    it = 1;
  }
  for (; it < full_end; ++it) step(it, std::integral_constant<int, 2>{}, std::false_type{});
  for (; it < seen_end; ++it) step(it, std::integral_constant<int, 1>{}, std::false_type{});
  for (; it < nt; ++it) step(it, std::integral_constant<int, 0>{}, std::false_type{});
}

// Kernel argument carrying the job permutation (ORD) or nothing.
template <bool ORD> struct PermArg {};
template <> struct PermArg<true> { JobPerm p; };

template <bool ORD>
__device__ __forceinline__ void job_of(const AttnArgs &a, const PermArg<ORD> &pa, int job, int &hb, int &rj) {
  if constexpr (ORD) job_ordered(a, pa.p, job, hb, rj);
  else job_plain(a, job, hb, rj);
}

template <int DT, int D, int NG, bool ORD>
__global__ __launch_bounds__(256, 2) void lse_kernel(AttnArgs a, PermArg<ORD> pa) {
  using G = Geom<DT, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::TILE];
  __shared__ int s_bad;

  const int job = xcd_job(blockIdx.x, gridDim.x);
  if (job >= a.total_jobs) return;
  const int TB = a.TB, KS = a.KS;
  // Jobs of a segment of n tokens: its row blocks, each split into ceil(n/KS)
  // key ranges of KS keys when KS > 0 (the splits past a causal row block's
  // last key are empty jobs).
  auto count = [&](int s) {
    int lo, hi;
    seg_tokens(a.L, a.segkind, s, lo, hi);
    const int nrb = (hi - lo + TB - 1) / TB;
    return KS ? nrb * ((hi - lo + KS - 1) / KS) : nrb;
  };
  int hb, rj;
  job_of<ORD>(a, pa, job, hb, rj);
  int local;
  const int seg = find_segment(a.nseg, rj, count, local);
  if (seg < 0) return;
  int seg_lo, seg_hi;
  seg_tokens(a.L, a.segkind, seg, seg_lo, seg_hi);
  // Layout values of this job are workgroup-uniform: keep them in scalar
  // registers (tile addresses built from them then stay scalar too).
  seg_lo = uni(seg_lo);
  seg_hi = uni(seg_hi);
  const int nks = KS ? (seg_hi - seg_lo + KS - 1) / KS : 1;
  const int nrb = (seg_hi - seg_lo + TB - 1) / TB;
  const int rbl = local / nks, ks = local % nks;
  const int rb = a.causal ? nrb - 1 - rbl : rbl;  // causal: heaviest row blocks first
  const int tok_lo = seg_lo + rb * TB;
  const int tok_hi = min(tok_lo + TB, seg_hi);

  const int lane = lane_id(), w = uni(threadIdx.x >> 6);
  const int F = a.F;
  const int wtok0 = uni(tok_lo + w * (NG * kRows / F));
  const int wtok_max = uni(wtok0 + NG * kRows / F - 1);
  const int h0 = uni(hb * F);
  const int g = uni(h0 / a.hg);
  // Keys of this job: the row block's whole range, or its ks-th split.
  const int key_lo = uni(seg_lo + ks * KS);
  const int key_end = a.causal ? tok_hi : seg_hi;
  const int key_hi = uni(KS ? min(key_end, key_lo + KS) : key_end);
  if (key_lo >= key_hi) return;  // a causal row block before this split
  const int ntiles = uni((key_hi - key_lo + kRows - 1) / kRows);
  // Tiles every row of this wave sees in full, and tiles some row sees
  // (causal: keys up to the wave's last token); a wave past the row block's
  // end sees none.
  auto tiles_upto = [&](int last_key) {  // tiles whose keys all lie at or before last_key
    const int x = last_key - key_lo - (kRows - 1);
    return x < 0 ? 0 : min(ntiles, x / kRows + 1);
  };
  auto tiles_from = [&](int last_key) {  // tiles whose first key lies at or before last_key
    const int x = last_key - key_lo;
    return x < 0 ? 0 : min(ntiles, x / kRows + 1);
  };
  const bool wave_live = wtok0 < tok_hi;
  const int full_end = uni(wave_live ? tiles_upto(a.causal ? min(key_hi - 1, wtok0) : key_hi - 1) : 0);
  const int seen_end = uni(wave_live ? (a.causal ? tiles_from(wtok_max) : ntiles) : 0);

  // Resident queries: row q of this wave is (token wtok0 + q / F, head h0 + q % F).
  Chunk<DT> qf[NG][G::KCH];
  int qtok[NG];
  const char *qbase = reinterpret_cast<const char *>(a.q);
  load_resident<DT, D, NG>(qf, [&](int q) -> const char * {
    const int t = wtok0 + q / F;
    if (t >= tok_hi) return nullptr;
    return qbase + ((long long)t * a.q_st + (long long)(h0 + q % F) * a.q_sh) * G::ES;
  });
#pragma unroll
  for (int n = 0; n < NG; ++n) qtok[n] = wtok0 + (n * kRows + (lane & 31)) / F;
  wait_vmem();

  // Key tile it starts at key row key_lo + 32*it of KV head g.
  const long long krow = a.k_st * G::ES;
  const char *kbase = reinterpret_cast<const char *>(a.k) + (long long)g * a.k_sh * G::ES + key_lo * krow;
  const int tile_bytes = (int)(kRows * krow);
  StageDirect<DT, D> st;
  st.init([&](int r) { return r * (int)krow; });

  // Offset m: max logit of the first key tile (which every row sees, except,
  // in a later key split of a causal row block, the rows before the split)
  // plus 32 (log2 units), taken from that tile inside the sum pass; the sum
  // then cannot overflow unless a later logit exceeds it by ~100, which the
  // check below catches.
  float m[NG], acc[NG];
#pragma unroll
  for (int n = 0; n < NG; ++n) m[n] = 0.f;
  if (threadIdx.x == 0) s_bad = 0;
  lse_pass<DT, D, NG, false, true>(smem, a, st, kbase, tile_bytes, key_lo, key_hi, ntiles, full_end, seen_end, qf,
                                   qtok, m, acc);
  float tot[NG];
  bool ok = true;
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    tot[n] = acc[n] + __shfl_xor(acc[n], 32, 64);
    const bool sees = qtok[n] < tok_hi && !(a.causal && qtok[n] < key_lo);
    if (sees) ok = ok && (tot[n] <= 0x1p100f) && (tot[n] >= 0x1p-100f);  // false for NaN
  }
  if (!ok) s_bad = 1;
  __syncthreads();
  if (s_bad) {
    // Exact two-pass fallback: true row max, then the sum against it.
    lse_pass<DT, D, NG, true>(smem, a, st, kbase, tile_bytes, key_lo, key_hi, ntiles, full_end, seen_end, qf,
                              qtok, m, acc);
#pragma unroll
    for (int n = 0; n < NG; ++n) m[n] = fmaxf(acc[n], __shfl_xor(acc[n], 32, 64)) * a.c1;
    lse_pass<DT, D, NG, false>(smem, a, st, kbase, tile_bytes, key_lo, key_hi, ntiles, full_end, seen_end, qf,
                               qtok, m, acc);
#pragma unroll
    for (int n = 0; n < NG; ++n) tot[n] = acc[n] + __shfl_xor(acc[n], 32, 64);
  }
  if (lane < 32) {
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const int q = n * kRows + lane;
      const int t = wtok0 + q / F;
      if (t < tok_hi) {
        const float lse2 = (a.causal && t < key_lo) ? kNegInf : m[n] + __log2f(tot[n]);
        const long long row = (long long)(h0 + q % F) * a.L.T + t;
        if (KS) a.lse_part[row * a.ksmax + ks] = lse2;
        else a.lse_out[row] = lse2 * 0.69314718055994530942f;
      }
    }
  }
}

// Key-split LSE: combine a row's per-split log2-sum-exp values l_s into
// LSE = ln 2 * (M + log2 sum_s 2^(l_s - M)), M = max_s l_s, splits in order.
// A row sees splits 0 .. (causal: the split holding its own token; else the
// last).  A NaN partial makes the row's LSE NaN.
__global__ __launch_bounds__(256) void lse_merge(AttnArgs a) {
  const long long T = a.L.T;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)a.hq * T) return;
  const int h = (int)(idx / T), t = (int)(idx % T);
  const DevLayout &L = a.L;
  int lo, hi;
  if (a.segkind == SEG_REQ) {
    const int b = upper_index(L.cu_seqlens, 0, L.B, t);
    lo = L.cu_seqlens[b];
    hi = L.cu_seqlens[b + 1];
  } else {
    const int s = upper_index(L.img_start, 0, L.S, t);
    lo = L.img_start[s];
    hi = lo + L.img_hw[2 * s] * L.img_hw[2 * s + 1];
  }
  const int last = a.causal ? (t - lo) / a.KS : (hi - lo - 1) / a.KS;
  const float *p = a.lse_part + idx * a.ksmax;
  float M = kNegInf;
  bool nan = false;
  for (int ks = 0; ks <= last; ++ks) {
    const float v = p[ks];
    nan = nan || (v != v);
    M = fmaxf(M, v);
  }
  float sum = 0.f;
  for (int ks = 0; ks <= last; ++ks) sum += fast_exp2(p[ks] - M);
  a.lse_out[idx] = nan ? __builtin_nanf("") : (M + __log2f(sum)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
// Column-score kernel.
// Job = (head block hb, segment a, row chunk rc, key block kb).  Each wave
// holds NG*32 candidate keys; query-row tiles of 32 rows (32/F tokens x F
// heads) stream through LDS, the rows' LSE terms are put in LDS once per job;
// per-column partial sums go to partial[(hb*RCmax + rc)*N + c].
// ---------------------------------------------------------------------------
template <int DT, int D, int NG, bool ORD>
__global__ __launch_bounds__(256, colscore_wgs(DT)) void colscore_kernel(AttnArgs a, PermArg<ORD> pa) {
  using G = Geom<DT, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::TILE];
  // Per row of the job (a row chunk holds at most kChunkRows rows) the value
  // its scores start from, -LSE / scale, padded to whole tiles with -inf
  // (rows that contribute 0): the initial value of the MFMA accumulation
  // chains, so that the epilogue is exp2(c1 * acc) and no LSE registers live
  // through it.  That frees the registers a fourth resident key group needs
  // at d = 96..128 with 16-bit inputs, and lets fp8 run three workgroups per
  // CU.
  __shared__ __attribute__((aligned(16))) float slse[kChunkRows + kRows];
  // Key token of each lane column of each resident group, per wave: read by
  // the masked tiles near the causal diagonal, which run after the unmasked
  // ones, so these values are not held in registers through the main loop.
  __shared__ int sktok[4][NG][kRows];

  const int job = xcd_job(blockIdx.x, gridDim.x);
  if (job >= a.total_jobs) return;
  const int KB = a.KB;
  auto count = [&](int s) {
    int lo, hi, sl, sh, cl, ch;
    seg_tokens(a.L, a.segkind, s, lo, hi);
    seg_images(a.L, a.segkind, s, sl, sh, cl, ch);
    return ((ch - cl + KB - 1) / KB) * chunk_count(hi - lo, a.RC, a.RCF);
  };
  int hb, rj;
  job_of<ORD>(a, pa, job, hb, rj);
  int local;
  const int seg = find_segment(a.nseg, rj, count, local);
  if (seg < 0) return;
  int seg_lo, seg_hi, s_lo, s_hi, c_lo, c_hi;
  seg_tokens(a.L, a.segkind, seg, seg_lo, seg_hi);
  seg_images(a.L, a.segkind, seg, s_lo, s_hi, c_lo, c_hi);
  // Layout values of this job are workgroup-uniform: keep them in scalar
  // registers (tile addresses built from them then stay scalar too).
  seg_lo = uni(seg_lo);
  seg_hi = uni(seg_hi);
  s_lo = uni(s_lo);
  s_hi = uni(s_hi);
  c_lo = uni(c_lo);
  c_hi = uni(c_hi);
  const int nkb = (c_hi - c_lo + KB - 1) / KB;
  const int rc = local / nkb, kb = local % nkb;
  const int kb0 = c_lo + kb * KB;
  const int kb1 = min(kb0 + KB, c_hi);
  int chunk_lo, chunk_hi;
  chunk_range(rc, seg_hi - seg_lo, a.RC, a.RCF, chunk_lo, chunk_hi);
  chunk_lo = uni(seg_lo + chunk_lo);
  chunk_hi = uni(seg_lo + chunk_hi);
  // Candidate -> token lookups of this job.
  const ImgLanes im = img_lanes(a.L, s_lo, s_hi);
  const bool few = im.n <= 64;
  auto tok_u = [&](int c) { return uni(few ? img_token_uniform(im, c) : cand_token(a.L, s_lo, s_hi, c)); };
  const int first_ktok = tok_u(kb0);
  const int row_lo = uni(a.causal ? max(chunk_lo, first_ktok) : chunk_lo);
  if (row_lo >= chunk_hi) return;  // no row of this chunk sees any key of the block

  const int lane = lane_id(), w = uni(threadIdx.x >> 6);
  const int F = a.F;
  const int h0 = hb * F;
  const int g = h0 / a.hg;
  // Resident keys: group n of wave w holds the 32 candidates from
  // gbase(n) = kb0 + 32*(4n + w), lane column lane % 32.  Interleaving the
  // groups across the four waves splits the groups that a tile near the
  // causal diagonal reaches evenly between the waves (with contiguous
  // ranges the first wave would compute them all while the others wait at
  // the tile's barrier), and a tile computes only the groups it reaches.
  auto gbase = [&](int n) { return kb0 + kRows * (4 * n + w); };
  Chunk<DT> kf[NG][G::KCH];
  int ktok[NG];
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    const int c = gbase(n) + (lane & 31);
    const int t = few ? img_token(im, min(c, kb1 - 1)) : cand_token(a.L, s_lo, s_hi, min(c, kb1 - 1));
    ktok[n] = (c < kb1) ? t : 0x7fffffff;
  }
  // First and last key token of each group; the groups holding candidates
  // are the first nvalid (candidates are in token order), and so are the
  // groups a tile reaches.
  int gkmin[NG], gkmax[NG];
  int nvalid = 0;
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    const int last = min(kRows - 1, kb1 - 1 - gbase(n));
    gkmin[n] = last >= 0 ? uni(__shfl(ktok[n], 0, 64)) : 0x7fffffff;
    gkmax[n] = last >= 0 ? uni(__shfl(ktok[n], last, 64)) : 0x7fffffff;
    nvalid += last >= 0 ? 1 : 0;
  }
  nvalid = uni(nvalid);
  const char *kbase = reinterpret_cast<const char *>(a.k);
  load_resident<DT, D, NG>(kf, [&](int j) -> const char * {
    const int t = ktok[j / kRows];
    if (t == 0x7fffffff) return nullptr;
    return kbase + ((long long)t * a.k_st + (long long)g * a.k_sh) * G::ES;
  });

  const int tpt = kRows / F;  // tokens per streamed tile
  const int ntiles = uni((chunk_hi - row_lo + tpt - 1) / tpt);
  // The job's LSE, row r = (token row_lo + r/F, head h0 + r%F), converted to
  // log2 units; rows of tokens from chunk_hi on get +inf and so contribute
  // exp2(-inf) = 0.
  {
    const long long T = a.L.T;
    const float *lb = a.lse_in + (long long)h0 * T + row_lo;
    const int nr = ntiles * kRows;
    const int dmax = chunk_hi - 1 - row_lo;   // last token offset of the chunk
    const int lf = 31 - __builtin_clz(F);     // F is a power of two
    const float inv_c1 = 1.0f / a.c1;
    // Batches of eight independent loads per thread (token offsets clamped
    // into the chunk, so every address is valid), then the stores.
    for (int r0 = 0; r0 < nr; r0 += 256 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + 256 * u + (int)threadIdx.x;
        v[u] = lb[(long long)(r & (F - 1)) * T + min(r >> lf, dmax)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + 256 * u + (int)threadIdx.x;
        if (r < nr) slse[r] = (r >> lf) <= dmax ? -(v[u] * 1.44269504088896340736f) * inv_c1 : kNegInf;
      }
    }
  }
  // Query tile it: row r is (token row_lo + it*tpt + r/F, head h0 + r%F),
  // read through one buffer resource at the byte offset of its first token.
  const long long qtok_bytes = a.q_st * G::ES;
  const int qhead_bytes = (int)(a.q_sh * G::ES);
  const __amdgpu_buffer_rsrc_t qrs =
      buffer_rsrc(reinterpret_cast<const char *>(a.q) + ((long long)row_lo * a.q_st + (long long)h0 * a.q_sh) * G::ES);
  const int tile_step = tpt * (int)qtok_bytes;
  const int last_rows = (chunk_hi - (row_lo + (ntiles - 1) * tpt)) * F;
  float cs[NG];
#pragma unroll
  for (int n = 0; n < NG; ++n) cs[n] = 0.f;

  StageDirect<DT, D> st;
  st.init([&](int r) { return (r / F) * (int)qtok_bytes + (r % F) * qhead_bytes; });
  auto buf = [&](int it) { return smem + (it & 1) * G::TILE; };
  auto load = [&](int it) {
    if (it + 1 < ntiles) st.template load_at<false>(buf(it), qrs, it * tile_step, kRows);
    else st.template load_at<true>(buf(it), qrs, it * tile_step, last_rows);
  };
#pragma unroll
  for (int n = 0; n < NG; ++n) sktok[w][n][lane & 31] = ktok[n];
  load(ntiles - 1);
  __syncthreads();

  // Runs of tiles for this wave (causal): rows before every key (skipped);
  // rows that reach the first m groups, m = 1..nvalid (masked where a
  // group's last key is later than the tile's first row); then rows past
  // all its keys (unmasked).  Tile it reaches group n from live(n) on.
  // Every wave runs every tile's barrier and load.
  auto live = [&](int n) {
    return n < nvalid ? (a.causal ? uni(min(ntiles, max(0, (gkmin[n] - row_lo) / tpt))) : 0) : ntiles;
  };
  const int full_start = uni(
      nvalid == 0 ? ntiles
                  : (a.causal ? min(ntiles, max(live(nvalid - 1), (gkmax[nvalid - 1] - row_lo + tpt - 1) / tpt)) : 0));

  // One tile: start loading the next one (tile it - 1) into the other buffer
  // (read last step), then the MFMAs and the epilogue of this tile for the
  // first M groups (MODE 0: skipped, 1: masked where needed, 2: unmasked).
  auto step = [&](int it, auto mode, auto groups) {
    constexpr int MODE = decltype(mode)::value;
    constexpr int M = decltype(groups)::value;
    const char *b = buf(it);
    Chunk<DT> af[G::KCH];
    float l2[16];
    if (MODE != 0) {
      // Start values of this lane's rows 8q + 4*(lane/32) + 0..3, q = 0..3,
      // read before the fragments: the chains need them at their first
      // MFMA, and LDS reads return in order.
      const float *lb = slse + it * kRows + 4 * (lane >> 5);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4v v4 = *reinterpret_cast<const f32x4v *>(lb + 8 * q4);
#pragma unroll
        for (int j = 0; j < 4; ++j) l2[4 * q4 + j] = v4[j];
      }
      read_frag<DT, D>(af, b);
    }
    if (it > 0) load(it - 1);
    if (MODE != 0) {
      f32x16 s[NG];
      f32x16 seed;
#pragma unroll
      for (int v = 0; v < 16; ++v) seed[v] = l2[v];
      tile_mma_seeded<DT, D, NG, M>(af, kf, s, seed);
      const int tt0 = row_lo + it * tpt;
      auto epi = [&](int n, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        // Row of register v has token tt0 + (acc_row_c(v) + 4*(lane/32)) / F;
        // it sees key token kt iff acc_row_c(v) >= (kt - tt0)*F - 4*(lane/32)
        // (the clamp keeps past-the-end columns invisible).
        const int thr = MASKED ? min(sktok[w][n][lane & 31] - tt0, kRows) * F - 4 * (lane >> 5) : 0;
        float p[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          p[v] = fast_exp2(s[n][v] * a.c1);
          if (MASKED) p[v] = (acc_row_c(v) >= thr) ? p[v] : 0.0f;
        }
        cs[n] += tree16(p);
      };
      if (MODE == 2) {
#pragma unroll
        for (int n = 0; n < M; ++n) epi(n, std::false_type{});
      } else {
        // Near the diagonal only the groups whose last key is later than the
        // tile's first token need the mask.
#pragma unroll
        for (int n = 0; n < M; ++n) {
          if (tt0 < gkmax[n]) epi(n, std::true_type{});
          else epi(n, std::false_type{});
        }
      }
    }
    // The barrier (and its wait for the next tile's load) stays after this
    // tile's MFMAs and epilogue: the scheduler would otherwise hoist it above
    // them in the branch-free runs and expose the load's latency.
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  using Skip = std::integral_constant<int, 0>;
  using Masked = std::integral_constant<int, 1>;
  using Full = std::integral_constant<int, 2>;
  // The tiles run from the last one down: every job of a row chunk then
  // starts on the chunk's last tile whatever its key block, so the jobs of
  // one chunk that run at the same time read the same query tiles in step
  // (one fetch into L2 serves them all).  First the tiles past all of this
  // wave's keys, then those reaching its first m groups, m = nvalid .. 1,
  // then the tiles before its first key.
  int it = ntiles - 1;
  auto full_run = [&](auto groups) {
    for (; it >= full_start; --it) step(it, Full{}, groups);
  };
  if (nvalid == NG) full_run(std::integral_constant<int, NG>{});
  else if constexpr (NG >= 2) {
    if (nvalid == 1) full_run(std::integral_constant<int, 1>{});
    else if constexpr (NG >= 3) {
      if (nvalid == 2) full_run(std::integral_constant<int, 2>{});
      else if constexpr (NG >= 4) {
        if (nvalid == 3) full_run(std::integral_constant<int, 3>{});
      }
    }
  }
  // m groups reached: down to the first tile that reaches group m.
  auto masked_run = [&](auto groups) {
    constexpr int M = decltype(groups)::value;
    if (M > nvalid) return;
    for (const int e = uni(live(M - 1)); it >= e; --it) step(it, Masked{}, groups);
  };
  static_assert(NG <= 4, "runs are written out for up to four groups");
  if constexpr (NG >= 4) masked_run(std::integral_constant<int, 4>{});
  if constexpr (NG >= 3) masked_run(std::integral_constant<int, 3>{});
  if constexpr (NG >= 2) masked_run(std::integral_constant<int, 2>{});
  masked_run(std::integral_constant<int, 1>{});
  // Tiles before the wave's first key (all of them for a wave without
  // candidates, which only a segment's last key block has).
  for (; it >= 0; --it) step(it, Skip{}, std::integral_constant<int, 1>{});

  float *out = a.partial + ((long long)hb * a.RCmax + rc) * a.N;
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    const float v = cs[n] + __shfl_xor(cs[n], 32, 64);
    const int c = gbase(n) + (lane & 31);
    if (lane < 32 && c < kb1) out[c] = v;
  }
}

// score[c] = (sum over head blocks and row chunks that see c) / (Hq * n_b).
// A workgroup covers 32 columns; thread t sums head blocks t/32, t/32 + 8, ...
// over their row chunks (four independent partial sums, so the loads overlap),
// then the eight per-thread totals of a column are added in head-block-group
// order.  The order is fixed, so the result is deterministic.
__global__ __launch_bounds__(256) void colscore_finalize(AttnArgs a, float *score) {
  __shared__ float part[8][33];
  const int cl = threadIdx.x & 31, hg = threadIdx.x >> 5;
  const int c = blockIdx.x * 32 + cl;
  float sum = 0.f;
  int b = 0;
  if (c < a.N) {
    const DevLayout &L = a.L;
    const int s = upper_index(L.cu_cands, 0, L.S, c);  // image holding c
    b = upper_index(L.cu_images, 0, L.B, s);           // request holding image s
    const int seg = (a.segkind == SEG_REQ) ? b : s;
    int seg_lo, seg_hi;
    seg_tokens(L, a.segkind, seg, seg_lo, seg_hi);
    const int tok = L.img_start[s] + (c - L.cu_cands[s]);
    const int nrc = chunk_count(seg_hi - seg_lo, a.RC, a.RCF);
    const int rc0 = a.causal ? chunk_of(tok - seg_lo, seg_hi - seg_lo, a.RC, a.RCF) : 0;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int hb = hg; hb < a.nhb; hb += 8) {
      const float *p = a.partial + (long long)hb * a.RCmax * a.N + c;
      int rc = rc0;
      for (; rc + 4 <= nrc; rc += 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += p[(long long)(rc + j) * a.N];
      }
      for (; rc < nrc; ++rc) acc[0] += p[(long long)rc * a.N];
    }
    sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  part[hg][cl] = sum;
  __syncthreads();
  if (hg == 0 && c < a.N) {
    float t = part[0][cl];
#pragma unroll
    for (int j = 1; j < 8; ++j) t += part[j][cl];
    const int n_b = a.L.cu_seqlens[b + 1] - a.L.cu_seqlens[b];
    score[c] = t / ((float)a.hq * (float)n_b);
  }
}

// ---------------------------------------------------------------------------
// Launchers.  NG (resident 32-row groups per wave) is NGMAX<DT, D> or 1.
// ---------------------------------------------------------------------------
namespace {

template <int DT, int D>
constexpr int kNGMax = lse_groups(DT, D);
template <int DT, int D>
constexpr int kColNG = colscore_groups(DT, D);

// The permuted variants exist for the widest group count only (the
// one-group fallback serves small grids, where order matters little).
template <int DT, int D, int NG>
hipError_t lse_go(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  const int grid = (int)((p.total_jobs + 7) / 8 * 8);
  if constexpr (NG == kNGMax<DT, D>) {
    if (perm != nullptr) {
      hipLaunchKernelGGL((lse_kernel<DT, D, NG, true>), dim3(grid), dim3(256), 0, s, a, PermArg<true>{*perm});
      return hipGetLastError();
    }
  }
  AttnArgs b = a;
  b.order = kOrderPlain;
  hipLaunchKernelGGL((lse_kernel<DT, D, NG, false>), dim3(grid), dim3(256), 0, s, b, PermArg<false>{});
  return hipGetLastError();
}

template <int DT, int D, int NG>
hipError_t col_go(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  const int grid = (int)((p.total_jobs + 7) / 8 * 8);
  if constexpr (NG == kColNG<DT, D>) {
    if (perm != nullptr) {
      hipLaunchKernelGGL((colscore_kernel<DT, D, NG, true>), dim3(grid), dim3(256), 0, s, a,
                         PermArg<true>{*perm});
      return hipGetLastError();
    }
  }
  AttnArgs b = a;
  b.order = kOrderPlain;
  hipLaunchKernelGGL((colscore_kernel<DT, D, NG, false>), dim3(grid), dim3(256), 0, s, b, PermArg<false>{});
  return hipGetLastError();
}

template <int DT, int D>
hipError_t lse_ng(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  if (p.NT == kNGMax<DT, D>) return lse_go<DT, D, kNGMax<DT, D>>(p, a, perm, s);
  return lse_go<DT, D, 1>(p, a, perm, s);
}
template <int DT, int D>
hipError_t col_ng(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  if (p.NT == kColNG<DT, D>) return col_go<DT, D, kColNG<DT, D>>(p, a, perm, s);
  return col_go<DT, D, 1>(p, a, perm, s);
}

// fp8 runs head_dim 64 and 128 only (whole 64-wide k chunks); the host
// rejects the others before any launch.
template <int DT>
hipError_t lse_d(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  if constexpr (DT == TSEL_FP8_E4M3) {
    return p.D == 64 ? lse_ng<DT, 64>(p, a, perm, s) : lse_ng<DT, 128>(p, a, perm, s);
  } else {
    switch (p.D) {
      case 64: return lse_ng<DT, 64>(p, a, perm, s);
      case 72: return lse_ng<DT, 72>(p, a, perm, s);
      case 80: return lse_ng<DT, 80>(p, a, perm, s);
      case 96: return lse_ng<DT, 96>(p, a, perm, s);
      default: return lse_ng<DT, 128>(p, a, perm, s);
    }
  }
}
template <int DT>
hipError_t col_d(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  if constexpr (DT == TSEL_FP8_E4M3) {
    return p.D == 64 ? col_ng<DT, 64>(p, a, perm, s) : col_ng<DT, 128>(p, a, perm, s);
  } else {
    switch (p.D) {
      case 64: return col_ng<DT, 64>(p, a, perm, s);
      case 72: return col_ng<DT, 72>(p, a, perm, s);
      case 80: return col_ng<DT, 80>(p, a, perm, s);
      case 96: return col_ng<DT, 96>(p, a, perm, s);
      default: return col_ng<DT, 128>(p, a, perm, s);
    }
  }
}

}  // namespace

hipError_t launch_lse(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s) {
  if (p.total_jobs == 0) return hipSuccess;
  hipError_t e;
  switch (p.dtype) {
    case TSEL_F32: e = lse_d<TSEL_F32>(p, a, perm, s); break;
    case TSEL_F16: e = lse_d<TSEL_F16>(p, a, perm, s); break;
    case TSEL_FP8_E4M3: e = lse_d<TSEL_FP8_E4M3>(p, a, perm, s); break;
    default: e = lse_d<TSEL_BF16>(p, a, perm, s); break;
  }
  if (e != hipSuccess || a.KS == 0) return e;
  const long long rows = (long long)a.hq * a.L.T;
  hipLaunchKernelGGL(lse_merge, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_colscore(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, float *score,
                           hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (p.total_jobs > 0) {
    switch (p.dtype) {
      case TSEL_F32: e = col_d<TSEL_F32>(p, a, perm, s); break;
      case TSEL_F16: e = col_d<TSEL_F16>(p, a, perm, s); break;
      case TSEL_FP8_E4M3: e = col_d<TSEL_FP8_E4M3>(p, a, perm, s); break;
      default: e = col_d<TSEL_BF16>(p, a, perm, s); break;
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colscore_finalize, dim3((a.N + 31) / 32), dim3(256), 0, s, a, score);
  return hipGetLastError();
}

}  // namespace tsel
