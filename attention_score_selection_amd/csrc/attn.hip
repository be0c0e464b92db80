// Softmax LSE and column-score kernels for gfx950.
//
// Both kernels share one shape: a RESIDENT operand held in VGPRs for the whole
// workgroup lifetime (as the B operand of v_mfma_f32_16x16x32_{bf16,f16}, or
// of eight v_mfma_f32_16x16x4_f32 for fp32), and a STREAMED operand that the
// workgroup stages through LDS in tiles of 16 rows (the A operand).  The
// 16x16 accumulator then holds, per lane, one column of the resident side
// (lane % 16) and four rows of the streamed side (4 * (lane / 16) + r), so
// every reduction the method needs along the streamed side happens inside the
// lane; the four lane groups are combined once at the very end.
//
//  * LSE (per-row softmax normaliser, REDtech article section 3.2 reuses it):
//    resident = 128 query rows per wave, streamed = key tiles.  Rows reduce
//    in-lane.
//  * Column score (attention a vision token receives, LiteVLM review formula
//    section; column-wise reduction without materialising the attention
//    matrix, REDtech article section 3.2): resident = 128 candidate keys per
//    wave, streamed = query-row tiles together with their LSE.  Columns
//    reduce in-lane; nothing of P leaves the registers.
//
// Heads that share a KV head are folded into the row dimension (F heads per
// tile row group), so one resident key fragment serves F query heads.
//
// The k-dimension of a 32-wide chunk is split over the four lane groups, 8
// consecutive values each (16 B for 16-bit types).  For fp32 the same 8
// values feed eight 16x16x4 steps; A and B use the same permutation of k, so
// the contraction is unchanged.
#include "device.h"

namespace tsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int DT> struct Elem { static constexpr int ES = 2; };
template <> struct Elem<TSEL_F32> { static constexpr int ES = 4; };

template <int DT>
struct Chunk {
  uint4 v[Elem<DT>::ES / 2];
};

template <int DT>
__device__ __forceinline__ void zero_chunk(Chunk<DT> &c) {
#pragma unroll
  for (int i = 0; i < Elem<DT>::ES / 2; ++i) c.v[i] = make_uint4(0u, 0u, 0u, 0u);
}

template <int DT>
__device__ __forceinline__ void load_chunk(Chunk<DT> &c, const char *p) {
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
  for (int i = 0; i < Elem<DT>::ES / 2; ++i) c.v[i] = q[i];
}

template <int DT>
__device__ __forceinline__ f32x4 mma(const Chunk<DT> &a, const Chunk<DT> &b, f32x4 acc);

template <>
__device__ __forceinline__ f32x4 mma<TSEL_BF16>(const Chunk<TSEL_BF16> &a, const Chunk<TSEL_BF16> &b,
                                                f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[0]),
                                                 __builtin_bit_cast(bf16x8, b.v[0]), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma<TSEL_F16>(const Chunk<TSEL_F16> &a, const Chunk<TSEL_F16> &b,
                                               f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a.v[0]),
                                                __builtin_bit_cast(f16x8, b.v[0]), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma<TSEL_F32>(const Chunk<TSEL_F32> &a, const Chunk<TSEL_F32> &b,
                                               f32x4 acc) {
  const f32x4v a0 = __builtin_bit_cast(f32x4v, a.v[0]), a1 = __builtin_bit_cast(f32x4v, a.v[1]);
  const f32x4v b0 = __builtin_bit_cast(f32x4v, b.v[0]), b1 = __builtin_bit_cast(f32x4v, b.v[1]);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[s], b0[s], acc, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[s], b1[s], acc, 0, 0, 0);
  return acc;
}

// Geometry of one streamed 16-row tile in LDS.
template <int DT, int D>
struct Geom {
  static constexpr int ES = Elem<DT>::ES;
  static constexpr int KCH = (D + 31) / 32;          // 32-wide k chunks
  static constexpr int ROW = KCH * 32 * ES;          // bytes of a zero-padded row
  static constexpr int RS = ROW + 16;                // LDS row stride (bank spread)
  static constexpr int UNITS = ROW / 16;             // 16-byte units per row
  static constexpr int UPT = (16 * UNITS + 255) / 256;  // units per thread (256 threads)
  static constexpr int TILE = 16 * RS;               // bytes of one tile
  static constexpr int VALID_UNITS = D * ES / 16;    // units that hold real data
};

// Register staging of one streamed tile: global -> VGPR -> LDS.
template <int DT, int D>
struct Stage {
  using G = Geom<DT, D>;
  uint4 r[G::UPT];

  // rowptr(row) returns the global address of a row, or nullptr (zero row).
  template <typename RowPtr>
  __device__ __forceinline__ void load(RowPtr rowptr) {
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
      const int u = threadIdx.x + 256 * i;
      r[i] = make_uint4(0u, 0u, 0u, 0u);
      if (u < 16 * G::UNITS) {
        const int row = u / G::UNITS, col = u % G::UNITS;
        const char *p = rowptr(row);
        if (p != nullptr && col < G::VALID_UNITS) r[i] = *reinterpret_cast<const uint4 *>(p + col * 16);
      }
    }
  }
  __device__ __forceinline__ void store(char *tile) const {
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
      const int u = threadIdx.x + 256 * i;
      if (u < 16 * G::UNITS) {
        const int row = u / G::UNITS, col = u % G::UNITS;
        *reinterpret_cast<uint4 *>(tile + row * G::RS + col * 16) = r[i];
      }
    }
  }
};

// This lane's fragment (row lane%16, k values 32*kc + 8*(lane/16) .. +8) of
// an LDS tile.
template <int DT, int D>
__device__ __forceinline__ void read_frag(Chunk<DT> (&f)[(D + 31) / 32], const char *tile) {
  using G = Geom<DT, D>;
  const int lane = lane_id();
  const char *p = tile + (lane & 15) * G::RS + (lane >> 4) * 8 * G::ES;
#pragma unroll
  for (int kc = 0; kc < G::KCH; ++kc) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p + kc * 32 * G::ES);
#pragma unroll
    for (int i = 0; i < G::ES / 2; ++i) f[kc].v[i] = q[i];
  }
}

// Load the resident fragments of NT 16-row groups straight from global memory.
template <int DT, int D, int NT, typename RowPtr>
__device__ __forceinline__ void load_resident(Chunk<DT> (&res)[NT][(D + 31) / 32], RowPtr rowptr) {
  using G = Geom<DT, D>;
  const int lane = lane_id();
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const char *p = rowptr(n * 16 + (lane & 15));
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc) {
      const int e = 32 * kc + 8 * (lane >> 4);
      if (p != nullptr && e < D) load_chunk<DT>(res[n][kc], p + e * G::ES);
      else zero_chunk<DT>(res[n][kc]);
    }
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// ---------------------------------------------------------------------------
// LSE kernel.
// Job = (head block hb, segment a, row block rb): TB tokens x F heads of one
// segment; each of the 4 waves owns NT*16 of those rows.  Keys stream in
// tiles of 16 over [seg_lo, key_hi).
// ---------------------------------------------------------------------------

// One pass over key tiles [t0, t1).  MAXMODE: acc = running max of the raw
// logit over this lane's keys.  Otherwise acc = running sum of
// exp2(c1*s - m) over this lane's keys.
template <int DT, int D, int NT, bool MAXMODE>
__device__ __forceinline__ void lse_pass(char *smem, const AttnArgs &a, int g, int key_lo,
                                         int key_hi, int t0, int t1,
                                         const Chunk<DT> (&qf)[NT][(D + 31) / 32],
                                         const int (&qtok)[NT], int wtok_min, int wtok_max,
                                         const float (&m)[NT], float (&acc)[NT]) {
  using G = Geom<DT, D>;
  const int lane = lane_id();
  const char *kbase = reinterpret_cast<const char *>(a.k);
  auto rowptr = [&](int it) {
    return [=](int r) -> const char * {
      const int key = key_lo + 16 * it + r;
      if (key >= key_hi) return nullptr;
      return kbase + ((long long)key * a.k_st + (long long)g * a.k_sh) * G::ES;
    };
  };
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = MAXMODE ? kNegInf : 0.0f;

  Stage<DT, D> st;
  st.load(rowptr(t0));
  st.store(smem);
  if (t0 + 1 < t1) st.load(rowptr(t0 + 1));
  __syncthreads();
  for (int it = t0; it < t1; ++it) {
    const char *tile = smem + ((it - t0) & 1) * G::TILE;
    const int k0 = key_lo + 16 * it;
    if (!(a.causal && k0 > wtok_max)) {  // otherwise no row of this wave sees the tile
    Chunk<DT> af[G::KCH];
    read_frag<DT, D>(af, tile);
    const bool need_mask = (k0 + 16 > key_hi) || (a.causal && k0 + 15 > wtok_min);
    const int kl = k0 + 4 * (lane >> 4);  // this lane's keys: kl + r
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < G::KCH; ++kc) s = mma<DT>(af[kc], qf[n][kc], s);
      if (MAXMODE) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = s[r];
          if (need_mask) {
            const int key = kl + r;
            const bool vis = key < key_hi && (!a.causal || key <= qtok[n]);
            v[r] = vis ? v[r] : kNegInf;
          }
        }
        acc[n] = fmaxf(acc[n], fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
      } else {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = fast_exp2(fmaf(s[r], a.c1, -m[n]));
          if (need_mask) {
            const int key = kl + r;
            const bool vis = key < key_hi && (!a.causal || key <= qtok[n]);
            p[r] = vis ? p[r] : 0.0f;
          }
        }
        acc[n] += (p[0] + p[1]) + (p[2] + p[3]);
      }
    }
    }
    if (it + 1 < t1) {
      st.store(smem + ((it + 1 - t0) & 1) * G::TILE);
      if (it + 2 < t1) st.load(rowptr(it + 2));
    }
    __syncthreads();
  }
}

template <int DT, int D, int NT>
__global__ __launch_bounds__(256, 2) void lse_kernel(AttnArgs a) {
  using G = Geom<DT, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::TILE];
  __shared__ int s_bad;

  const int job = xcd_job(blockIdx.x, gridDim.x);
  if (job >= a.total_jobs) return;
  const int hb = job / a.jobs_per_hb;
  const int rj = job % a.jobs_per_hb;
  const int TB = a.TB;
  int local;
  const int seg = find_segment(a.nseg, rj, [&](int s) {
    int lo, hi;
    seg_tokens(a.L, a.segkind, s, lo, hi);
    return (hi - lo + TB - 1) / TB;
  }, local);
  if (seg < 0) return;
  int seg_lo, seg_hi;
  seg_tokens(a.L, a.segkind, seg, seg_lo, seg_hi);
  const int nrb = (seg_hi - seg_lo + TB - 1) / TB;
  const int rb = a.causal ? nrb - 1 - local : local;  // causal: heaviest row blocks first
  const int tok_lo = seg_lo + rb * TB;
  const int tok_hi = min(tok_lo + TB, seg_hi);

  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int F = a.F;
  const int wtok0 = tok_lo + w * (NT * 16 / F);
  const int wtok_max = wtok0 + NT * 16 / F - 1;
  const int h0 = hb * F;
  const int g = h0 / a.hg;
  const int key_lo = seg_lo;
  const int key_hi = a.causal ? tok_hi : seg_hi;
  const int ntiles = (key_hi - key_lo + 15) / 16;

  // Resident queries: row q of this wave is (token wtok0 + q / F, head h0 + q % F).
  Chunk<DT> qf[NT][G::KCH];
  int qtok[NT];
  const char *qbase = reinterpret_cast<const char *>(a.q);
  load_resident<DT, D, NT>(qf, [&](int q) -> const char * {
    const int t = wtok0 + q / F;
    if (t >= tok_hi) return nullptr;
    return qbase + ((long long)t * a.q_st + (long long)(h0 + q % F) * a.q_sh) * G::ES;
  });
#pragma unroll
  for (int n = 0; n < NT; ++n) qtok[n] = wtok0 + (n * 16 + (lane & 15)) / F;

  // Offset m: max logit of the first key tile (which every row sees) plus 32
  // (log2 units); the sum pass then cannot overflow unless a later logit
  // exceeds it by ~100, which the check below catches.
  float m[NT], acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) m[n] = 0.f;
  if (threadIdx.x == 0) s_bad = 0;
  lse_pass<DT, D, NT, true>(smem, a, g, key_lo, key_hi, 0, 1, qf, qtok, wtok0, wtok_max, m, acc);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float mx = acc[n];
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    m[n] = mx * a.c1 + 32.0f;
  }
  lse_pass<DT, D, NT, false>(smem, a, g, key_lo, key_hi, 0, ntiles, qf, qtok, wtok0, wtok_max, m, acc);
  float tot[NT];
  bool ok = true;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float v = acc[n];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    tot[n] = v;
    if (qtok[n] < tok_hi) ok = ok && (v <= 0x1p100f) && (v >= 0x1p-100f);  // false for NaN
  }
  if (!ok) s_bad = 1;
  __syncthreads();
  if (s_bad) {
    // Exact two-pass fallback: true row max, then the sum against it.
    lse_pass<DT, D, NT, true>(smem, a, g, key_lo, key_hi, 0, ntiles, qf, qtok, wtok0, wtok_max, m, acc);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float mx = acc[n];
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      m[n] = mx * a.c1;
    }
    lse_pass<DT, D, NT, false>(smem, a, g, key_lo, key_hi, 0, ntiles, qf, qtok, wtok0, wtok_max, m, acc);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float v = acc[n];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      tot[n] = v;
    }
  }
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int q = n * 16 + lane;
      const int t = wtok0 + q / F;
      if (t < tok_hi) {
        const float lse2 = m[n] + __log2f(tot[n]);
        a.lse_out[(long long)(h0 + q % F) * a.L.T + t] = lse2 * 0.69314718055994530942f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Column-score kernel.
// Job = (head block hb, segment a, row chunk rc, key block kb).  Each wave
// holds NT*16 candidate keys; query-row tiles of 16 rows (16/F tokens x F
// heads) and their LSE stream through LDS; per-column partial sums go to
// partial[(hb*RCmax + rc)*N + c].
// ---------------------------------------------------------------------------
template <int DT, int D, int NT>
__global__ __launch_bounds__(256, 2) void colscore_kernel(AttnArgs a) {
  using G = Geom<DT, D>;
  constexpr int BUF = G::TILE + 64;  // tile + 16 floats of LSE (log2 units)
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

  const int job = xcd_job(blockIdx.x, gridDim.x);
  if (job >= a.total_jobs) return;
  const int hb = job / a.jobs_per_hb;
  const int rj = job % a.jobs_per_hb;
  const int KB = a.KB, RC = a.RC;
  int local;
  const int seg = find_segment(a.nseg, rj, [&](int s) {
    int lo, hi, sl, sh, cl, ch;
    seg_tokens(a.L, a.segkind, s, lo, hi);
    seg_images(a.L, a.segkind, s, sl, sh, cl, ch);
    return ((ch - cl + KB - 1) / KB) * ((hi - lo + RC - 1) / RC);
  }, local);
  if (seg < 0) return;
  int seg_lo, seg_hi, s_lo, s_hi, c_lo, c_hi;
  seg_tokens(a.L, a.segkind, seg, seg_lo, seg_hi);
  seg_images(a.L, a.segkind, seg, s_lo, s_hi, c_lo, c_hi);
  const int nkb = (c_hi - c_lo + KB - 1) / KB;
  const int rc = local / nkb, kb = local % nkb;
  const int kb0 = c_lo + kb * KB;
  const int kb1 = min(kb0 + KB, c_hi);
  const int chunk_lo = seg_lo + rc * RC;
  const int chunk_hi = min(chunk_lo + RC, seg_hi);
  const int first_ktok = cand_token(a.L, s_lo, s_hi, kb0);
  const int row_lo = a.causal ? max(chunk_lo, first_ktok) : chunk_lo;
  if (row_lo >= chunk_hi) return;  // no row of this chunk sees any key of the block

  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int F = a.F;
  const int h0 = hb * F;
  const int g = h0 / a.hg;
  const int wc0 = kb0 + w * NT * 16;
  const int wlast = min(wc0 + NT * 16, kb1) - 1;
  // Largest key token of this wave (candidates are in token order).
  const int wkmax = (wlast >= wc0) ? cand_token(a.L, s_lo, s_hi, wlast) : -1;
  const int wkmin = (wlast >= wc0) ? cand_token(a.L, s_lo, s_hi, wc0) : 0x7fffffff;

  // Resident keys.
  Chunk<DT> kf[NT][G::KCH];
  int ktok[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int c = wc0 + n * 16 + (lane & 15);
    ktok[n] = (c < kb1) ? cand_token(a.L, s_lo, s_hi, c) : 0x7fffffff;
  }
  const char *kbase = reinterpret_cast<const char *>(a.k);
  load_resident<DT, D, NT>(kf, [&](int j) -> const char * {
    const int t = ktok[j >> 4];
    if (t == 0x7fffffff) return nullptr;
    return kbase + ((long long)t * a.k_st + (long long)g * a.k_sh) * G::ES;
  });

  const int tpt = 16 / F;  // tokens per streamed tile
  const int ntiles = (chunk_hi - row_lo + tpt - 1) / tpt;
  const char *qbase = reinterpret_cast<const char *>(a.q);
  const long long T = a.L.T;
  auto rowptr = [&](int it) {
    return [=](int r) -> const char * {
      const int t = row_lo + it * tpt + r / F;
      if (t >= chunk_hi) return nullptr;
      return qbase + ((long long)t * a.q_st + (long long)(h0 + r % F) * a.q_sh) * G::ES;
    };
  };
  auto lse_load = [&](int it) -> float {
    const int r = threadIdx.x;
    const int t = row_lo + it * tpt + r / F;
    if (t >= chunk_hi) return kPosInf;
    return a.lse_in[(long long)(h0 + r % F) * T + t] * 1.44269504088896340736f;
  };

  float cs[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) cs[n] = 0.f;

  Stage<DT, D> st;
  float lreg = 0.f;
  st.load(rowptr(0));
  if (threadIdx.x < 16) lreg = lse_load(0);
  st.store(smem);
  if (threadIdx.x < 16) reinterpret_cast<float *>(smem + G::TILE)[threadIdx.x] = lreg;
  if (ntiles > 1) {
    st.load(rowptr(1));
    if (threadIdx.x < 16) lreg = lse_load(1);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const char *buf = smem + (it & 1) * BUF;
    const int tt0 = row_lo + it * tpt;
    if (!(a.causal && tt0 + tpt - 1 < wkmin)) {  // otherwise every row precedes every key
    Chunk<DT> af[G::KCH];
    read_frag<DT, D>(af, buf);
    const f32x4v l4 = *reinterpret_cast<const f32x4v *>(buf + G::TILE + 16 * (lane >> 4));
    const bool need_mask = a.causal && tt0 < wkmax;
    int rtok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rtok[r] = tt0 + (4 * (lane >> 4) + r) / F;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < G::KCH; ++kc) s = mma<DT>(af[kc], kf[n][kc], s);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = fast_exp2(fmaf(s[r], a.c1, -l4[r]));
        if (need_mask) p[r] = (ktok[n] <= rtok[r]) ? p[r] : 0.0f;
      }
      cs[n] += (p[0] + p[1]) + (p[2] + p[3]);
    }
    }
    if (it + 1 < ntiles) {
      char *nb = smem + ((it + 1) & 1) * BUF;
      st.store(nb);
      if (threadIdx.x < 16) reinterpret_cast<float *>(nb + G::TILE)[threadIdx.x] = lreg;
      if (it + 2 < ntiles) {
        st.load(rowptr(it + 2));
        if (threadIdx.x < 16) lreg = lse_load(it + 2);
      }
    }
    __syncthreads();
  }
  float *out = a.partial + ((long long)hb * a.RCmax + rc) * a.N;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float v = cs[n];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    const int c = wc0 + n * 16 + (lane & 15);
    if ((lane >> 4) == 0 && c < kb1) out[c] = v;
  }
}

// score[c] = (sum over head blocks and row chunks that see c, fixed order) / (Hq * n_b).
__global__ __launch_bounds__(256) void colscore_finalize(AttnArgs a, float *score) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.N) return;
  const DevLayout &L = a.L;
  const int s = upper_index(L.cu_cands, 0, L.S, c);  // image holding c
  const int b = upper_index(L.cu_images, 0, L.B, s);  // request holding image s
  const int seg = (a.segkind == SEG_REQ) ? b : s;
  int seg_lo, seg_hi;
  seg_tokens(L, a.segkind, seg, seg_lo, seg_hi);
  const int tok = L.img_start[s] + (c - L.cu_cands[s]);
  const int nrc = (seg_hi - seg_lo + a.RC - 1) / a.RC;
  const int rc0 = a.causal ? (tok - seg_lo) / a.RC : 0;
  float sum = 0.f;
  for (int hb = 0; hb < a.nhb; ++hb) {
    const float *p = a.partial + (long long)hb * a.RCmax * a.N + c;
    for (int rc = rc0; rc < nrc; ++rc) sum += p[(long long)rc * a.N];
  }
  const int n_b = L.cu_seqlens[b + 1] - L.cu_seqlens[b];
  score[c] = sum / ((float)a.hq * (float)n_b);
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
namespace {

template <int DT, int D, int NT>
hipError_t lse_go(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  const int grid = (int)((p.total_jobs + 7) / 8 * 8);
  hipLaunchKernelGGL((lse_kernel<DT, D, NT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D, int NT>
hipError_t col_go(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  const int grid = (int)((p.total_jobs + 7) / 8 * 8);
  hipLaunchKernelGGL((colscore_kernel<DT, D, NT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Eight resident 16-row groups fit the register budget except for fp32 with
// head_dim > 64, which only gets the four-group variant.
template <int DT, int D>
constexpr bool kWide = !(DT == TSEL_F32 && D > 64);

template <int DT, int D>
hipError_t lse_nt(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  if constexpr (kWide<DT, D>) {
    if (p.NT == 8) return lse_go<DT, D, 8>(p, a, s);
  }
  return lse_go<DT, D, 4>(p, a, s);
}
template <int DT, int D>
hipError_t col_nt(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  if constexpr (kWide<DT, D>) {
    if (p.NT == 8) return col_go<DT, D, 8>(p, a, s);
  }
  return col_go<DT, D, 4>(p, a, s);
}

template <int DT>
hipError_t lse_d(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  switch (p.D) {
    case 64: return lse_nt<DT, 64>(p, a, s);
    case 80: return lse_nt<DT, 80>(p, a, s);
    case 96: return lse_nt<DT, 96>(p, a, s);
    default: return lse_nt<DT, 128>(p, a, s);
  }
}
template <int DT>
hipError_t col_d(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  switch (p.D) {
    case 64: return col_nt<DT, 64>(p, a, s);
    case 80: return col_nt<DT, 80>(p, a, s);
    case 96: return col_nt<DT, 96>(p, a, s);
    default: return col_nt<DT, 128>(p, a, s);
  }
}

}  // namespace

hipError_t launch_lse(const AttnPlan &p, const AttnArgs &a, hipStream_t s) {
  if (p.total_jobs == 0) return hipSuccess;
  switch (p.dtype) {
    case TSEL_F32: return lse_d<TSEL_F32>(p, a, s);
    case TSEL_F16: return lse_d<TSEL_F16>(p, a, s);
    default: return lse_d<TSEL_BF16>(p, a, s);
  }
}

hipError_t launch_colscore(const AttnPlan &p, const AttnArgs &a, float *score, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (p.total_jobs > 0) {
    switch (p.dtype) {
      case TSEL_F32: e = col_d<TSEL_F32>(p, a, s); break;
      case TSEL_F16: e = col_d<TSEL_F16>(p, a, s); break;
      default: e = col_d<TSEL_BF16>(p, a, s); break;
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colscore_finalize, dim3((a.N + 255) / 256), dim3(256), 0, s, a, score);
  return hipGetLastError();
}

}  // namespace tsel
