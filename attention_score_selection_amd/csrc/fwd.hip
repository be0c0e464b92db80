// Attention forward with the LSE as a by-product, for gfx950.
//
// The REDtech article (section 3.2) reuses the softmax normaliser that the
// layer's FlashAttention pass already computes; this kernel is that pass for
// bf16/f16 inputs: O = softmax(scale * Q K^T) V per query head and row over
// the row's visible keys (same masks and segments as the selection kernels),
// and LSE = log sum exp of the same logits.
//
// Job = (head block, segment, row block) as in the LSE kernel; each of the 4
// waves keeps one 32-row query group resident (the MFMA's B operand).  Per
// 32-key tile: S^T = K_tile . Q^T on v_mfma_f32_32x32x16 (lane = query row,
// registers = 16 of the 32 keys), an online softmax in log2 units per lane,
// and O^T += V_tile^T . P^T, where P^T is the B operand straight from the S^T
// registers (converted to the input type) and V^T is read from the row-major
// value tile with gfx950's transposing LDS read (ds_read_b64_tr_b16).  The
// contraction's k slots of lane half h are the keys 16c + {0..3, 8..11} + 4h
// of chunk c, which is how the S^T accumulator already holds them; each group
// of four keys is one transposing read.  Key and value tiles reach LDS through
// the LDS-direct form of the buffer load, one tile ahead.
//
// The running maximum only moves when a tile's maximum exceeds it by more
// than 2^8 (so P stays below 2^8, safe for f16 operands); the accumulators are
// rescaled then, and the LSE uses the final maximum and sum.
#include "vtile.h"

namespace tsel {

namespace {

constexpr float kRescale = 8.0f;  // log2 headroom before the running max moves

template <int DT> struct PackT;
template <> struct PackT<TSEL_BF16> { typedef __bf16 T; };
template <> struct PackT<TSEL_F16> { typedef _Float16 T; };

// Eight probabilities (k slots 0..7 of one lane half) as one MFMA operand.
template <int DT>
__device__ __forceinline__ Chunk<DT> pack_p(const float (&p)[16], int c) {
  typedef typename PackT<DT>::T E;
  typedef E E8 __attribute__((ext_vector_type(8)));
  E8 x;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (E)p[8 * c + j];
  Chunk<DT> r;
  r.v[0] = __builtin_bit_cast(uint4, x);
  return r;
}

// V^T fragment of column group dg, key chunk c: lane column dg*32 + lane%32,
// keys 16c + 4h + {0..3} and 16c + 8 + 4h + {0..3} (h = lane / 32).  Columns
// from D on read the row's zero padding and only reach O^T rows that are
// never written out.
template <int DT, int D>
__device__ __forceinline__ Chunk<DT> read_vt(const char *vtile, int lane_off, int dg, int c) {
  using G = VGeom<DT, D>;
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  // vtile + vt_read_offset(lane, dg, c, 0 / 1), the lane part held in lane_off.
  const char *p = vtile + lane_off + 16 * c * G::RS + dg * 32 * G::ES;
  const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)p);
  const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p + 8 * G::RS));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  Chunk<DT> r;
  r.v[0] = make_uint4(a.x, a.y, b.x, b.y);
  return r;
}

template <int DT, int D>
__global__ __launch_bounds__(256, 3) void fwd_kernel(FwdArgs fa) {
  using G = Geom<DT, D>;
  constexpr int DG = OGroups<D>::DG;
  using VG = VGeom<DT, D>;
  static_assert(OGroups<D>::DG * 32 * G::ES <= VG::RS, "padded columns stay inside a value row");
  constexpr int BUF = G::TILE + VG::TILE;  // key tile, then value tile
  __shared__ __attribute__((aligned(16))) char stage0[BUF];
  __shared__ __attribute__((aligned(16))) char stage1[BUF];
  const AttnArgs &a = fa.at;

  const int job = xcd_job(blockIdx.x, gridDim.x);
  if (job >= a.total_jobs) return;
  const int TB = a.TB;
  auto count = [&](int s) {
    int lo, hi;
    seg_tokens(a.L, a.segkind, s, lo, hi);
    return (hi - lo + TB - 1) / TB;
  };
  int hb, rj;
  job_plain(a, job, hb, rj);
  int local;
  const int seg = find_segment(a.nseg, rj, count, local);
  if (seg < 0) return;
  int seg_lo, seg_hi;
  seg_tokens(a.L, a.segkind, seg, seg_lo, seg_hi);
  seg_lo = uni(seg_lo);
  seg_hi = uni(seg_hi);
  const int nrb = (seg_hi - seg_lo + TB - 1) / TB;
  const int rb = a.causal ? nrb - 1 - local : local;  // causal: heaviest row blocks first
  const int tok_lo = uni(seg_lo + rb * TB);
  const int tok_hi = uni(min(tok_lo + TB, seg_hi));

  const int lane = lane_id(), w = uni(threadIdx.x >> 6);
  const int F = a.F;
  const int wtok0 = uni(tok_lo + w * (kRows / F));
  const int wtok_max = uni(wtok0 + kRows / F - 1);
  const int h0 = hb * F;
  const int g = h0 / a.hg;
  const int key_lo = seg_lo;
  const int key_hi = uni(a.causal ? tok_hi : seg_hi);
  const int ntiles = uni((key_hi - key_lo + kRows - 1) / kRows);

  // Resident queries: row r of this wave is (token wtok0 + r / F, head h0 + r % F).
  Chunk<DT> qf[1][G::KCH];
  const char *qbase = reinterpret_cast<const char *>(a.q);
  load_resident<DT, D, 1>(qf, [&](int r) -> const char * {
    const int t = wtok0 + r / F;
    if (t >= tok_hi) return nullptr;
    return qbase + ((long long)t * a.q_st + (long long)(h0 + r % F) * a.q_sh) * G::ES;
  });
  const int qtok = wtok0 + (lane & 31) / F;
  wait_vmem();

  // Key and value tiles it: rows key_lo + 32*it + r of KV head g.
  const char *kbase = reinterpret_cast<const char *>(a.k) + (long long)g * a.k_sh * G::ES;
  const long long krow = a.k_st * G::ES;
  const char *vbase = reinterpret_cast<const char *>(fa.v) + (long long)g * fa.v_sh * G::ES;
  const long long vrow = fa.v_st * G::ES;
  StageDirect<DT, D> sk;
  StageDirect<DT, D, VG> sv;
  sk.init([&](int r) { return r * (int)krow; });
  sv.init([&](int r) { return r * (int)vrow; });
  const int vt_off = vt_lane_offset_of<DT, D>(lane_id());
  // Start copying key and value tile it into buffer dst (one scalar base per
  // tile).  Rows past key_hi read as zero: the last tile's resources end
  // after its valid rows (a valid row's units lie below nv row strides, every
  // later row's at or above), so no per-lane row test is needed.
  auto load = [&](int it, char *dst) {
    const long long first = key_lo + kRows * it;
    const int nv = key_hi - (int)first;
    const bool whole = nv >= kRows;
    const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kbase + first * krow, whole ? kOOB : nv * (int)krow);
    const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vbase + first * vrow, whole ? kOOB : nv * (int)vrow);
    sk.template load_at<false>(dst, krs, 0, kRows);
    sv.template load_at<false>(dst + G::TILE, vrs, 0, kRows);
  };

  f32x16 o[DG];
#pragma unroll
  for (int dg = 0; dg < DG; ++dg)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dg][v] = 0.f;
  float m = kNegInf, l = 0.f;

  load(0, stage0);
  __syncthreads();
  // Tiles in three runs for this wave: keys every row of the wave sees, keys
  // near its rows (masked per lane: past the segment end or, causal, past
  // the row's token), keys after its last row (causal; skipped, still staged).
  auto tiles_upto = [&](int last_key) {  // tiles whose keys all lie at or before last_key
    const int x = last_key - key_lo - (kRows - 1);
    return x < 0 ? 0 : min(ntiles, x / kRows + 1);
  };
  auto tiles_from = [&](int last_key) {  // tiles whose first key lies at or before last_key
    const int x = last_key - key_lo;
    return x < 0 ? 0 : min(ntiles, x / kRows + 1);
  };
  const int full_end = uni(tiles_upto(a.causal ? min(key_hi - 1, wtok0) : key_hi - 1));
  const int seen_end = uni(a.causal ? tiles_from(wtok_max) : ntiles);

  // Tile it sits in stage it % 2, named at compile time (ST) so that the
  // compiler sees the reads of this tile and the copy into the other stage
  // touch different LDS objects and does not make the reads wait for it.
  auto step = [&](int it, auto mode, auto st) {
    constexpr int MODE = decltype(mode)::value;  // 0: skipped, 1: masked, 2: every key visible
    constexpr int ST = decltype(st)::value;
    char *const b = ST ? stage1 : stage0;
    char *const nb = ST ? stage0 : stage1;
    if (MODE != 0) {
      const int k0 = key_lo + kRows * it;
      Chunk<DT> af[G::KCH];
      read_frag<DT, D>(af, b);
      if (it + 1 < ntiles) load(it + 1, nb);
      f32x16 s[1];
      tile_mma<DT, D, 1>(af, qf, s);
      // Raw logits; invisible keys (past the segment end, or later than the
      // row's token under the causal mask) become -inf.  c1 > 0, so the
      // tile's log2-scaled maximum is c1 times the raw one, and each
      // probability is exp2(fma(s, c1, -m)).
      float x[16];
      const int lim = MODE == 1 ? min(key_hi - 1, a.causal ? qtok : key_hi - 1) - (k0 + 4 * (lane >> 5)) : 0;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[v] = s[0][v];
        if (MODE == 1) x[v] = (acc_row_c(v) <= lim) ? x[v] : kNegInf;
      }
      float tmax = x[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, x[v]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * a.c1;
      const bool move = tmax > m + kRescale;
      if (__ballot(move)) {
        const float m_new = move ? tmax : m;
        const float alpha = fast_exp2(m - m_new);  // 0 while m is still -inf
        l *= alpha;
#pragma unroll
        for (int dg = 0; dg < DG; ++dg)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[dg][v] *= alpha;
        m = m_new;
      }
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(x[v], a.c1, -m));
      l += tree16(p);
      const Chunk<DT> p0 = pack_p<DT>(p, 0), p1 = pack_p<DT>(p, 1);
      const char *vt = b + G::TILE;
#pragma unroll
      for (int dg = 0; dg < DG; ++dg) {
        o[dg] = mma<DT>(read_vt<DT, D>(vt, vt_off, dg, 0), p0, o[dg]);
        o[dg] = mma<DT>(read_vt<DT, D>(vt, vt_off, dg, 1), p1, o[dg]);
      }
    } else if (it + 1 < ntiles) {
      load(it + 1, nb);
    }
    __syncthreads();
  };
  int it = 0;
  const std::integral_constant<int, 0> s0;
  const std::integral_constant<int, 1> s1;
  auto run = [&](int end, auto mode) {
    if ((it & 1) && it < end) step(it++, mode, s1);
    for (; it + 1 < end; it += 2) {
      step(it, mode, s0);
      step(it + 1, mode, s1);
    }
    if (it < end) step(it++, mode, s0);
  };
  run(full_end, std::integral_constant<int, 2>{});
  run(seen_end, std::integral_constant<int, 1>{});
  run(ntiles, std::integral_constant<int, 0>{});

  // Both lane halves hold the same rows over different keys: combine the sums.
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = 1.0f / lt;
  const int r = lane & 31;
  const int t = wtok0 + r / F;
  if (t < tok_hi) {
    const int h = h0 + r % F;
    typedef typename PackT<DT>::T E;
    char *orow = reinterpret_cast<char *>(fa.out) + ((long long)t * fa.o_st + (long long)h * fa.o_sh) * G::ES;
#pragma unroll
    for (int dg = 0; dg < DG; ++dg) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = dg * 32 + 8 * i + 4 * (lane >> 5);  // columns d .. d+3 in registers 4i .. 4i+3
        if (d < D) {
          typedef E E4 __attribute__((ext_vector_type(4)));
          E4 y;
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = (E)(o[dg][4 * i + j] * inv);
          *reinterpret_cast<uint2 *>(orow + d * G::ES) = __builtin_bit_cast(uint2, y);
        }
      }
    }
    if (lane < 32)
      a.lse_out[(long long)h * a.L.T + t] = (m + __log2f(lt)) * 0.69314718055994530942f;
  }
}

template <int DT, int D>
hipError_t fwd_go(const AttnPlan &p, const FwdArgs &a, hipStream_t s) {
  const int grid = (int)((p.total_jobs + 7) / 8 * 8);
  hipLaunchKernelGGL((fwd_kernel<DT, D>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t fwd_d(const AttnPlan &p, const FwdArgs &a, hipStream_t s) {
  switch (p.D) {
    case 64: return fwd_go<DT, 64>(p, a, s);
    case 72: return fwd_go<DT, 72>(p, a, s);
    case 80: return fwd_go<DT, 80>(p, a, s);
    case 96: return fwd_go<DT, 96>(p, a, s);
    default: return fwd_go<DT, 128>(p, a, s);
  }
}

}  // namespace

hipError_t launch_fwd(const AttnPlan &p, const FwdArgs &a, hipStream_t s) {
  if (p.total_jobs == 0) return hipSuccess;
  return p.dtype == TSEL_F16 ? fwd_d<TSEL_F16>(p, a, s) : fwd_d<TSEL_BF16>(p, a, s);
}

}  // namespace tsel
