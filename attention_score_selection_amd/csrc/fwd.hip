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
// registers (converted to the input type) and V^T comes from an LDS copy of
// the value tile stored transposed.  The contraction's k slots of lane half h
// are the keys 16c + {0..3, 8..11} + 4h of chunk c, which is how the S^T
// accumulator already holds them; the transposed copy stores the keys in that
// order, so a V^T fragment is one 16-byte LDS read.
//
// The running maximum only moves when a tile's maximum exceeds it by more
// than 2^8 (so P stays below 2^8, safe for f16 operands); the accumulators are
// rescaled then, and the LSE uses the final maximum and sum.
#include "tiles.h"

namespace tsel {

namespace {

constexpr float kRescale = 8.0f;  // log2 headroom before the running max moves

// Transposed LDS copy of one 32-key value tile: row d (one per value column,
// padded to whole 32-row groups) holds the 32 keys' values, VS bytes apart.
// Within each 16-key chunk the keys are stored in the order 0-3, 8-11, 4-7,
// 12-15, so the eight keys one lane half contracts over (16c + {0..3, 8..11}
// + 4h) are adjacent: one 16-byte read per fragment.
__device__ __forceinline__ constexpr int vt_slot(int key) {
  return (key & ~15) | (key & 3) | ((key & 4) << 1) | ((key & 8) >> 1);
}
template <int DT, int D>
struct VGeom {
  static constexpr int ES = Elem<DT>::ES;
  static constexpr int DG = (D + 31) / 32;     // 32-row groups of O^T
  static constexpr int VS = kRows * ES + 16;   // row stride (bank spread)
  static constexpr int BYTES = DG * 32 * VS;
  static constexpr int DB = D / 8;             // 8-value column blocks
};

// Register staging of a value tile with the transpose: thread t moves key
// pair t % 16 (keys 2p, 2p+1) times column block t / 16 (8 columns); it
// writes 8 LDS words, each holding the two keys' values of one column.
template <int DT, int D>
struct VStage {
  using VG = VGeom<DT, D>;
  uint4 r0, r1;
  int off0, off1;  // byte offsets of the two 16-byte units from the tile base
  int key0;        // first key of the pair (tile row)
  bool active;

  __device__ __forceinline__ void init(long long vrow_bytes) {
    const int t = threadIdx.x;
    key0 = 2 * (t & 15);
    const int db = t >> 4;
    active = db < VG::DB;
    off0 = (int)(key0 * vrow_bytes) + db * 8 * VG::ES;
    off1 = (int)((key0 + 1) * vrow_bytes) + db * 8 * VG::ES;
  }
  // Tile rows [0, nvalid) come from `base` (wave-uniform); the rest are zero.
  __device__ __forceinline__ void load(const char *base, int nvalid) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base);
    r0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rs, (active && key0 < nvalid) ? off0 : kOOB, 0, 0));
    r1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rs, (active && key0 + 1 < nvalid) ? off1 : kOOB, 0, 0));
  }
  __device__ __forceinline__ void store(char *vt) const {
    if (!active) return;
    const int db = threadIdx.x >> 4;
    const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
    const uint32_t b[4] = {r1.x, r1.y, r1.z, r1.w};
    char *col = vt + (8 * db) * VG::VS + vt_slot(key0) * VG::ES;  // key0 + 1 is the next slot
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Column 8db + 2i: low halves of a[i] and b[i]; column 8db + 2i + 1:
      // their high halves.  (Selector bytes 4..7 pick from the first source.)
      const uint32_t lo = __builtin_amdgcn_perm(b[i], a[i], 0x05040100u);
      const uint32_t hi = __builtin_amdgcn_perm(b[i], a[i], 0x07060302u);
      *reinterpret_cast<uint32_t *>(col + (2 * i) * VG::VS) = lo;
      *reinterpret_cast<uint32_t *>(col + (2 * i + 1) * VG::VS) = hi;
    }
  }
};

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

// V^T fragment of row group dg, key chunk c: lane row dg*32 + lane%32, keys
// 16c + 4h + {0..3} and 16c + 8 + 4h + {0..3} (h = lane / 32), stored
// adjacently at slots 16c + 8h .. +7.
template <int DT, int D>
__device__ __forceinline__ Chunk<DT> read_vt(const char *vt, int dg, int c) {
  using VG = VGeom<DT, D>;
  const int lane = lane_id();
  const char *row = vt + (dg * 32 + (lane & 31)) * VG::VS + (16 * c + 8 * (lane >> 5)) * VG::ES;
  Chunk<DT> r;
  r.v[0] = *reinterpret_cast<const uint4 *>(row);
  return r;
}

template <int DT, int D>
__global__ __launch_bounds__(256, 3) void fwd_kernel(FwdArgs fa) {
  using G = Geom<DT, D>;
  using VG = VGeom<DT, D>;
  constexpr int BUF = G::TILE + VG::BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
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

  // Zero the padding rows of both transposed value tiles once (value columns
  // D .. 32*DG-1 never get data).
  if (VG::DG * 32 > D) {
    for (int i = threadIdx.x; i < (VG::DG * 32 - D) * VG::VS / 4; i += 256) {
      reinterpret_cast<uint32_t *>(smem + G::TILE + D * VG::VS)[i] = 0u;
      reinterpret_cast<uint32_t *>(smem + BUF + G::TILE + D * VG::VS)[i] = 0u;
    }
  }

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
  auto rows_of = [&](int it) { return key_hi - (key_lo + kRows * it); };
  StageRegs<DT, D> sk;
  sk.init([&](int r) { return r * (int)krow; });
  VStage<DT, D> sv;
  sv.init(vrow);
  auto buf = [&](int it) { return smem + (it & 1) * BUF; };
  auto load = [&](int it) {
    const long long first = key_lo + kRows * it;
    sk.load(kbase + first * krow, rows_of(it));
    sv.load(vbase + first * vrow, rows_of(it));
  };
  auto store = [&](int it) {
    sk.store(buf(it));
    sv.store(buf(it) + G::TILE);
  };

  f32x16 o[VG::DG];
#pragma unroll
  for (int dg = 0; dg < VG::DG; ++dg)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dg][v] = 0.f;
  float m = kNegInf, l = 0.f;

  load(0);
  store(0);
  if (1 < ntiles) load(1);
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

  auto step = [&](int it, auto mode) {
    constexpr int MODE = decltype(mode)::value;  // 0: skipped, 1: masked, 2: every key visible
    if (MODE != 0) {
      const int k0 = key_lo + kRows * it;
      const char *b = buf(it);
      Chunk<DT> af[G::KCH];
      read_frag<DT, D>(af, b);
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
        for (int dg = 0; dg < VG::DG; ++dg)
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
      for (int dg = 0; dg < VG::DG; ++dg) {
        o[dg] = mma<DT>(read_vt<DT, D>(vt, dg, 0), p0, o[dg]);
        o[dg] = mma<DT>(read_vt<DT, D>(vt, dg, 1), p1, o[dg]);
      }
    }
    if (it + 1 < ntiles) {
      store(it + 1);
      if (it + 2 < ntiles) load(it + 2);
    }
    __syncthreads();
  };
  int it = 0;
  for (; it < full_end; ++it) step(it, std::integral_constant<int, 2>{});
  for (; it < seen_end; ++it) step(it, std::integral_constant<int, 1>{});
  for (; it < ntiles; ++it) step(it, std::integral_constant<int, 0>{});

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
    for (int dg = 0; dg < VG::DG; ++dg) {
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
