// Tile building blocks shared by the attention kernels (LSE, column score,
// attention forward): operand chunks and the MFMA step per data type, the
// LDS geometry of a streamed 32-row tile, global -> LDS staging through
// buffer loads, fragment reads, and small epilogue helpers.
//
// Streamed tiles reach LDS through buffer loads whose per-lane offsets are
// fixed for the whole job.  Register staging (one tile ahead) and the
// LDS-direct form of the buffer load (no staging registers) are both here;
// each kernel uses the one that measured faster for it.
//
// A k chunk is split over the two lane halves, KW/2 consecutive values each.
// For fp32 the same 8 values feed eight 32x32x2 steps; A and B use the same
// permutation of k, so the contraction is unchanged.
#pragma once

#include <type_traits>

#include "device.h"

namespace tsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element size ES (bytes) and k width KW of one MFMA step per data type.
// 16-bit types: one 32x32x16 MFMA per 16 k values; fp32: eight 32x32x2
// MFMAs per 16 k values; fp8 (OCP E4M3): one 32x32x64 MFMA per 64 k values.
template <int DT> struct Elem { static constexpr int ES = 2, KW = 16; };
template <> struct Elem<TSEL_F32> { static constexpr int ES = 4, KW = 16; };
template <> struct Elem<TSEL_FP8_E4M3> { static constexpr int ES = 1, KW = 64; };

// This lane's share of one k chunk of one row: KW/2 consecutive k values
// (16 B for 16-bit types, 32 B for fp32 and fp8).
template <int DT>
struct Chunk {
  static constexpr int NV = Elem<DT>::KW / 2 * Elem<DT>::ES / 16;
  uint4 v[NV];
};

template <int DT>
__device__ __forceinline__ void zero_chunk(Chunk<DT> &c) {
#pragma unroll
  for (int i = 0; i < Chunk<DT>::NV; ++i) c.v[i] = make_uint4(0u, 0u, 0u, 0u);
}

template <int DT>
__device__ __forceinline__ void load_chunk(Chunk<DT> &c, const char *p) {
  const uint4 *q = reinterpret_cast<const uint4 *>(p);
#pragma unroll
  for (int i = 0; i < Chunk<DT>::NV; ++i) c.v[i] = q[i];
}

template <int DT>
__device__ __forceinline__ f32x16 mma(const Chunk<DT> &a, const Chunk<DT> &b, f32x16 acc);

template <>
__device__ __forceinline__ f32x16 mma<TSEL_BF16>(const Chunk<TSEL_BF16> &a, const Chunk<TSEL_BF16> &b,
                                                 f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v[0]),
                                                 __builtin_bit_cast(bf16x8, b.v[0]), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mma<TSEL_F16>(const Chunk<TSEL_F16> &a, const Chunk<TSEL_F16> &b,
                                                f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.v[0]),
                                                __builtin_bit_cast(f16x8, b.v[0]), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mma<TSEL_F32>(const Chunk<TSEL_F32> &a, const Chunk<TSEL_F32> &b,
                                                f32x16 acc) {
  const f32x4v a0 = __builtin_bit_cast(f32x4v, a.v[0]), a1 = __builtin_bit_cast(f32x4v, a.v[1]);
  const f32x4v b0 = __builtin_bit_cast(f32x4v, b.v[0]), b1 = __builtin_bit_cast(f32x4v, b.v[1]);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[s], b0[s], acc, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[s], b1[s], acc, 0, 0, 0);
  return acc;
}

// fp8 E4M3 operands (format code 0 for both A and B), no block scaling.  A
// and B fragments are loaded the same way (lane half h holds k values
// 32h .. 32h+31 of the chunk), so the contraction pairs matching k.
template <>
__device__ __forceinline__ f32x16 mma<TSEL_FP8_E4M3>(const Chunk<TSEL_FP8_E4M3> &a,
                                                     const Chunk<TSEL_FP8_E4M3> &b, f32x16 acc) {
  struct P { uint4 x, y; };
  const i32x8 av = __builtin_bit_cast(i32x8, P{a.v[0], a.v[1]});
  const i32x8 bv = __builtin_bit_cast(i32x8, P{b.v[0], b.v[1]});
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
}

constexpr int kRows = 32;  // rows of a streamed tile and of a resident group

// k chunks of a head dim (rounded up to whole chunks).
constexpr int kch(int dt, int d) {
  const int kw = dt == TSEL_FP8_E4M3 ? 64 : 16;
  return (d + kw - 1) / kw;
}

// Geometry of one streamed 32-row tile in LDS.  A head dim that is not a
// multiple of the k width (72 for 16-bit types) is padded with zeros to the
// next one: the padded units are staged as zeros and the padded k values of
// the resident operand are zero, so they add nothing to the contraction.
// SLOTS (0: one more than the row's units) sets the LDS row stride in 16-byte
// slots.
template <int DT, int D, int SLOTS = 0>
struct Geom {
  static_assert((D * Elem<DT>::ES) % 16 == 0, "a row must be whole 16-byte units");
  static constexpr int ES = Elem<DT>::ES;
  static constexpr int KW = Elem<DT>::KW;
  static constexpr int KCH = kch(DT, D);               // KW-wide k chunks (one MFMA step each)
  static constexpr int ROW = KCH * KW * ES;            // bytes of a (padded) row in LDS
  static constexpr int UNITS = ROW / 16;               // 16-byte units per (padded) row
  static constexpr int UNITS_D = D * ES / 16;          // ... of which hold data
  static constexpr int UPT = (kRows * UNITS + 255) / 256;  // units per thread (256 threads)
  // LDS tile: 16-byte slots, SLOTS_ROW per row (by default UNITS + 1, the
  // last padding the row so that the 32 rows of a fragment read fall in
  // different banks), the slot count rounded up to whole 64-slot blocks (one
  // wave's direct load).
  static_assert(SLOTS == 0 || SLOTS >= UNITS, "a row needs its units");
  static constexpr int SLOTS_ROW = SLOTS ? SLOTS : UNITS + 1;
  static constexpr int RS = 16 * SLOTS_ROW;            // LDS row stride in bytes
  static constexpr int NBLK = (kRows * SLOTS_ROW + 63) / 64;
  static constexpr int TILE = NBLK * 64 * 16;          // bytes of one tile
};

// Buffer offset past every valid byte: a load there returns zero.  Host-side
// planning guarantees that all in-tile offsets stay below it.
constexpr int kOOB = kBufferLimit;

// Buffer resource for raw (unstructured) loads from `base`; on gfx9 parts the
// third word selects 32-bit data format so that offset range checking applies.
// `base` must be wave-uniform; it is moved to scalar registers explicitly so
// that the resource never needs a per-lane loop.  Loads at byte offsets from
// `limit` on (wave-uniform, at most kOOB) return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int limit = kOOB) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  const unsigned long long u = (unsigned long long)(unsigned)uni((int)(p >> 32)) << 32 |
                               (unsigned)uni((int)(unsigned)p);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), (short)0, uni(limit), 0x00020000);
}

// Register staging of one streamed tile: global -> VGPR -> LDS.  Each thread
// moves UPT fixed 16-byte units of the tile; their byte offsets from the
// tile's first row are computed once, so a step costs one compare and one
// select per unit.  Units of rows past the valid range read as zero.
template <int DT, int D>
struct StageRegs {
  using G = Geom<DT, D>;
  uint4 r[G::UPT];
  int off[G::UPT];  // byte offset of unit i from the tile base
  int row[G::UPT];  // tile row of unit i (kRows: the unit is past the tile)

  // rowoff(row): byte offset of tile row `row` from the tile base.
  template <typename RowOff>
  __device__ __forceinline__ void init(RowOff rowoff) {
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
      const int u = threadIdx.x + 256 * i;
      if (u < kRows * G::UNITS) {
        row[i] = u / G::UNITS;
        off[i] = (u % G::UNITS < G::UNITS_D) ? rowoff(row[i]) + (u % G::UNITS) * 16 : kOOB;
      } else {
        row[i] = kRows;
        off[i] = kOOB;
      }
    }
  }
  // Tile rows [0, nvalid) come from `base` (wave-uniform), the rest are zero;
  // without PART all 32 rows are valid (units past the tile still read zero).
  template <bool PART = true>
  __device__ __forceinline__ void load(const char *base, int nvalid) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base);
#pragma unroll
    for (int i = 0; i < G::UPT; ++i)
      r[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (!PART || row[i] < nvalid) ? off[i] : kOOB, 0, 0));
  }
  __device__ __forceinline__ void store(char *tile) const {
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
      const int u = threadIdx.x + 256 * i;
      if (kRows * G::UNITS == 256 * G::UPT || u < kRows * G::UNITS) {  // (every unit is real when the tile fills the threads)
        const int rr = u / G::UNITS, col = u % G::UNITS;
        *reinterpret_cast<uint4 *>(tile + rr * G::RS + col * 16) = r[i];
      }
    }
  }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Staging of one streamed tile straight from global memory into LDS (buffer
// loads with the LDS-direct option: lane l of a wave writes 16 bytes at the
// block's LDS base + 16*l).  The tile's 64-slot blocks are dealt to the waves
// round-robin; each lane's slot maps to a fixed (row, 16-byte unit), whose
// byte offset from the tile base is computed once.  Padding slots, and rows
// past the valid range, read as zero.
template <int DT, int D, typename GT = Geom<DT, D>>
struct StageDirect {
  using G = GT;
  static constexpr int BPW = (G::NBLK + 3) / 4;  // blocks per wave (at most)
  int off[BPW];  // byte offset of this lane's unit in block 4*j + wave
  int row[BPW];  // its tile row (kRows: padding or past the tile)

  // rowoff(row): byte offset of tile row `row` from the tile base.
  template <typename RowOff>
  __device__ __forceinline__ void init(RowOff rowoff) {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int slot = 64 * (4 * j + w) + lane_id();
      const int r = slot / G::SLOTS_ROW, u = slot % G::SLOTS_ROW;
      if (r < kRows && u < G::UNITS_D) {
        row[j] = r;
        off[j] = rowoff(r) + u * 16;
      } else {
        row[j] = kRows;
        off[j] = kOOB;
      }
    }
  }
  // Start the copy of the tile at byte `soff` past the resource's base into
  // `tile` (tile rows [0, nvalid) when PART, else all 32 rows); the rest of
  // the tile reads as zero.  Every wave but the last of a partial block row
  // issues the same loads, so only the last block needs a (wave-uniform)
  // test.  Complete once this wave's vector-memory counter drains.
  template <bool PART>
  __device__ __forceinline__ void load_at(char *tile, __amdgpu_buffer_rsrc_t rs, int soff, int nvalid) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int w = uni(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int blk = 4 * j + w;
      if (j < BPW - 1 || blk < G::NBLK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(tile + blk * 1024), 16,
                                                 (!PART || row[j] < nvalid) ? off[j] : kOOB, soff, 0, 0);
    }
#endif
  }
  // Start the copy of tile rows [0, nvalid) from `base` (wave-uniform) into
  // `tile`; the rest of the tile reads as zero.  Complete once this wave's
  // vector-memory counter drains (a __syncthreads() waits for that).
  __device__ __forceinline__ void load(char *tile, const char *base, int nvalid) const {
    // (The host pass of the compiler only sees the declaration: the LDS-direct
    // builtin has no host form, and referencing it there would make the host
    // side drop the kernels that use it.)
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base);
    const int w = uni(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int blk = 4 * j + w;
      if (blk < G::NBLK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void_t *)(tile + blk * 1024), 16, row[j] < nvalid ? off[j] : kOOB, 0, 0, 0);
    }
#endif
  }
};

// This lane's fragment (row lane%32, k values 16*kc + 8*(lane/32) .. +8) of
// an LDS tile.
template <int DT, int D>
__device__ __forceinline__ void read_frag(Chunk<DT> (&f)[kch(DT, D)], const char *tile) {
  using G = Geom<DT, D>;
  const int lane = lane_id();
  const char *p = tile + (lane & 31) * G::RS + (lane >> 5) * (G::KW / 2) * G::ES;
#pragma unroll
  for (int kc = 0; kc < G::KCH; ++kc) load_chunk<DT>(f[kc], p + kc * G::KW * G::ES);
}

// Load the resident fragments of NG 32-row groups straight from global memory.
template <int DT, int D, int NG, typename RowPtr>
__device__ __forceinline__ void load_resident(Chunk<DT> (&res)[NG][kch(DT, D)], RowPtr rowptr) {
  using G = Geom<DT, D>;
  const int lane = lane_id();
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    const char *p = rowptr(n * kRows + (lane & 31));
#pragma unroll
    for (int kc = 0; kc < G::KCH; ++kc) {
      const int e = G::KW * kc + (G::KW / 2) * (lane >> 5);
      if (p != nullptr && e < D) load_chunk<DT>(res[n][kc], p + e * G::ES);
      else zero_chunk<DT>(res[n][kc]);
    }
  }
}

// acc[n] = A . R[n]^T for one streamed tile against all NG resident groups,
// k chunks outermost so that the NG accumulation chains are independent.
template <int DT, int D, int NG>
__device__ __forceinline__ void tile_mma(const Chunk<DT> (&af)[kch(DT, D)],
                                         const Chunk<DT> (&res)[NG][kch(DT, D)],
                                         f32x16 (&acc)[NG]) {
#pragma unroll
  for (int n = 0; n < NG; ++n) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[n][v] = 0.f;
  }
#pragma unroll
  for (int kc = 0; kc < kch(DT, D); ++kc) {
#pragma unroll
    for (int n = 0; n < NG; ++n) acc[n] = mma<DT>(af[kc], res[n][kc], acc[n]);
  }
}

// The same with every accumulation chain starting from `seed` instead of 0,
// for the first M of the NG resident groups only.
template <int DT, int D, int NG, int M = NG>
__device__ __forceinline__ void tile_mma_seeded(const Chunk<DT> (&af)[kch(DT, D)],
                                                const Chunk<DT> (&res)[NG][kch(DT, D)],
                                                f32x16 (&acc)[NG], const f32x16 &seed) {
  static_assert(M >= 1 && M <= NG, "group count");
#pragma unroll
  for (int n = 0; n < M; ++n) acc[n] = mma<DT>(af[0], res[n][0], seed);
#pragma unroll
  for (int kc = 1; kc < kch(DT, D); ++kc) {
#pragma unroll
    for (int n = 0; n < M; ++n) acc[n] = mma<DT>(af[kc], res[n][kc], acc[n]);
  }
}

// Row of the 32x32 accumulator held in register v by this lane is
// acc_row_c(v) + 4 * (lane / 32); acc_row_c is a compile-time constant, so a
// mask test against a per-lane threshold costs one compare per register.
__device__ __forceinline__ constexpr int acc_row_c(int v) { return 8 * (v >> 2) + (v & 3); }

// Sum of 16 values as a balanced tree (shorter dependency chains, smaller
// rounding growth than a running sum).
__device__ __forceinline__ float tree16(const float (&p)[16]) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = p[2 * i] + p[2 * i + 1];
  return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until every outstanding vector-memory load of this wave has landed
// (s_waitcnt vmcnt(0)); issued once after the resident operand is loaded so
// that the streaming loop never waits on it.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

}  // namespace tsel
