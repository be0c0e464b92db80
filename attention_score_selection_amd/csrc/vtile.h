// Geometry of the attention forward's value tile and the per-lane addresses
// of its transposing reads (ds_read_b64_tr_b16).  Host- and device-callable,
// so that a host test can check the mapping for every head dim.
#pragma once

#include "tiles.h"

namespace tsel {

// Column groups of O^T: 32 output columns each (the last one padded).
template <int D> struct OGroups { static constexpr int DG = (D + 31) / 32; };

// Row stride of the value tile, in 16-byte slots: the smallest that holds a
// row and is 64 or 192 bytes past a multiple of 256.  A transposing read
// touches four consecutive rows per 32 lanes, 64 bytes of each; with that
// stride they start 16 banks apart (of 64) and never share a bank.  It also
// leaves room for the padded columns of the last column group (d = 72, 80).
__host__ __device__ constexpr int vt_slots(int units) {
  int s = units;
  while ((16 * s) % 256 != 64 && (16 * s) % 256 != 192) ++s;
  return s;
}
template <int DT, int D>
using VGeom = Geom<DT, D, vt_slots(Geom<DT, D>::UNITS)>;

// Byte offset of lane `lane`'s 8-byte unit in a row-major value tile for the
// transposing reads.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane i
// of a group receives value i % 4 of the 8-byte units that lanes i/4 + 4m
// (m = 0..3) of its group address.  Here lane j of group gr = lane/16
// addresses the four values of columns 16*(gr % 2) + 4*(j % 4) .. +3 in key
// row 4*(gr / 2) + j/4, so lane i receives, for its own column
// 16*(gr % 2) + i = lane % 32, the values of keys 4*(gr / 2) + 0..3 =
// 4*(lane / 32) + 0..3: the first four k slots of its lane half.  The next
// four (keys + 8) are the same read 8 rows further on.
template <int DT, int D>
__host__ __device__ constexpr int vt_lane_offset_of(int lane) {
  using G = VGeom<DT, D>;
  const int gr = lane >> 4, j = lane & 15;
  return (4 * (gr >> 1) + (j >> 2)) * G::RS + (16 * (gr & 1) + 4 * (j & 3)) * G::ES;
}

// Byte offset, from the tile base, of lane `lane`'s unit in the read `half`
// (0: keys 16c + 4h + 0..3, 1: keys 16c + 8 + 4h + 0..3) of the V^T fragment
// of column group dg, key chunk c.
template <int DT, int D>
__host__ __device__ constexpr int vt_read_offset(int lane, int dg, int c, int half) {
  using G = VGeom<DT, D>;
  return vt_lane_offset_of<DT, D>(lane) + (16 * c + 8 * half) * G::RS + dg * 32 * G::ES;
}

}  // namespace tsel
