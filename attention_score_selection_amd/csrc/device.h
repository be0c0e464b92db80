// Device-side helpers: wave scans, layout lookups, workgroup-to-XCD mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace tsel {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A value the caller knows to be the same in every lane, moved to a scalar
// register.  Branches on such values then need no exec-mask bookkeeping.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The hardware hands workgroup i to XCD i % 8.  Give each XCD one contiguous
// range of job ids so that jobs sharing operands (same head block, same rows)
// meet in the same L2.  `grid` is a multiple of 8.
__device__ __forceinline__ int xcd_job(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Token range of attention segment a.
__device__ __forceinline__ void seg_tokens(const DevLayout &L, int kind, int a, int &lo, int &hi) {
  if (kind == SEG_REQ) {
    lo = L.cu_seqlens[a];
    hi = L.cu_seqlens[a + 1];
  } else {
    lo = L.img_start[a];
    hi = lo + L.img_hw[2 * a] * L.img_hw[2 * a + 1];
  }
}

// Image range [s_lo, s_hi) and candidate range [c_lo, c_hi) of segment a.
__device__ __forceinline__ void seg_images(const DevLayout &L, int kind, int a, int &s_lo, int &s_hi,
                                           int &c_lo, int &c_hi) {
  if (kind == SEG_REQ) {
    s_lo = L.cu_images[a];
    s_hi = L.cu_images[a + 1];
  } else {
    s_lo = a;
    s_hi = a + 1;
  }
  c_lo = L.cu_cands[s_lo];
  c_hi = L.cu_cands[s_hi];
}

// Largest index i in [lo, hi) with arr[i] <= x (arr sorted ascending);
// returns lo - 1 if none.
__device__ __forceinline__ int upper_index(const int *arr, int lo, int hi, int x) {
  int a = lo, b = hi;  // answer in [a-1, b-1]
  while (a < b) {
    int mid = (a + b) >> 1;
    if (arr[mid] <= x) a = mid + 1; else b = mid;
  }
  return a - 1;
}

// Token of candidate c, given the image range [s_lo, s_hi) that holds it.
__device__ __forceinline__ int cand_token(const DevLayout &L, int s_lo, int s_hi, int c) {
  int s = upper_index(L.cu_cands, s_lo, s_hi, c);
  return L.img_start[s] + (c - L.cu_cands[s]);
}

// The images [s_lo, s_hi) of a segment spread over the lanes of a wave, one
// image per lane, when there are at most 64: the candidate -> token lookup
// then needs one round of loads for the whole job instead of a binary search
// through memory per lookup.  All 64 lanes must call these.
struct ImgLanes {
  int n;      // images (wave-uniform); more than 64: use cand_token instead
  int cand0;  // lane i < n: first candidate of image s_lo + i (INT_MAX past n)
  int tok0;   // lane i < n: first token of image s_lo + i
};
__device__ __forceinline__ ImgLanes img_lanes(const DevLayout &L, int s_lo, int s_hi) {
  ImgLanes t;
  t.n = s_hi - s_lo;
  const int i = lane_id();
  const bool in = i < t.n;
  t.cand0 = in ? L.cu_cands[s_lo + i] : 0x7fffffff;
  t.tok0 = in ? L.img_start[s_lo + i] : 0;
  return t;
}
// Token of candidate c of the segment, c wave-uniform: its image is the last
// one whose first candidate is at or before c.
__device__ __forceinline__ int img_token_uniform(const ImgLanes &t, int c) {
  const unsigned long long m = __ballot(t.cand0 <= c);
  const int s = 63 - __builtin_clzll(m);
  return __builtin_amdgcn_readlane(t.tok0, s) + c - __builtin_amdgcn_readlane(t.cand0, s);
}
// The same for a per-lane candidate c.
__device__ __forceinline__ int img_token(const ImgLanes &t, int c) {
  int s = 0;
  for (int j = 1; j < t.n; ++j) s += __builtin_amdgcn_readlane(t.cand0, j) <= c ? 1 : 0;
  return __shfl(t.tok0, s, 64) + c - __shfl(t.cand0, s, 64);
}

// Find which segment owns item `idx` when segment a owns count(a) items,
// segments in order.  Wave-uniform; all 64 lanes must call it.  Returns the
// segment, and the item's index inside it in `local`; returns -1 if idx is
// past the end.
template <typename CountFn>
__device__ __forceinline__ int find_segment(int nseg, int idx, CountFn count, int &local) {
  const int lane = lane_id();
  int base = 0;
  for (int a0 = 0; a0 < nseg; a0 += 64) {
    const int a = a0 + lane;
    const int c = (a < nseg) ? count(a) : 0;
    const int incl = wave_incl_scan(c);
    const int total = __shfl(incl, 63, 64);
    if (idx < base + total) {
      const unsigned long long m = __ballot(base + incl > idx);
      const int ln = __ffsll((long long)m) - 1;
      // Wave-uniform results: keep them in scalar registers.
      local = __builtin_amdgcn_readfirstlane(idx - base - __shfl(incl - c, ln, 64));
      return __builtin_amdgcn_readfirstlane(a0 + ln);
    }
    base += total;
  }
  local = 0;
  return -1;
}

// A workgroup's head block hb and job rj (within the head block) from its
// job index, in enumeration order (segment by segment), head block by head
// block.
__device__ __forceinline__ void job_plain(const AttnArgs &a, int job, int &hb, int &rj) {
  hb = job / a.jobs_per_hb;
  rj = job % a.jobs_per_hb;
}

// The same from the host's heaviest-first permutation: kOrderRankMajor runs an
// XCD's jobs rank by rank across the head blocks it holds (the head blocks
// are a multiple of 8, a contiguous group of them per XCD, see xcd_job);
// kOrderSorted keeps head block by head block.
__device__ __forceinline__ void job_ordered(const AttnArgs &a, const JobPerm &perm, int job, int &hb,
                                            int &rj) {
  int r;
  if (a.order == kOrderRankMajor) {
    const int H = a.nhb >> 3, per = H * a.jobs_per_hb;
    const int p = job % per;
    hb = (job / per) * H + p % H;
    r = p / H;
  } else {
    hb = job / a.jobs_per_hb;
    r = job % a.jobs_per_hb;
  }
  const unsigned w = uni((int)perm.w[r >> 1]);  // two 16-bit entries per word (scalar load)
  rj = (int)((r & 1) ? (w >> 16) : (w & 0xffffu));
}

}  // namespace tsel
