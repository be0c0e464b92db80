// Internal declarations shared by the host layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "tsel.h"

namespace tsel {

// Layout as the kernels see it (device pointers, passed by value).
struct DevLayout {
  int B, S, T;
  const int *cu_seqlens, *cu_images, *img_start, *img_hw, *cu_cands;
};

// How attention segments are formed: one per request (full / causal masks)
// or one per image (block-diagonal mask).
enum SegKind { SEG_REQ = 0, SEG_IMG = 1 };

// Order in which a launch runs the jobs of a head block (see job_order).  A
// permutation travels in the kernel arguments, so launches with at most
// kOrderMaxJobs jobs per head block can be reordered.  Only the reordered
// launches carry it: a kilobyte more of kernel arguments measured 6% slower
// on the column score.  (The 16384-token GQA layer's column score has 570
// jobs per head block.)
enum JobOrder { kOrderPlain = 0, kOrderRankMajor = 1, kOrderSorted = 2 };
constexpr int kOrderMaxJobs = 1024;
struct JobPerm {
  unsigned w[kOrderMaxJobs / 2];  // heaviest-first job permutation, 16 bits per entry (low half first)
};

// Parameters of the LSE and column-score kernels.
struct AttnArgs {
  DevLayout L;
  const void *q;
  long long q_st, q_sh;  // element strides
  const void *k;
  long long k_st, k_sh;
  int hq, hg;            // query heads, query heads per KV head
  int F;                 // query heads folded into one 16-row tile (power of two dividing hg)
  int nhb;               // head blocks = hq / F
  int causal;            // 1 for TSEL_MASK_CAUSAL
  int segkind;           // SegKind
  int nseg;              // B or S
  float c1;              // softmax scale * log2(e)
  int jobs_per_hb;       // jobs of one head block
  int total_jobs;        // nhb * jobs_per_hb
  int order;             // JobOrder
  // LSE kernel
  float *lse_out;
  int TB;                // tokens per row block
  int KS;                // keys per key split (0: every job sees its row block's whole key range)
  int ksmax;             // splits of the longest segment (stride of lse_part)
  float *lse_part;       // [Hq][T][ksmax] per-split log2-sum-exp (workspace), when KS > 0
  // column-score kernel
  const float *lse_in;
  float *partial;        // [nhb][RCmax][N]
  int N, RC, RCF;        // candidates, row-chunk tokens, tokens of a piece of the last chunk
  int RCmax, KB;         // max chunks per segment, keys per block
};

// Attention forward: the LSE kernel's job split plus the values and output.
struct FwdArgs {
  AttnArgs at;           // q, k, layout, head fold, masks, TB, lse_out
  const void *v;
  long long v_st, v_sh;  // element strides of v
  void *out;
  long long o_st, o_sh;  // element strides of out
};

// Host-side plan of one attention launch.
struct AttnPlan {
  int dtype, D, NT;
  int F, nhb, TB, KB, RC, RCF, RCmax;
  int KS, ksmax;         // LSE key split (0: none) and the splits of the longest segment
  int nseg, segkind;
  long long jobs_per_hb, total_jobs;
  size_t partial_bytes;
};

// Row chunks of the column score over a segment of n tokens: chunks of RC
// tokens, except that a segment longer than RC has the range after its last
// whole chunk cut into pieces of RCF tokens (RCF divides RC; RCF == RC leaves
// it whole).  The pieces come last in the enumeration, so a launch whose jobs
// are long ends on short ones.  A segment of at most RC tokens is one chunk.
__host__ __device__ inline int chunk_whole(int n, int RC) { return n > RC ? (n - 1) / RC : 1; }
__host__ __device__ inline int chunk_count(int n, int RC, int RCF) {
  if (n <= 0) return 0;
  const int whole = chunk_whole(n, RC);
  const int rest = n - whole * RC;
  return whole + (rest > 0 ? (rest + RCF - 1) / RCF : 0);
}
// Token range [lo, hi) of chunk r, relative to the segment start.
__host__ __device__ inline void chunk_range(int r, int n, int RC, int RCF, int &lo, int &hi) {
  const int whole = chunk_whole(n, RC);
  if (r < whole) {
    lo = r * RC;
    hi = lo + RC;
  } else {
    lo = whole * RC + (r - whole) * RCF;
    hi = lo + RCF;
  }
  if (hi > n) hi = n;
}
// Chunk holding token t (relative to the segment start, 0 <= t < n).
__host__ __device__ inline int chunk_of(int t, int n, int RC, int RCF) {
  const int whole = chunk_whole(n, RC);
  return t < whole * RC ? t / RC : whole + (t - whole * RC) / RCF;
}

// Error reporting (thread-local message).
int fail(int code, const char *fmt, ...);
void clear_error();

int plan_lse(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p);
int plan_colscore(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p);

// Kernel launchers (attn.hip / select.hip).  Return hipError_t of the launch.
// perm: the job permutation when a.order is not kOrderPlain, else null.
hipError_t launch_lse(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, hipStream_t s);
hipError_t launch_colscore(const AttnPlan &p, const AttnArgs &a, const JobPerm *perm, float *score,
                           hipStream_t s);
hipError_t launch_fwd(const AttnPlan &p, const FwdArgs &a, hipStream_t s);
int plan_fwd(const tsel_attn_t *a, const tsel_layout_t *l, AttnPlan *p);

struct TopkChunk {
  int b0;        // first pool of this launch
  int k[256];    // k of pools b0 .. b0+255
};
hipError_t launch_topk(const DevLayout &L, const float *score, const TopkChunk &ks, int npools,
                       uint8_t *keep, hipStream_t s);

// Pools larger than one top-k workgroup holds in registers are spread over
// blocks of kTopkSplit candidates each (64 such pools a launch).  Workspace
// (ints): per pool a state record and a 256-bin histogram, then one tie count
// per block.
constexpr int kTopkRegLimit = 32768;
constexpr int kTopkSplit = 16384;
constexpr int kTopkLargeChunk = 64;
struct TopkLarge {
  int np;                       // large pools in this launch
  int pool[kTopkLargeChunk];    // their pool indices
  int k[kTopkLargeChunk];       // k of each
  int blk[kTopkLargeChunk + 1]; // first block of each; blk[np] = blocks of the launch
};
struct TopkLargeWs {
  int *state;  // [kTopkLargeChunk][4]: tau prefix, keys still to keep at tau, keys equal to tau, blocks done
  int *hist;   // [kTopkLargeChunk][256]
  int *blkeq;  // [blocks]: keys equal to tau per block
};
inline size_t topk_large_ws_bytes(long long max_blocks) {
  return (size_t)(kTopkLargeChunk * 4 + kTopkLargeChunk * 256 + max_blocks) * sizeof(int);
}
hipError_t launch_topk_large(const DevLayout &L, const float *score, const TopkLarge &tl, const TopkLargeWs &ws,
                             uint8_t *keep, hipStream_t s);

// Input-dependent budget: per-pool target fraction and k bounds (64 pools a launch).
constexpr int kMassChunk = 64;
struct MassChunk {
  int b0;                 // first pool of this launch
  int kmin[kMassChunk];   // floor(r_min * N_b + 1e-6)
  int kmax[kMassChunk];   // floor(r_max * N_b + 1e-6)
  double tau[kMassChunk];  // target fraction of the pool's mass, in [0, 1]
};
hipError_t launch_mass_budget(const DevLayout &L, const float *score, const MassChunk &mc, int npools,
                              int *k_out, uint8_t *keep, hipStream_t s);

struct CompactArgs {
  DevLayout L;
  const uint8_t *keep;
  int N;
  int nblk;
  int *blk_cnt, *blk_off, *total;  // workspace
  int fused;                        // 1: the scatter forms the block offsets and image counts itself
  int cap;
  int *out_token_idx, *out_spatial, *out_cu_seqlens, *out_img_counts;
};
hipError_t launch_compact(const CompactArgs &c, hipStream_t s);
hipError_t launch_gather(const void *emb, long long emb_stride, long long row_bytes, void *out,
                         long long out_stride, const int *token_idx, const int *total, int cap,
                         hipStream_t s);

hipError_t launch_mrope(const DevLayout &L, int *adj, const int *tok, const int *sp, int n, int *pos,
                        hipStream_t s);

constexpr int kCompactBlock = 1024;

// Query rows (tokens x folded heads) of one column-score row chunk at most.
constexpr int kChunkRows = 8192;

// The static device scratch of tsel_colscore_noalloc (static_scratch.hip):
// its size, and its address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(void **out);

// Streamed tiles are read through buffer resources whose range ends here;
// offsets at or past it read as zero.
constexpr int kBufferLimit = 0x7FFFFFF0;

// Resident 32-row groups per wave for a (dtype, head_dim): one group holds
// head_dim values of 32 rows, i.e. head_dim * elem_size / 8 VGPRs per lane;
// the total must leave room for the accumulators within 256 VGPRs (two waves
// per SIMD).
constexpr int max_groups(int dtype, int head_dim) {
  const int es = dtype == TSEL_F32 ? 4 : dtype == TSEL_FP8_E4M3 ? 1 : 2;
  const int kw = dtype == TSEL_FP8_E4M3 ? 64 : 16;
  const int per_group = (head_dim + kw - 1) / kw * kw * es / 8;  // VGPRs (padded k)
  return per_group <= 20 ? 4 : per_group <= 32 ? 3 : per_group <= 48 ? 2 : 1;
}

// Resident key groups per wave of the column score, and its workgroups per
// CU.  The column score starts its accumulation chains from the rows' LSE
// (no LSE registers live through the epilogue), which leaves room for a
// fourth group where max_groups allows three (16-bit inputs, d = 96..128):
// 5% faster on the 16384-token layer and the varlen batch, 9% on the
// 3214-token one.  Two groups at three workgroups per CU measured the same
// as three at two on the 16384-token layer and 1% slower on the varlen batch.
// fp8 (four groups of half the registers) fits three workgroups per CU,
// where its VALU-bound epilogue gains from the third wave per SIMD: 10%
// faster on the 16384-token layer.
constexpr int colscore_groups(int dtype, int head_dim) {
  return max_groups(dtype, head_dim) == 3 && dtype != TSEL_F32 ? 4 : max_groups(dtype, head_dim);
}
constexpr int colscore_wgs(int dtype) { return dtype == TSEL_FP8_E4M3 ? 3 : 2; }

// Resident query groups per wave of the LSE kernel.  A lane's 16 values of a
// group all belong to one query row, so the row's offset and sum are one
// register each and a fourth group fits where max_groups allows three
// (16-bit inputs, d = 96..128).
constexpr int lse_groups(int dtype, int head_dim) {
  return max_groups(dtype, head_dim) == 3 && dtype != TSEL_F32 ? 4 : max_groups(dtype, head_dim);
}

}  // namespace tsel
