// Budget top-k, stable compaction and row gather for gfx950.
//
// Top-k (one global pool per request, REDtech article sections 3.1-3.2): one
// 1024-thread workgroup per pool runs an exact MSB-first radix select on
// order-preserving 32-bit keys of the fp32 scores (four 8-bit digits, integer
// LDS histograms), which yields the k-th largest key tau and how many keys
// equal to tau still fit; a block-wide ordered scan then admits those equal
// keys by ascending candidate index.  No floating-point atomics: the result
// is exact and deterministic.
//
// Compaction (new lengths, image boundaries and original spatial indices,
// REDtech article section 3.2): per-block keep counts, one scan block, then a
// scatter pass that recomputes each token's flag and writes its original
// index and (image, row, col); a separate gather copies embedding rows with
// 16-byte vector loads.
#include <type_traits>

#include "device.h"

namespace tsel {

namespace {

constexpr int kTopkThreads = 1024;

// Order-preserving key: larger score -> larger key.  Non-finite -> 0 (ranks
// below every finite score); -0 and +0 share one key.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (!__builtin_isfinite(s)) return 0u;
  if (s == 0.0f) return 0x80000000u;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of v across a 1024-thread block; `total` gets the sum.
// `sh` needs 17 ints.  Contains barriers: call from every thread.
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) sh[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int x = (lane < nw) ? sh[lane] : 0;
    const int xs = wave_incl_scan(x);
    if (lane < nw) sh[lane] = xs - x;
    if (lane == nw - 1) sh[16] = xs;
  }
  __syncthreads();
  const int res = incl - v + sh[wid];
  total = sh[16];
  __syncthreads();
  return res;
}

// Pools of up to kTopkThreads * kTopkRegKeys candidates: every thread holds
// a contiguous run of at most kTopkRegKeys keys in registers for all passes.
// Histogram adds are merged per thread while consecutive keys share a digit
// (the keys of one pool often share their leading digits), and the final
// ordered admission of keys equal to tau needs one block scan of per-thread
// counts.
constexpr int kTopkRegKeys = 32;

__device__ __forceinline__ void topk_registers(const float *score, int n, int k, uint8_t *keep,
                                               int *hist, int *sh, int &s_digit, int &s_above) {
  const int tid = threadIdx.x;
  const int per = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  uint32_t u[kTopkRegKeys];
#pragma unroll
  for (int j = 0; j < kTopkRegKeys; ++j) u[j] = (i0 + j < i1) ? score_key(score[i0 + j]) : 0u;
  uint32_t prefix = 0u, pmask = 0u;
  int kr = k;  // how many of the keys matching `prefix` must still be kept
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    int cur = -1, cnt = 0;
#pragma unroll
    for (int j = 0; j < kTopkRegKeys; ++j) {
      if (i0 + j < i1 && (u[j] & pmask) == prefix) {
        const int d = (int)((u[j] >> shift) & 255u);
        if (d != cur) {
          if (cnt) atomicAdd(&hist[cur], cnt);
          cur = d;
          cnt = 0;
        }
        ++cnt;
      }
    }
    if (cnt) atomicAdd(&hist[cur], cnt);
    __syncthreads();
    // Suffix counts over digits: scan the histogram from digit 255 down.
    const int hv = (tid < 256) ? hist[255 - tid] : 0;
    int tot;
    const int excl = block_excl_scan(hv, sh, tot);
    if (tid < 256) {
      const int above = excl, upto = excl + hv;
      if (above < kr && upto >= kr) {
        s_digit = 255 - tid;
        s_above = above;
      }
    }
    __syncthreads();
    kr -= s_above;
    prefix |= (uint32_t)s_digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix = tau; the kr lowest-index keys equal to tau are kept.
  int eq = 0;
#pragma unroll
  for (int j = 0; j < kTopkRegKeys; ++j) eq += (i0 + j < i1 && u[j] == prefix) ? 1 : 0;
  int tot;
  int rank = block_excl_scan(eq, sh, tot);
#pragma unroll
  for (int j = 0; j < kTopkRegKeys; ++j) {
    if (i0 + j < i1) {
      const bool e = u[j] == prefix;
      keep[i0 + j] = (u[j] > prefix || (e && rank < kr)) ? 1 : 0;
      rank += e ? 1 : 0;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(DevLayout L, const float *score,
                                                           TopkChunk ks, uint8_t *keep) {
  __shared__ int hist[256];
  __shared__ int sh[17];
  __shared__ int s_digit, s_above;
  const int b = ks.b0 + blockIdx.x;
  const int lo = L.cu_cands[L.cu_images[b]];
  const int hi = L.cu_cands[L.cu_images[b + 1]];
  const int n = hi - lo;
  const int k = ks.k[blockIdx.x];
  const int tid = threadIdx.x;
  if (n <= 0) return;
  if (k <= 0 || k >= n) {
    const uint8_t f = (k >= n) ? 1 : 0;
    for (int i = tid; i < n; i += kTopkThreads) keep[lo + i] = f;
    return;
  }
  if (n <= kTopkThreads * kTopkRegKeys) {
    topk_registers(score + lo, n, k, keep + lo, hist, sh, s_digit, s_above);
    return;
  }
  uint32_t prefix = 0u, pmask = 0u;
  int kr = k;  // how many of the keys matching `prefix` must still be kept
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = score_key(score[lo + i]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    // Suffix counts over digits: scan the histogram from digit 255 down.
    const int hv = (tid < 256) ? hist[255 - tid] : 0;
    int tot;
    const int excl = block_excl_scan(hv, sh, tot);
    if (tid < 256) {
      const int above = excl;         // keys with a larger digit
      const int upto = excl + hv;     // ... plus this digit
      if (above < kr && upto >= kr) {
        s_digit = 255 - tid;
        s_above = above;
      }
    }
    __syncthreads();
    const int d = s_digit;
    kr -= s_above;
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix = tau (the k-th largest key); kr keys equal to tau are kept, lowest index first.
  int seen = 0;
  for (int base = 0; base < n; base += kTopkThreads) {
    const int i = base + tid;
    const uint32_t u = (i < n) ? score_key(score[lo + i]) : 0u;
    const int eq = (i < n && u == prefix) ? 1 : 0;
    int tot;
    const int rank = block_excl_scan(eq, sh, tot) + seen;
    if (i < n) keep[lo + i] = (u > prefix || (eq && rank < kr)) ? 1 : 0;
    seen += tot;
  }
}

// Keep decision of token t: text tokens stay, candidates follow their flag.
// Also returns the image s (or -1) and the offset inside it.
__device__ __forceinline__ int token_keep(const DevLayout &L, const uint8_t *keep, int t, int &s,
                                          int &off) {
  s = upper_index(L.img_start, 0, L.S, t);
  if (s >= 0) {
    const int n = L.img_hw[2 * s] * L.img_hw[2 * s + 1];
    off = t - L.img_start[s];
    if (off < n) return keep[L.cu_cands[s] + off] ? 1 : 0;
  }
  s = -1;
  off = 0;
  return 1;
}

__global__ __launch_bounds__(kCompactBlock) void compact_count(CompactArgs c) {
  __shared__ int sh[17];
  const int t = blockIdx.x * kCompactBlock + threadIdx.x;
  int s, off;
  const int k = (t < c.L.T) ? token_keep(c.L, c.keep, t, s, off) : 0;
  int tot;
  block_excl_scan(k, sh, tot);
  if (threadIdx.x == 0) c.blk_cnt[blockIdx.x] = tot;
}

// One block: offsets of the token blocks, the total, trailing empty requests,
// and the kept count of every image (one wave per image).
__global__ __launch_bounds__(kCompactBlock) void compact_scan(CompactArgs c) {
  __shared__ int sh[17];
  int carry = 0;
  for (int base = 0; base < c.nblk; base += kCompactBlock) {
    const int i = base + threadIdx.x;
    const int v = (i < c.nblk) ? c.blk_cnt[i] : 0;
    int tot;
    const int ex = block_excl_scan(v, sh, tot);
    if (i < c.nblk) c.blk_off[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) *c.total = carry;
  if (c.out_cu_seqlens != nullptr) {
    for (int b = threadIdx.x; b <= c.L.B; b += kCompactBlock)
      if (c.L.cu_seqlens[b] == c.L.T) c.out_cu_seqlens[b] = carry;
  }
  if (c.out_img_counts != nullptr) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int s = wid; s < c.L.S; s += kCompactBlock / 64) {
      const int c0 = c.L.cu_cands[s], c1 = c.L.cu_cands[s + 1];
      int cnt = 0;
      for (int i = c0 + lane; i < c1; i += 64) cnt += c.keep[i] ? 1 : 0;
      cnt = wave_sum(cnt);
      if (lane == 0) c.out_img_counts[s] = cnt;
    }
  }
}

__global__ __launch_bounds__(kCompactBlock) void compact_scatter(CompactArgs c) {
  __shared__ int sh[17];
  const int t = blockIdx.x * kCompactBlock + threadIdx.x;
  int s = -1, off = 0;
  const int k = (t < c.L.T) ? token_keep(c.L, c.keep, t, s, off) : 0;
  int tot;
  const int pos = c.blk_off[blockIdx.x] + block_excl_scan(k, sh, tot);
  if (t >= c.L.T) return;
  if (k && pos < c.cap) {
    c.out_token_idx[pos] = t;
    if (c.out_spatial != nullptr) {
      int3 v = make_int3(-1, -1, -1);
      if (s >= 0) {
        const int w = c.L.img_hw[2 * s + 1];
        v = make_int3(s, off / w, off % w);
      }
      c.out_spatial[3 * (long long)pos + 0] = v.x;
      c.out_spatial[3 * (long long)pos + 1] = v.y;
      c.out_spatial[3 * (long long)pos + 2] = v.z;
    }
  }
  if (c.out_cu_seqlens != nullptr) {
    // Every request that starts at token t (empty requests share starts).
    int b = upper_index(c.L.cu_seqlens, 0, c.L.B, t);
    while (b >= 0 && c.L.cu_seqlens[b] == t) {
      c.out_cu_seqlens[b] = pos;
      --b;
    }
  }
}

// Row gather: one wave per output row per iteration, VEC-byte units.
template <int VEC>
__global__ __launch_bounds__(256) void gather_rows(const char *emb, long long emb_stride,
                                                   long long row_bytes, char *out,
                                                   long long out_stride, const int *token_idx,
                                                   const int *total, int cap) {
  using U = typename std::conditional<VEC == 16, uint4, typename std::conditional<VEC == 4, uint32_t, uint8_t>::type>::type;
  const int nrows = min(*total, cap);
  const int lane = threadIdx.x & 63;
  const long long units = row_bytes / VEC;
  for (int p = blockIdx.x * 4 + (threadIdx.x >> 6); p < nrows; p += gridDim.x * 4) {
    const U *src = reinterpret_cast<const U *>(emb + (long long)token_idx[p] * emb_stride);
    U *dst = reinterpret_cast<U *>(out + (long long)p * out_stride);
    long long i = lane;
    for (; i + 192 < units; i += 256) {
      const U a0 = src[i], a1 = src[i + 64], a2 = src[i + 128], a3 = src[i + 192];
      dst[i] = a0;
      dst[i + 64] = a1;
      dst[i + 128] = a2;
      dst[i + 192] = a3;
    }
    for (; i < units; i += 64) dst[i] = src[i];
  }
}

// mRoPE positions of the compacted sequence.  Running index of a request:
// text tokens advance it by 1, an image of rows x cols by max(rows, cols);
// adj[s] is what the images of s's request before s add on top of their
// token counts (sum of max(rows, cols) - rows*cols), one thread per request.
__global__ __launch_bounds__(256) void mrope_image_adjust(DevLayout L, int *adj) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= L.B) return;
  int acc = 0;
  for (int s = L.cu_images[b]; s < L.cu_images[b + 1]; ++s) {
    adj[s] = acc;
    const int gh = L.img_hw[2 * s], gw = L.img_hw[2 * s + 1];
    acc += max(gh, gw) - gh * gw;
  }
}

// One thread per output row p: (i, i, i) for a text token whose running index
// is i; (i0, i0 + row, i0 + col) for an image token, i0 being the index at
// its image's first token.  Rows whose token index is out of range get -1.
__global__ __launch_bounds__(256) void mrope_positions(DevLayout L, const int *adj, const int *tok,
                                                       const int *sp, int n, int *pos) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= n) return;
  const int t = tok[p];
  int x = -1, y = -1, z = -1;
  if (t >= 0 && t < L.T) {
    const int b = upper_index(L.cu_seqlens, 0, L.B, t);
    const int lo = L.cu_seqlens[b];
    const int s = sp[3 * p];
    if (s >= 0 && s < L.S) {
      const int i0 = L.img_start[s] - lo + adj[s];
      x = i0;
      y = i0 + sp[3 * p + 1];
      z = i0 + sp[3 * p + 2];
    } else {
      const int j = upper_index(L.img_start, L.cu_images[b], L.cu_images[b + 1], t);
      int i = t - lo;
      if (j >= L.cu_images[b]) {
        const int gh = L.img_hw[2 * j], gw = L.img_hw[2 * j + 1];
        i += adj[j] + max(gh, gw) - gh * gw;
      }
      x = y = z = i;
    }
  }
  pos[3 * p] = x;
  pos[3 * p + 1] = y;
  pos[3 * p + 2] = z;
}

}  // namespace

hipError_t launch_mrope(const DevLayout &L, int *adj, const int *tok, const int *sp, int n, int *pos,
                        hipStream_t s) {
  if (L.B > 0 && L.S > 0)
    hipLaunchKernelGGL(mrope_image_adjust, dim3((L.B + 255) / 256), dim3(256), 0, s, L, adj);
  if (n > 0)
    hipLaunchKernelGGL(mrope_positions, dim3((n + 255) / 256), dim3(256), 0, s, L, adj, tok, sp, n, pos);
  return hipGetLastError();
}

hipError_t launch_topk(const DevLayout &L, const float *score, const TopkChunk &ks, int npools,
                       uint8_t *keep, hipStream_t s) {
  if (npools <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(npools), dim3(kTopkThreads), 0, s, L, score, ks, keep);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &c, hipStream_t s) {
  if (c.nblk > 0) {
    hipLaunchKernelGGL(compact_count, dim3(c.nblk), dim3(kCompactBlock), 0, s, c);
  }
  hipLaunchKernelGGL(compact_scan, dim3(1), dim3(kCompactBlock), 0, s, c);
  if (c.nblk > 0) {
    hipLaunchKernelGGL(compact_scatter, dim3(c.nblk), dim3(kCompactBlock), 0, s, c);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const void *emb, long long emb_stride, long long row_bytes, void *out,
                         long long out_stride, const int *token_idx, const int *total, int cap,
                         hipStream_t s) {
  if (cap <= 0 || row_bytes <= 0) return hipSuccess;
  const int grid = min((cap + 3) / 4, 65536);
  const uintptr_t bits = (uintptr_t)emb | (uintptr_t)out | (uintptr_t)emb_stride |
                         (uintptr_t)out_stride | (uintptr_t)row_bytes;
  const char *e = reinterpret_cast<const char *>(emb);
  char *o = reinterpret_cast<char *>(out);
  if ((bits & 15) == 0)
    hipLaunchKernelGGL(gather_rows<16>, dim3(grid), dim3(256), 0, s, e, emb_stride, row_bytes, o,
                       out_stride, token_idx, total, cap);
  else if ((bits & 3) == 0)
    hipLaunchKernelGGL(gather_rows<4>, dim3(grid), dim3(256), 0, s, e, emb_stride, row_bytes, o,
                       out_stride, token_idx, total, cap);
  else
    hipLaunchKernelGGL(gather_rows<1>, dim3(grid), dim3(256), 0, s, e, emb_stride, row_bytes, o,
                       out_stride, token_idx, total, cap);
  return hipGetLastError();
}

}  // namespace tsel
