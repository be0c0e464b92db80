// Budget top-k, stable compaction and row gather for gfx950.
//
// Top-k (one global pool per request, REDtech article sections 3.1-3.2): one
// 1024-thread workgroup per pool runs an exact MSB-first radix select on
// order-preserving 32-bit keys of the fp32 scores (four 8-bit digits, integer
// LDS histograms), which yields the k-th largest key tau and how many keys
// equal to tau still fit; those equal keys are then admitted by ascending
// candidate index.  No floating-point atomics: the result is exact and
// deterministic.  The input-dependent budget reuses that
// descent with integer mass histograms to find how many candidates a pool
// keeps (the REDtech article's section 6.2 names choosing the rate from the
// input; the mass-coverage rule is this library's reading).
//
// Compaction (new lengths, image boundaries and original spatial indices,
// REDtech article section 3.2): per-block keep counts, then a scatter pass
// that forms each block's offset from those counts, recomputes each token's
// flag and writes its original index and (image, row, col), plus the image
// counts (integer atomics); very long layouts put a one-block scan between
// the two.  A separate gather copies embedding rows with 16-byte vector
// loads.
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

// Pools of up to kTopkThreads * kTopkRegKeys candidates keep their keys in
// registers for all passes: key j of thread t is candidate t + 1024 j, so
// every load and flag store of a wave covers 64 consecutive candidates.
// Histogram adds are merged per thread while its consecutive keys share a
// digit (a pool's scores mostly share their leading digits, so unmerged adds
// would serialise on one address).  Keys equal to tau are admitted in index
// order, i.e. by (j, wave, lane): ballots count them per (j, wave), one
// block scan over those counts gives each (j, wave) its offset.
constexpr int kTopkRegKeys = 32;
constexpr int kTopkWaves = kTopkThreads / 64;

// known: tau = `known_tau` and `known_kr` keys equal to it are kept (the
// caller found them already, and that the pool holds `known_neq` keys equal
// to tau, or -1); the descent is skipped.  LDS: hist 512 ints,
// eqbuf RK * 16 ints.
template <int RK>
__device__ __forceinline__ void topk_registers(const float *score, int n, int k, uint8_t *keep,
                                               int *hist, int *sh, int *eqbuf, int &s_digit, int &s_above,
                                               bool known = false, uint32_t known_tau = 0u,
                                               int known_kr = 0, int known_neq = -1) {
  const int tid = threadIdx.x, lane = lane_id(), wid = tid >> 6;
  // Loads from clamped indices without branches, so that all are in flight
  // at once; keys past the pool are masked out by index below.
  float f[RK];
#pragma unroll
  for (int j = 0; j < RK; ++j) f[j] = score[min(tid + kTopkThreads * j, n - 1)];
  uint32_t u[RK];
#pragma unroll
  for (int j = 0; j < RK; ++j) u[j] = score_key(f[j]);
  uint32_t prefix = known ? known_tau : 0u, pmask = 0u;
  int kr = known ? known_kr : k;  // how many of the keys matching `prefix` must still be kept
  int neq = known ? known_neq : -1;  // keys equal to tau, when known (-1: not known)
  // Two histograms (hist[0..511]) alternate between passes, so clearing the
  // next one overlaps this pass's digit walk: two barriers per pass.
  if (!known) {
    if (tid < 512) hist[tid] = 0;
    __syncthreads();
  }
  for (int pass = 0; pass < (known ? 0 : 4); ++pass) {
    const int shift = 24 - 8 * pass;
    int *H = hist + 256 * (pass & 1);
    int cur = -1, cnt = 0;
#pragma unroll
    for (int j = 0; j < RK; ++j) {
      if (tid + kTopkThreads * j < n && (u[j] & pmask) == prefix) {
        const int d = (int)((u[j] >> shift) & 255u);
        if (d != cur) {
          if (cnt) atomicAdd(&H[cur], cnt);
          cur = d;
          cnt = 0;
        }
        ++cnt;
      }
    }
    if (cnt) atomicAdd(&H[cur], cnt);
    __syncthreads();
    if (wid == 0) {
      // Wave 0 walks the digits from 255 down: lane l holds 255-4l .. 252-4l.
      int c[4], csum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = H[255 - 4 * lane - j];
        csum += c[j];
      }
      int cb = wave_incl_scan(csum) - csum;  // keys with a larger digit
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cb < kr && cb + c[j] >= kr) {
          s_digit = 255 - 4 * lane - j;
          s_above = cb;
          sh[0] = c[j];
        }
        cb += c[j];
      }
    } else if (tid < 64 + 256) {
      hist[256 * ((pass + 1) & 1) + tid - 64] = 0;
    }
    __syncthreads();
    kr -= s_above;
    prefix |= (uint32_t)s_digit << shift;
    pmask |= 255u << shift;
    if (pass == 3) neq = sh[0];
  }
  // prefix = tau; the kr lowest-index keys equal to tau are kept.  When all
  // of them are (the usual case: ties at tau are rare), no ranks are needed.
  if (neq == kr) {
#pragma unroll
    for (int j = 0; j < RK; ++j) {
      const int i = tid + kTopkThreads * j;
      if (i < n) keep[i] = (u[j] >= prefix) ? 1 : 0;
    }
    return;
  }
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < RK; ++j) {
    const unsigned long long m = __ballot(tid + kTopkThreads * j < n && u[j] == prefix);
    if (lane == 0) eqbuf[j * kTopkWaves + wid] = __popcll(m);
  }
  __syncthreads();
  int tot;
  const int cv = (tid < RK * kTopkWaves) ? eqbuf[tid] : 0;
  const int cx = block_excl_scan(cv, sh, tot);
  if (tid < RK * kTopkWaves) eqbuf[tid] = cx;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < RK; ++j) {
    const int i = tid + kTopkThreads * j;
    const bool e = i < n && u[j] == prefix;
    const unsigned long long m = __ballot(e);
    const int rank = eqbuf[j * kTopkWaves + wid] + __popcll(m & below);
    if (i < n) keep[i] = (u[j] > prefix || (e && rank < kr)) ? 1 : 0;
  }
}

// Keep flags of one pool of n candidates: the k largest keys, equal keys by
// ascending index.  Every thread of the 1024-thread block calls it.
__device__ __forceinline__ void topk_pool(const float *score, int n, int k, uint8_t *keep, int *hist, int *sh,
                                          int *eqbuf, int &s_digit, int &s_above, bool known = false,
                                          uint32_t known_tau = 0u, int known_kr = 0, int known_neq = -1) {
  const int tid = threadIdx.x;
  if (n <= 0) return;
  if (k <= 0 || k >= n) {
    const uint8_t f = (k >= n) ? 1 : 0;
    for (int i = tid; i < n; i += kTopkThreads) keep[i] = f;
    return;
  }
  if (n <= kTopkThreads * kTopkRegKeys) {
    // Register runs sized to the pool: short runs skip the empty iterations.
    const int per = (n + kTopkThreads - 1) / kTopkThreads;
    if (per <= 1) topk_registers<1>(score, n, k, keep, hist, sh, eqbuf, s_digit, s_above, known, known_tau, known_kr,
                                           known_neq);
    else if (per <= 4) topk_registers<4>(score, n, k, keep, hist, sh, eqbuf, s_digit, s_above, known, known_tau, known_kr,
                                           known_neq);
    else if (per <= 16) topk_registers<16>(score, n, k, keep, hist, sh, eqbuf, s_digit, s_above, known, known_tau, known_kr,
                                           known_neq);
    else topk_registers<kTopkRegKeys>(score, n, k, keep, hist, sh, eqbuf, s_digit, s_above, known, known_tau, known_kr,
                                           known_neq);
    return;
  }
  uint32_t prefix = known ? known_tau : 0u, pmask = 0u;
  int kr = known ? known_kr : k;  // how many of the keys matching `prefix` must still be kept
  for (int pass = 0; pass < (known ? 0 : 4); ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = score_key(score[i]);
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
    const uint32_t u = (i < n) ? score_key(score[i]) : 0u;
    const int eq = (i < n && u == prefix) ? 1 : 0;
    int tot;
    const int rank = block_excl_scan(eq, sh, tot) + seen;
    if (i < n) keep[i] = (u > prefix || (eq && rank < kr)) ? 1 : 0;
    seen += tot;
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(DevLayout L, const float *score,
                                                           TopkChunk ks, uint8_t *keep) {
  __shared__ int hist[512];
  __shared__ int sh[17];
  __shared__ int eqbuf[kTopkRegKeys * kTopkWaves];
  __shared__ int s_digit, s_above;
  const int b = ks.b0 + blockIdx.x;
  const int lo = L.cu_cands[L.cu_images[b]];
  const int hi = L.cu_cands[L.cu_images[b + 1]];
  if (hi - lo > kTopkRegLimit) return;  // spread over many blocks (topk_large_*)
  topk_pool(score + lo, hi - lo, ks.k[blockIdx.x], keep + lo, hist, sh, eqbuf, s_digit, s_above);
}

// ---------------------------------------------------------------------------
// Top-k of pools larger than kTopkRegLimit candidates, spread over blocks of
// kTopkSplit candidates: four launches of the MSB-first radix descent (each
// block adds its chunk's digit histogram to the pool's with integer atomics;
// the last block of the pool to finish, found with an atomic counter after a
// fence, picks the digit and clears the histogram for the next pass), then a
// count of the keys equal to tau per block, then the flags (keys equal to tau
// ranked by index across the pool's blocks in block order).
// ---------------------------------------------------------------------------

// The large pool slot and chunk of block `bid`.
__device__ __forceinline__ int large_slot(const TopkLarge &tl, int bid) {
  int i = 0;
  while (i + 1 < tl.np && tl.blk[i + 1] <= bid) ++i;
  return i;
}

__device__ __forceinline__ void large_pool_range(const DevLayout &L, const TopkLarge &tl, int i, int &lo, int &n) {
  const int b = tl.pool[i];
  lo = L.cu_cands[L.cu_images[b]];
  n = L.cu_cands[L.cu_images[b + 1]] - lo;
}

__global__ __launch_bounds__(256) void topk_large_init(TopkLarge tl, TopkLargeWs ws) {
  const int i = blockIdx.x;
  ws.hist[256 * i + threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    ws.state[4 * i + 0] = 0;         // tau prefix
    ws.state[4 * i + 1] = tl.k[i];   // keys still to keep among those matching the prefix
    ws.state[4 * i + 2] = -1;        // keys equal to tau (after the last pass)
    ws.state[4 * i + 3] = 0;         // blocks of this pass done
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_large_pass(DevLayout L, const float *score, TopkLarge tl,
                                                               TopkLargeWs ws, int pass) {
  __shared__ int hist[256];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = lane_id();
  const int i = large_slot(tl, blockIdx.x);
  int lo, n;
  large_pool_range(L, tl, i, lo, n);
  const int k = tl.k[i];
  if (k <= 0 || k >= n) return;
  const int c0 = (blockIdx.x - tl.blk[i]) * kTopkSplit, c1 = min(c0 + kTopkSplit, n);
  const int shift = 24 - 8 * pass;
  const uint32_t pmask = pass == 0 ? 0u : 0xffffffffu << (shift + 8);
  const uint32_t prefix = (uint32_t)ws.state[4 * i + 0];
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int c = c0 + tid; c < c1; c += kTopkThreads) {
    const uint32_t u = score_key(score[lo + c]);
    if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
  }
  __syncthreads();
  int *H = ws.hist + 256 * i;
  if (tid < 256 && hist[tid] != 0) atomicAdd(&H[tid], hist[tid]);
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int nblk = tl.blk[i + 1] - tl.blk[i];
    s_last = atomicAdd(&ws.state[4 * i + 3], 1) == nblk - 1;
  }
  __syncthreads();
  if (!s_last || tid >= 64) return;
  // The pool's last block: walk the digits from 255 down (lane l holds
  // 255-4l .. 252-4l), reading the counts at the device level.
  __threadfence();
  const int kr = ws.state[4 * i + 1];
  int c[4], csum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = __hip_atomic_load(&H[255 - 4 * lane - j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    csum += c[j];
  }
  int cb = wave_incl_scan(csum) - csum;  // keys with a larger digit
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (cb < kr && cb + c[j] >= kr) {
      ws.state[4 * i + 0] = (int)(prefix | ((uint32_t)(255 - 4 * lane - j) << shift));
      ws.state[4 * i + 1] = kr - cb;
      ws.state[4 * i + 2] = c[j];
    }
    cb += c[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) H[4 * lane + j] = 0;
  if (lane == 0) ws.state[4 * i + 3] = 0;
}

// Keys equal to tau per block, when not all of them are kept.
__global__ __launch_bounds__(kTopkThreads) void topk_large_count(DevLayout L, const float *score, TopkLarge tl,
                                                                TopkLargeWs ws) {
  __shared__ int sh[17];
  const int tid = threadIdx.x;
  const int i = large_slot(tl, blockIdx.x);
  int lo, n;
  large_pool_range(L, tl, i, lo, n);
  const int k = tl.k[i];
  if (k <= 0 || k >= n || ws.state[4 * i + 2] == ws.state[4 * i + 1]) return;
  const uint32_t tau = (uint32_t)ws.state[4 * i + 0];
  const int c0 = (blockIdx.x - tl.blk[i]) * kTopkSplit, c1 = min(c0 + kTopkSplit, n);
  int cnt = 0;
  for (int c = c0 + tid; c < c1; c += kTopkThreads) cnt += score_key(score[lo + c]) == tau ? 1 : 0;
  int tot;
  block_excl_scan(cnt, sh, tot);
  if (tid == 0) ws.blkeq[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kTopkThreads) void topk_large_flags(DevLayout L, const float *score, TopkLarge tl,
                                                                TopkLargeWs ws, uint8_t *keep) {
  __shared__ int sh[17];
  const int tid = threadIdx.x;
  const int i = large_slot(tl, blockIdx.x);
  int lo, n;
  large_pool_range(L, tl, i, lo, n);
  const int k = tl.k[i];
  const int c0 = (blockIdx.x - tl.blk[i]) * kTopkSplit, c1 = min(c0 + kTopkSplit, n);
  if (k <= 0 || k >= n) {
    for (int c = c0 + tid; c < c1; c += kTopkThreads) keep[lo + c] = k >= n ? 1 : 0;
    return;
  }
  const uint32_t tau = (uint32_t)ws.state[4 * i + 0];
  const int kr = ws.state[4 * i + 1], neq = ws.state[4 * i + 2];
  if (neq == kr) {
    for (int c = c0 + tid; c < c1; c += kTopkThreads) keep[lo + c] = score_key(score[lo + c]) >= tau ? 1 : 0;
    return;
  }
  // Keys equal to tau before this block, in block order.
  int seen = 0;
  for (int b = tl.blk[i]; b < (int)blockIdx.x; ++b) seen += ws.blkeq[b];
  for (int base = c0; base < c1; base += kTopkThreads) {
    const int c = base + tid;
    const uint32_t u = c < c1 ? score_key(score[lo + c]) : 0u;
    const int eq = (c < c1 && u == tau) ? 1 : 0;
    int tot;
    const int rank = block_excl_scan(eq, sh, tot) + seen;
    if (c < c1) keep[lo + c] = (u > tau || (eq && rank < kr)) ? 1 : 0;
    seen += tot;
  }
}

// ---------------------------------------------------------------------------
// Input-dependent budget.  Mass of a candidate in integer units of 2^-32:
// floor(min(s, 1) * 2^32) for a finite s > 0, else 0; mass never decreases
// with the score, so the candidates ranked first are the heaviest.  Per pool:
// total M, target = min(M, ceil((tau * M) * (1 - 1e-12))) in binary64, and
// k* = fewest top-ranked candidates whose mass reaches the target, found by
// the same MSB-first radix descent as the top-k with per-digit mass (64-bit
// integer) as well as count histograms: the descent stops at the key whose
// candidates (all of one mass m*) complete the target, k* = (candidates
// above it) + ceil(remaining / m*).  Integer sums make k* independent of the
// summation order.
// ---------------------------------------------------------------------------
// Mass of the candidate whose order key is u, in integer arithmetic on the
// float's bits: a finite positive score s = man * 2^(ex - 150) (ex the biased
// exponent, man the 24-bit significand) has floor(s * 2^32) = man shifted by
// ex - 118; s >= 1 clamps to 2^32; non-finite, zero and negative scores (keys
// at or below 0x80000000) carry none.
__device__ __forceinline__ unsigned long long key_mass(uint32_t u) {
  if (u <= 0x80000000u) return 0ull;
  const uint32_t bits = u & 0x7fffffffu;
  if (bits >= 0x3f800000u) return 1ull << 32;
  const int ex = (int)(bits >> 23);
  if (ex < 95) return 0ull;  // s < 2^-32 (subnormals included)
  const uint32_t man = (bits & 0x7fffffu) | 0x800000u;
  const int sh = ex - 118;
  return (unsigned long long)(sh >= 0 ? (man << sh) : (man >> (-sh)));
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

__global__ __launch_bounds__(kTopkThreads) void mass_budget_kernel(DevLayout L, const float *score, MassChunk mc,
                                                                  int *k_out, uint8_t *keep) {
  __shared__ int hist[512];  // two count histograms, alternating between passes
  __shared__ int sh[17];
  __shared__ int eqbuf[kTopkRegKeys * kTopkWaves];
  __shared__ int s_digit, s_above;
  __shared__ unsigned long long hmass[512];  // two mass histograms, likewise
  __shared__ unsigned long long s_target, s_mabove, s_mstar;
  __shared__ int s_neq;
  __shared__ int s_k;
  const int b = mc.b0 + blockIdx.x;
  const int lo = L.cu_cands[L.cu_images[b]];
  const int n = L.cu_cands[L.cu_images[b + 1]] - lo;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid >> 6;
  const float *sc = score + lo;
  // Pools of up to kTopkThreads * kTopkRegKeys candidates keep their keys in
  // registers as the top-k does (key j of thread t is candidate t + 1024 j)
  // and merge histogram adds while a thread's consecutive keys share a digit.
  const bool regs = n <= kTopkThreads * kTopkRegKeys;
  const int nr = regs ? n : 0;
  uint32_t u[kTopkRegKeys];
  if (nr > 0) {  // loads from clamped indices, all in flight at once
    float f[kTopkRegKeys];
#pragma unroll
    for (int j = 0; j < kTopkRegKeys; ++j) f[j] = sc[min(tid + kTopkThreads * j, nr - 1)];
#pragma unroll
    for (int j = 0; j < kTopkRegKeys; ++j) u[j] = score_key(f[j]);
  } else {
#pragma unroll
    for (int j = 0; j < kTopkRegKeys; ++j) u[j] = 0u;
  }

  uint32_t prefix = 0u, pmask = 0u;
  unsigned long long R = 0ull;  // mass still to cover among keys matching `prefix`
  unsigned long long mstar = 0ull;
  int kstar = 0, neq = -1;
  // Two count and mass histograms alternate between passes (wave 0 walks one
  // while the other waves clear the other): two barriers per pass.
  if (tid < 512) {
    hist[tid] = 0;
    hmass[tid] = 0ull;
  }
  __syncthreads();
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    int *H = hist + 256 * (pass & 1);
    unsigned long long *M = hmass + 256 * (pass & 1);
    if (regs) {
      // (Recompute the masses every pass: kept across passes they would take
      // 64 more registers per thread.)
#pragma unroll
      for (int j = 0; j < kTopkRegKeys; ++j) asm volatile("" : "+v"(u[j]));
      int cur = -1, cnt = 0;
      unsigned long long ms = 0ull;
#pragma unroll
      for (int j = 0; j < kTopkRegKeys; ++j) {
        if (tid + kTopkThreads * j < nr && (u[j] & pmask) == prefix) {
          const int d = (int)((u[j] >> shift) & 255u);
          if (d != cur) {
            if (cnt) {
              atomicAdd(&H[cur], cnt);
              if (ms) atomicAdd(&M[cur], ms);
            }
            cur = d;
            cnt = 0;
            ms = 0ull;
          }
          ++cnt;
          ms += key_mass(u[j]);
        }
      }
      if (cnt) {
        atomicAdd(&H[cur], cnt);
        if (ms) atomicAdd(&M[cur], ms);
      }
    } else {
      for (int i = tid; i < n; i += kTopkThreads) {
        const uint32_t v = score_key(sc[i]);
        if ((v & pmask) == prefix) {
          const int d = (int)((v >> shift) & 255u);
          atomicAdd(&H[d], 1);
          const unsigned long long m = key_mass(v);
          if (m) atomicAdd(&M[d], m);
        }
      }
    }
    __syncthreads();
    if (wid == 0) {
      // Wave 0 walks the digits from 255 down: lane l holds 255-4l .. 252-4l.
      unsigned long long mj[4], msum = 0ull;
      int cj[4], csum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mj[j] = M[255 - 4 * lane - j];
        cj[j] = H[255 - 4 * lane - j];
        msum += mj[j];
        csum += cj[j];
      }
      unsigned long long mb = wave_incl_scan_u64(msum);  // inclusive for now
      unsigned long long Rw = R;
      if (pass == 0) {
        // The first histogram covers the whole pool: total mass and target.
        const unsigned long long total = __shfl(mb, 63, 64);
        const double x = ceil((mc.tau[blockIdx.x] * (double)total) * (1.0 - 1e-12));
        const unsigned long long tg = (unsigned long long)x;
        Rw = tg < total ? tg : total;
        if (lane == 0) s_target = Rw;
      }
      mb -= msum;                                // mass of larger digits
      int cb = wave_incl_scan(csum) - csum;      // count of larger digits
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (mb < Rw && mb + mj[j] >= Rw) {
          s_digit = 255 - 4 * lane - j;
          s_above = cb;
          s_mabove = mb;
          s_mstar = cj[j] ? mj[j] / (unsigned long long)cj[j] : 0ull;  // last pass: one key, one mass
          s_neq = cj[j];                                               // ... and its count
        }
        mb += mj[j];
        cb += cj[j];
      }
    } else if (tid < 64 + 256) {
      hist[256 * ((pass + 1) & 1) + tid - 64] = 0;
      hmass[256 * ((pass + 1) & 1) + tid - 64] = 0ull;
    }
    __syncthreads();
    if (pass == 0) {
      R = s_target;
      if (R == 0ull) break;  // uniform across the block
    }
    R -= s_mabove;
    kstar += s_above;
    prefix |= (uint32_t)s_digit << shift;
    pmask |= 255u << shift;
    if (pass == 3) {
      mstar = s_mstar;
      neq = s_neq;
    }
  }
  // R > 0 here only if the descent ran: the candidates of key `prefix` (each
  // of mass mstar) complete the target, and the k*-th largest key is
  // `prefix` itself, with `need` of its candidates kept.
  int need = 0;
  if (R > 0ull) {
    need = (int)((R + mstar - 1ull) / mstar);
    kstar += need;
  }
  if (tid == 0) {
    const int k = min(max(kstar, mc.kmin[blockIdx.x]), mc.kmax[blockIdx.x]);
    s_k = k;
    k_out[b] = k;
  }
  __syncthreads();
  const int k = s_k;
  // Unclamped and inside the pool: reuse the threshold; otherwise select anew.
  const bool known = need > 0 && k == kstar && k < n;
  topk_pool(sc, n, k, keep + lo, hist, sh, eqbuf, s_digit, s_above, known, prefix, need, neq);
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
  // Fused path: the scatter adds the per-image counts up, so clear them here.
  if (c.fused && c.out_img_counts != nullptr)
    for (int i = blockIdx.x * kCompactBlock + threadIdx.x; i < c.L.S; i += gridDim.x * kCompactBlock)
      c.out_img_counts[i] = 0;
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
      int cnt = 0, i = c0 + lane;
      for (; i + 448 < c1; i += 512) {  // eight independent loads in flight
        int t = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += c.keep[i + 64 * j] ? 1 : 0;
        cnt += t;
      }
      for (; i < c1; i += 64) cnt += c.keep[i] ? 1 : 0;
      cnt = wave_sum(cnt);
      if (lane == 0) c.out_img_counts[s] = cnt;
    }
  }
}

// Fused path (c.fused): every block sums the counts of the blocks before it
// (a few dozen for the usual sizes), the last block writes the total and the
// trailing requests, and each wave adds its kept image tokens to their
// images' counts, one integer atomic per (wave, image).
__global__ __launch_bounds__(kCompactBlock) void compact_scatter(CompactArgs c) {
  __shared__ int sh[17];
  __shared__ int s_base;
  const int t = blockIdx.x * kCompactBlock + threadIdx.x;
  int s = -1, off = 0;
  const int k = (t < c.L.T) ? token_keep(c.L, c.keep, t, s, off) : 0;
  if (c.fused && threadIdx.x < 64) {
    int v = 0;
    for (int i = threadIdx.x; i < (int)blockIdx.x; i += 64) v += c.blk_cnt[i];
    v = wave_sum(v);
    if (threadIdx.x == 0) s_base = v;
  }
  int tot;
  const int ex = block_excl_scan(k, sh, tot);  // its barriers also publish s_base
  const int base = c.fused ? s_base : c.blk_off[blockIdx.x];
  const int pos = base + ex;
  if (c.fused) {
    if (blockIdx.x == gridDim.x - 1) {
      if (threadIdx.x == 0) *c.total = base + tot;
      if (c.out_cu_seqlens != nullptr)
        for (int b = threadIdx.x; b <= c.L.B; b += kCompactBlock)
          if (c.L.cu_seqlens[b] == c.L.T) c.out_cu_seqlens[b] = base + tot;
    }
    if (c.out_img_counts != nullptr) {
      const bool mine = k && s >= 0;
      unsigned long long m = __ballot(mine);
      while (m) {  // wave-uniform
        const int l0 = __ffsll((long long)m) - 1;
        const int s0 = __shfl(s, l0, 64);
        const unsigned long long same = __ballot(mine && s == s0);
        if (lane_id() == l0) atomicAdd(&c.out_img_counts[s0], (int)__popcll(same));
        m &= ~same;
      }
    }
  }
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

hipError_t launch_topk_large(const DevLayout &L, const float *score, const TopkLarge &tl, const TopkLargeWs &ws,
                             uint8_t *keep, hipStream_t s) {
  if (tl.np <= 0) return hipSuccess;
  const int nblk = tl.blk[tl.np];
  hipLaunchKernelGGL(topk_large_init, dim3(tl.np), dim3(256), 0, s, tl, ws);
  for (int pass = 0; pass < 4; ++pass)
    hipLaunchKernelGGL(topk_large_pass, dim3(nblk), dim3(kTopkThreads), 0, s, L, score, tl, ws, pass);
  hipLaunchKernelGGL(topk_large_count, dim3(nblk), dim3(kTopkThreads), 0, s, L, score, tl, ws);
  hipLaunchKernelGGL(topk_large_flags, dim3(nblk), dim3(kTopkThreads), 0, s, L, score, tl, ws, keep);
  return hipGetLastError();
}

hipError_t launch_mass_budget(const DevLayout &L, const float *score, const MassChunk &mc, int npools,
                              int *k_out, uint8_t *keep, hipStream_t s) {
  if (npools <= 0) return hipSuccess;
  hipLaunchKernelGGL(mass_budget_kernel, dim3(npools), dim3(kTopkThreads), 0, s, L, score, mc, k_out, keep);
  return hipGetLastError();
}

// Up to kCompactFusedBlocks token blocks (4M tokens) the scatter forms its
// own offsets (two launches); beyond, and for an empty layout, a one-block
// scan runs between count and scatter.
constexpr int kCompactFusedBlocks = 4096;

hipError_t launch_compact(const CompactArgs &args, hipStream_t s) {
  CompactArgs c = args;
  c.fused = (c.nblk > 0 && c.nblk <= kCompactFusedBlocks) ? 1 : 0;
  if (c.nblk > 0) {
    hipLaunchKernelGGL(compact_count, dim3(c.nblk), dim3(kCompactBlock), 0, s, c);
  }
  if (!c.fused) hipLaunchKernelGGL(compact_scan, dim3(1), dim3(kCompactBlock), 0, s, c);
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
