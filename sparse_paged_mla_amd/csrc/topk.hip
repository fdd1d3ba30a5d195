// topk_select kernels: exact per-request Top-k by radix selection on an
// order-preserving 32-bit key, ties broken toward the lower token index.
//
// Key: NaN -> 0 (below everything), -0.0 -> +0.0, then the usual sign flip so
// that unsigned order equals numeric order.  The selection is the k_eff best
// entries under (key desc, index asc), a total order, so the result is unique
// whatever order atomics land in.
//
// Launches per call (all on the caller's stream), over (request, chunk)
// workgroups except the last:
//  1. range:  each chunk's min and max key go to the workspace, and the chunk
//             clears its share of the request's histogram and counters.
//  2. hist:   every chunk folds the per-chunk ranges into the request's key
//             range, picks the 11-bit digit that starts at the highest bit in
//             which the request's keys differ (so the digit spreads whatever
//             the score scale), histograms it in LDS and adds the histogram
//             into the request's global one.
//  3. filter: every chunk finds the bin b0 holding the k-th best key and
//             streams its keys again: keys above b0 are selected outright,
//             keys in b0 become candidates.  Each thread counts both, one
//             block scan gives every thread its offsets and each workgroup
//             reserves its output ranges with one atomic per kind.
//  4. finish: one workgroup per request resolves the candidates in LDS
//             (further 11-bit rounds on the remaining key bits, then on the
//             token index for exact ties) and writes the k_eff indices in
//             ascending order: they are set in an LDS bitmap over [0, L) and
//             read back with a prefix popcount (bitonic sort when L exceeds
//             the bitmap).
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace spmla {

constexpr int kTkThreads = 256;
constexpr int kTkPer = 16;                       // keys per thread per chunk
constexpr int kTkChunk = kTkThreads * kTkPer;    // 4096 keys per workgroup
constexpr int kBins = 2048;
constexpr int kFinThreads = 1024;
constexpr int kMaxK = 4096;
constexpr int kCtrl = 8;                         // selected count, candidate count, digit shift
constexpr int kFinLdsWords = 32768;              // 128 KiB: candidates, then the bitmap
constexpr int kCandLds = kFinLdsWords / 2;       // candidates that fit in LDS (uint2 each)
constexpr int64_t kBitmapBits = (int64_t)kFinLdsWords * 32;

struct TopkWs {
  uint32_t* hist;   // [B, kBins]
  uint32_t* ctrl;   // [B, kCtrl]
  uint2* range;     // [B, chunks] (min key, max key)
  uint2* cand;      // [B, cap] (key, index)
  int64_t cap;
  int32_t chunks;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
static inline int32_t n_chunks(int64_t max_len) { return (int32_t)std::max<int64_t>(1, (max_len + kTkChunk - 1) / kTkChunk); }

size_t topk_workspace_size(int32_t batch, int64_t max_len, int32_t k) {
  (void)k;
  if (batch <= 0 || max_len < 0) return 0;
  const size_t b = (size_t)batch;
  return align_up(b * kBins * 4, 256) + align_up(b * kCtrl * 4, 256) + align_up(b * n_chunks(max_len) * 8, 256) +
         align_up(b * (size_t)std::max<int64_t>(max_len, 1) * 8, 256);
}

static TopkWs carve(void* ws, int32_t batch, int64_t max_len) {
  TopkWs w;
  const size_t b = (size_t)batch;
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  w.chunks = n_chunks(max_len);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align_up(b * kBins * 4, 256);
  w.ctrl = reinterpret_cast<uint32_t*>(p);
  p += align_up(b * kCtrl * 4, 256);
  w.range = reinterpret_cast<uint2*>(p);
  p += align_up(b * w.chunks * 8, 256);
  w.cand = reinterpret_cast<uint2*>(p);
  w.cap = std::max<int64_t>(max_len, 1);
  return w;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN ranks lowest
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool len_ok(int32_t L, int64_t max_len) { return L >= 0 && (int64_t)L <= max_len; }

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Block reduction helpers (any block size that is a multiple of 64).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)v, o);
    if (lane >= o) v += t;
  }
  return v;
}
// Inclusive block scan; `tmp` holds one word per wave.  Contains barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = v;
  __syncthreads();
  uint32_t pre = 0;
  for (int i = 0; i < wid; ++i) pre += tmp[i];
  __syncthreads();
  return v + pre;
}

// The digit that starts at the highest bit where the request's keys differ.
__device__ __forceinline__ int digit_shift(uint32_t kmin, uint32_t kmax) {
  const uint32_t diff = kmin ^ kmax;
  const int hb = diff ? 31 - __clz(diff) : 0;
  return max(hb + 1 - 11, 0);
}

__device__ __forceinline__ void request_range(const uint2* rng, int n, uint32_t* s_mm) {
  // Called by all threads; result in s_mm[0..1] after the trailing barrier.
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint2 r = rng[i];
    lo = min(lo, r.x);
    hi = max(hi, r.y);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (threadIdx.x == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { atomicMin(&s_mm[0], lo); atomicMax(&s_mm[1], hi); }
  __syncthreads();
}

// Thread-to-key mapping of a chunk: key j of thread tid is t0 + j*256 + tid
// (coalesced loads, all issued before any use).
__device__ __forceinline__ void load_chunk(const float* s, int64_t t0, int64_t t1, uint32_t* key, bool* in) {
  float v[kTkPer];
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const int64_t t = t0 + (int64_t)j * kTkThreads + threadIdx.x;
    in[j] = t < t1;
    v[j] = s[in[j] ? t : t1 - 1];  // unconditional load (t1 - 1 is in range)
  }
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) key[j] = order_key(v[j]);
}

__global__ __launch_bounds__(kTkThreads) void topk_range_kernel(const float* __restrict__ scores, int64_t stride,
                                                                const int32_t* __restrict__ lens, int64_t max_len,
                                                                int32_t k, TopkWs ws) {
  __shared__ uint32_t s_mm[2];
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int b = logical / ws.chunks, chunk = logical % ws.chunks;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int n_act = (int)((L + kTkChunk - 1) / kTkChunk);
  if (chunk >= n_act) return;
  // This chunk's share of the request's histogram (and the counters, chunk 0).
  const int per = (kBins + n_act - 1) / n_act;
  for (int i = chunk * per + threadIdx.x; i < min(kBins, (chunk + 1) * per); i += kTkThreads)
    ws.hist[(int64_t)b * kBins + i] = 0u;
  if (chunk == 0 && threadIdx.x < kCtrl) ws.ctrl[(int64_t)b * kCtrl + threadIdx.x] = 0u;
  const int64_t t0 = (int64_t)chunk * kTkChunk, t1 = min((int64_t)L, t0 + kTkChunk);
  uint32_t key[kTkPer];
  bool in[kTkPer];
  load_chunk(scores + (int64_t)b * stride, t0, t1, key, in);
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    if (in[j]) { lo = min(lo, key[j]); hi = max(hi, key[j]); }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (threadIdx.x == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { atomicMin(&s_mm[0], lo); atomicMax(&s_mm[1], hi); }
  __syncthreads();
  if (threadIdx.x == 0) ws.range[(int64_t)b * ws.chunks + chunk] = make_uint2(s_mm[0], s_mm[1]);
}

__global__ __launch_bounds__(kTkThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t stride,
                                                               const int32_t* __restrict__ lens, int64_t max_len,
                                                               int32_t k, TopkWs ws) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t s_mm[2];
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int b = logical / ws.chunks, chunk = logical % ws.chunks;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int n_act = (int)((L + kTkChunk - 1) / kTkChunk);
  if (chunk >= n_act) return;
  const int64_t t0 = (int64_t)chunk * kTkChunk, t1 = min((int64_t)L, t0 + kTkChunk);
  uint32_t key[kTkPer];
  bool in[kTkPer];
  load_chunk(scores + (int64_t)b * stride, t0, t1, key, in);
  for (int i = threadIdx.x; i < kBins; i += kTkThreads) h[i] = 0u;
  request_range(ws.range + (int64_t)b * ws.chunks, n_act, s_mm);
  const int sh = digit_shift(s_mm[0], s_mm[1]);
#pragma unroll
  for (int j = 0; j < kTkPer; ++j)
    if (in[j]) atomicAdd(&h[(key[j] >> sh) & (kBins - 1)], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)b * kBins;
  for (int i = threadIdx.x; i < kBins; i += kTkThreads) {
    const uint32_t c = h[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// Block-wide search over a histogram in LDS from the top bin down: the bin x
// with sum_{y > x} h[y] < need <= sum_{y >= x} h[y], and that sum above.
// NB a multiple of NT; need in [1, total].  Result in out[0..1]; barriers inside.
template <int NB, int NT>
__device__ void find_bin_desc(const uint32_t* h, uint32_t need, uint32_t* tmp, uint32_t* out) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  const int hi = NB - tid * PER;  // thread 0 owns the top PER bins
  uint32_t mine = 0;
#pragma unroll
  for (int j = 1; j <= PER; ++j) mine += h[hi - j];
  if (tid == 0) { out[0] = 0u; out[1] = 0u; }
  const uint32_t incl = block_incl_scan<NT>(mine, tmp);
  const uint32_t excl = incl - mine;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
    for (int j = 1; j <= PER; ++j) {
      const uint32_t c = h[hi - j];
      if (run + c >= need) { out[0] = (uint32_t)(hi - j); out[1] = run; break; }
      run += c;
    }
  }
  __syncthreads();
}

// Same from the lowest bin up (smallest indices first).
template <int NB, int NT>
__device__ void find_bin_asc(const uint32_t* h, uint32_t need, uint32_t* tmp, uint32_t* out) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  const int lo = tid * PER;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) mine += h[lo + j];
  if (tid == 0) { out[0] = 0u; out[1] = 0u; }
  const uint32_t incl = block_incl_scan<NT>(mine, tmp);
  const uint32_t excl = incl - mine;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
    for (int j = 0; j < PER; ++j) {
      const uint32_t c = h[lo + j];
      if (run + c >= need) { out[0] = (uint32_t)(lo + j); out[1] = run; break; }
      run += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTkThreads) void topk_filter_kernel(const float* __restrict__ scores, int64_t stride,
                                                                 const int32_t* __restrict__ lens, int64_t max_len,
                                                                 int32_t k, TopkWs ws, int32_t* __restrict__ out_idx) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t tmp[kTkThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t s_mm[2];
  __shared__ uint32_t base_sel, base_cnd;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int b = logical / ws.chunks, chunk = logical % ws.chunks;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int n_act = (int)((L + kTkChunk - 1) / kTkChunk);
  if (chunk >= n_act) return;
  const int64_t t0 = (int64_t)chunk * kTkChunk, t1 = min((int64_t)L, t0 + kTkChunk);
  uint32_t key[kTkPer];
  bool in[kTkPer];
  load_chunk(scores + (int64_t)b * stride, t0, t1, key, in);
  const uint32_t* gh = ws.hist + (int64_t)b * kBins;
  for (int i = threadIdx.x; i < kBins; i += kTkThreads) h[i] = gh[i];
  request_range(ws.range + (int64_t)b * ws.chunks, n_act, s_mm);
  const int sh = digit_shift(s_mm[0], s_mm[1]);
  find_bin_desc<kBins, kTkThreads>(h, (uint32_t)k, tmp, res);
  const uint32_t b0 = res[0];
  if (chunk == 0 && threadIdx.x == 0) ws.ctrl[(int64_t)b * kCtrl + 2] = (uint32_t)sh;
  // Two-phase compaction: count this thread's selected keys (above b0) and
  // candidates (in b0), one block scan of both counts packed in a word, one
  // global atomic per kind for the whole chunk, then direct writes.
  uint32_t cs = 0, cc = 0;
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const uint32_t d = (key[j] >> sh) & (kBins - 1);
    cs += (in[j] && d > b0) ? 1u : 0u;
    cc += (in[j] && d == b0) ? 1u : 0u;
  }
  const uint32_t packed = (cs << 16) | cc;  // at most kTkPer each
  const uint32_t incl = block_incl_scan<kTkThreads>(packed, tmp);
  if (threadIdx.x == kTkThreads - 1) {
    const uint32_t ns = incl >> 16, nc = incl & 0xFFFFu;
    base_sel = ns ? atomicAdd(ws.ctrl + (int64_t)b * kCtrl + 0, ns) : 0u;
    base_cnd = nc ? atomicAdd(ws.ctrl + (int64_t)b * kCtrl + 1, nc) : 0u;
  }
  __syncthreads();
  uint32_t ps = base_sel + ((incl - packed) >> 16), pc = base_cnd + ((incl - packed) & 0xFFFFu);
  int32_t* out = out_idx + (int64_t)b * k;
  uint2* cb = ws.cand + (int64_t)b * ws.cap;
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const uint32_t d = (key[j] >> sh) & (kBins - 1);
    const int64_t t = t0 + (int64_t)j * kTkThreads + threadIdx.x;
    if (in[j] && d > b0) out[ps++] = (int32_t)t;
    if (in[j] && d == b0) cb[pc++] = make_uint2(key[j], (uint32_t)t);
  }
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const int32_t* __restrict__ lens, int64_t max_len,
                                                                  int32_t k, TopkWs ws, int32_t* __restrict__ out_idx,
                                                                  int32_t* __restrict__ status) {
  __shared__ uint32_t big[kFinLdsWords];   // candidates (uint2), later the bitmap
  __shared__ uint32_t h[kBins];
  __shared__ int32_t sel[kMaxK];
  __shared__ uint32_t tmp[kFinThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t s_mm[2];
  __shared__ uint32_t cnt;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t L = lens[b];
  int32_t* out = out_idx + (int64_t)b * k;
  if (!len_ok(L, max_len)) {
    if (tid == 0 && status) atomicOr(status + b, kBadLen);
    for (int j = tid; j < k; j += kFinThreads) out[j] = -1;
    return;
  }
  if (L <= k) {
    for (int j = tid; j < k; j += kFinThreads) out[j] = j < L ? j : -1;
    return;
  }
  const int sh = (int)ws.ctrl[(int64_t)b * kCtrl + 2];  // the digit shift the filter used
  const uint32_t n_gt = ws.ctrl[(int64_t)b * kCtrl + 0];
  const uint32_t n_c = ws.ctrl[(int64_t)b * kCtrl + 1];
  // Candidates: in LDS when they fit, else read from the workspace.
  const uint2* cb = ws.cand + (int64_t)b * ws.cap;
  uint2* lc = reinterpret_cast<uint2*>(big);
  const bool in_lds = n_c <= (uint32_t)kCandLds;
  if (in_lds) {
    for (uint32_t j = tid; j < n_c; j += kFinThreads) lc[j] = cb[j];
    cb = lc;
  }
  __syncthreads();
  uint32_t need = (uint32_t)k - n_gt;  // >= 1 places for keys of bin b0
  // Key rounds over the bits below the first digit, 11 at a time.
  uint32_t kpre = 0, kmask = 0;  // determined low-bit prefix
  for (int hi = sh; hi > 0; hi -= 11) {
    const int lo = max(hi - 11, 0);
    const uint32_t wmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < kBins; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < n_c; j += kFinThreads) {
      const uint32_t key = cb[j].x;
      if ((key & kmask) == kpre) atomicAdd(&h[(key >> lo) & wmask], 1u);
    }
    __syncthreads();
    find_bin_desc<kBins, kFinThreads>(h, need, tmp, res);
    kpre |= res[0] << lo;
    kmask |= wmask << lo;
    need -= res[1];
  }
  // Threshold key T: candidates share bits >= sh (they are all in bin b0 of a
  // request whose keys agree above the digit); the low bits are kpre.
  // Among keys equal to T take the `need` lowest indices (index threshold I, inclusive).
  uint32_t I = 0xFFFFFFFFu;
  {
    for (int i = tid; i < kBins; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    uint32_t n_eq_local = 0;
    for (uint32_t j = tid; j < n_c; j += kFinThreads) n_eq_local += ((cb[j].x & kmask) == kpre) ? 1u : 0u;
    const uint32_t n_eq = block_incl_scan<kFinThreads>(n_eq_local, tmp);  // last thread holds the total
    if (tid == kFinThreads - 1) res[0] = n_eq;
    __syncthreads();
    const uint32_t total_eq = res[0];
    __syncthreads();
    if (total_eq > need) {
      uint32_t ipre = 0, imask = 0;
      for (int hi = 31; hi > 0; hi -= 11) {
        const int lo = max(hi - 11, 0);
        const uint32_t wmask = (1u << (hi - lo)) - 1u;
        for (int i = tid; i < kBins; i += kFinThreads) h[i] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < n_c; j += kFinThreads) {
          const uint2 e = cb[j];
          if ((e.x & kmask) == kpre && (e.y & imask) == ipre) atomicAdd(&h[(e.y >> lo) & wmask], 1u);
        }
        __syncthreads();
        find_bin_asc<kBins, kFinThreads>(h, need, tmp, res);
        ipre |= res[0] << lo;
        imask |= wmask << lo;
        need -= res[1];
      }
      I = ipre;
    }
  }
  // Gather the k indices: the n_gt already in the output row plus the chosen candidates.
  if (tid == 0) cnt = n_gt;
  for (uint32_t j = tid; j < n_gt; j += kFinThreads) sel[j] = out[j];
  __syncthreads();
  for (uint32_t j = tid; j < n_c; j += kFinThreads) {
    const uint2 e = cb[j];
    const uint32_t low = e.x & kmask;
    if (low > kpre || (low == kpre && e.y <= I)) {
      const uint32_t p = atomicAdd(&cnt, 1u);
      if (p < (uint32_t)k) sel[p] = (int32_t)e.y;
    }
  }
  __syncthreads();
  if ((int64_t)L <= kBitmapBits) {
    // Ascending order via an LDS bitmap over [0, L) and a prefix popcount.
    const int words = (int)((L + 31) / 32);
    for (int i = tid; i < words; i += kFinThreads) big[i] = 0u;
    __syncthreads();
    for (int j = tid; j < k; j += kFinThreads) {
      const int32_t t = sel[j];
      atomicOr(&big[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
    const int per = (words + kFinThreads - 1) / kFinThreads;
    const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
    uint32_t mine = 0;
    for (int i = w0; i < w1; ++i) mine += __popc(big[i]);
    uint32_t pos = block_incl_scan<kFinThreads>(mine, tmp) - mine;
    for (int i = w0; i < w1; ++i) {
      uint32_t m = big[i];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1u;
        out[pos++] = i * 32 + bit;
      }
    }
  } else {
    // Bitonic sort of the k entries (padded with INT_MAX) in place.
    int n2 = 1;
    while (n2 < k) n2 <<= 1;
    for (int j = k + tid; j < n2; j += kFinThreads) sel[j] = 0x7FFFFFFF;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2 / 2; i += kFinThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int32_t a = sel[lo], c = sel[hi];
          if ((a > c) == up) { sel[lo] = c; sel[hi] = a; }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < k; j += kFinThreads) out[j] = sel[j];
  }
}

int launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  if (a.k > kMaxK || a.k < 1) return -2;
  TopkWs ws = carve(a.workspace, a.batch, a.max_len);
  const int64_t grid = (int64_t)a.batch * ws.chunks;
  if (grid > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL(topk_range_kernel, dim3((unsigned)grid), dim3(kTkThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws);
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)grid), dim3(kTkThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws);
  hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)grid), dim3(kTkThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws, a.out_idx);
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.batch), dim3(kFinThreads), 0, s, a.lens, a.max_len, a.k,
                     ws, a.out_idx, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
