// topk_select kernels: exact per-request Top-k by radix selection on an
// order-preserving 32-bit key, ties broken toward the lower token index.
//
// Key: NaN -> 0 (below everything), -0.0 -> +0.0, then the usual sign flip so
// that unsigned order equals numeric order.  The selection is the k_eff best
// entries under (key desc, index asc), a total order, so the result is unique
// whatever order atomics land in.
//
// Launches per call (all on the caller's stream):
//  1. tau: one workgroup per request derives its threshold key tau from a
//     sample of its keys (all of them when the request has at most 4096,
//     else 16 evenly spread runs of 256):
//     one histogram of the sample over the 11 bits below the bits its keys
//     share, and tau the lower edge of the bin holding the sample key of
//     rank r: k when the sample is the whole request, else e + 4 sqrt(e) + 4
//     where e = k * 4096 / L is the expected count of sampled keys at or
//     above the request's k-th largest key, so somewhat more than k keys of
//     the request reach tau (fewer only if the sample count falls four
//     deviations short).
//  2. collect: (request, 4096-key chunk) workgroups.  Each copies its
//     chunk's keys >= tau, with their indices and in token order, to the
//     chunk's own slice of the candidate buffer, and writes their count and
//     smallest and largest key (no atomics, so nothing needs clearing
//     between calls).
//  3. finish: one workgroup per request gathers the chunks' candidates into
//     LDS (still in token order) and selects the k_eff best exactly: 11-bit
//     rounds over the key from the highest bit in which the candidates
//     differ; once the bin holding the k-th best key has at most 64 keys,
//     one wave ranks them by (key, index) and the k-th best fixes the
//     threshold; otherwise the rounds go on and ties are split by rounds
//     over the index.  The selected indices are written in ascending order
//     by one block scan over the token-ordered candidates.  Should tau admit
//     fewer than k keys (the sample fell far short: vanishingly rare for any
//     spread of scores, but adversarial orders can do it), or more than fit
//     in LDS (huge tie groups), the same steps run over the whole request
//     read from the scores, so the result is exact in every case.
//
// Rows of at most 64K keys (max_len), 16-byte aligned, take one launch
// instead (topk_fused_kernel): one workgroup per request does all three
// steps, with the candidates going straight to LDS; same candidates, same
// selection, same result.
#include "common.h"
#include "launch.h"
#include "topk_layout.h"

#include <algorithm>

namespace spmla {

constexpr int kBins = 2048;
constexpr int kFinThreads = 1024;
constexpr int kTauThreads = 1024;                // 4 sample keys per thread
constexpr int kMaxK = 4096;
constexpr int kSampleRuns = 16, kSampleRun = 256;
constexpr int kSample = kSampleRuns * kSampleRun;  // keys sampled from a long request
constexpr int kFinLdsWords = 32768;              // 128 KiB of gathered candidates
constexpr int kCandLds = kFinLdsWords / 2;       // candidates that fit in LDS (uint2 each)
static_assert(kSample == kTkChunk, "a collect workgroup holds one sample key per chunk key");

struct TopkWs {
  uint32_t* tau;    // [B] threshold key of each request longer than k
  uint4* meta;      // [B, chunks] (candidate count, smallest key, largest key, 0) of each chunk
  uint2* cand;      // [B, chunks, kTkChunk] (key, index), chunk c's in its own slice, ascending index
  int32_t chunks;
};

static TopkWs carve(void* ws, int32_t batch, int64_t max_len) {
  TopkWs w;
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  w.chunks = n_chunks(max_len);
  const size_t bc = (size_t)batch * (size_t)w.chunks;
  w.tau = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * 4, 256);
  w.meta = reinterpret_cast<uint4*>(p);
  w.cand = reinterpret_cast<uint2*>(p + align_up(bc * 16, 256));
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

// Block scan helpers (any block size that is a multiple of 64).
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

// Radix rounds over a key set whose smallest and largest keys are known
// start at the highest bit in which those two differ: the bits above are
// common to every key (returned as prefix and mask), and the first 11-bit
// round spreads the keys instead of piling them into a few bins.
__device__ __forceinline__ int first_round_top(uint32_t kmin, uint32_t kmax, uint32_t* pre, uint32_t* mask) {
  const uint32_t diff = kmin ^ kmax;
  const int top = diff ? 32 - __clz(diff) : 1;  // bits [0, top) can differ
  const int hi = max(top, 11);
  *mask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
  *pre = kmin & *mask;
  return hi;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
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

// Threshold key tau of a request whose length exceeds k (see the top of the
// file); called by all NT threads, barriers inside.
template <int NT>
__device__ __forceinline__ uint32_t request_tau(const float* __restrict__ s, int32_t L, int32_t k, uint32_t* h, uint32_t* tmp,
                                uint32_t* res, uint32_t* s_mm) {
  constexpr int PER = kSample / NT;
  const int tid = threadIdx.x;
  const bool whole = L <= kSample;
  uint32_t key[PER];
  bool in[PER];
  {
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = j * NT + tid;
      int64_t t;
      if (whole) {
        t = e;
      } else {
        const int64_t run = e / kSampleRun;
        t = run * ((int64_t)L - kSampleRun) / (kSampleRuns - 1) + e % kSampleRun;
      }
      in[j] = t < L;
      v[j] = s[in[j] ? t : 0];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) key[j] = order_key(v[j]);
  }
  uint32_t lo_k = 0xFFFFFFFFu, hi_k = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (in[j]) { lo_k = min(lo_k, key[j]); hi_k = max(hi_k, key[j]); }
  lo_k = wave_min_u32(lo_k);
  hi_k = wave_max_u32(hi_k);
  if (tid == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
  for (int i = tid; i < kBins; i += NT) h[i] = 0u;
  __syncthreads();
  if ((tid & 63) == 0) { atomicMin(&s_mm[0], lo_k); atomicMax(&s_mm[1], hi_k); }
  __syncthreads();
  uint32_t pre, mask;
  const int hi = first_round_top(s_mm[0], s_mm[1], &pre, &mask);
  const int lo = hi - 11;
  // Rank r of tau's bin in the sample: k for the whole request, else
  // e + 4 sqrt(e) + 4 with e = k * kSample / L.
  uint32_t need = (uint32_t)k;
  if (!whole) {
    const float e = (float)k * (float)kSample / (float)L;
    const float r = e + 4.f * sqrtf(e) + 4.f;
    need = (uint32_t)min((int64_t)kSample, (int64_t)ceilf(r));
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (in[j]) atomicAdd(&h[(key[j] >> lo) & 2047u], 1u);
  __syncthreads();
  find_bin_desc<kBins, NT>(h, need, tmp, res);
  return pre | (res[0] << lo);
}

// One workgroup per request longer than k: its tau into the workspace.
__global__ __launch_bounds__(kTauThreads) void topk_tau_kernel(const float* __restrict__ scores, int64_t stride,
                                                               const int32_t* __restrict__ lens, int64_t max_len,
                                                               int32_t k, TopkWs ws) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t tmp[kTauThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t s_mm[2];
  const int b = blockIdx.x;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const uint32_t tau = request_tau<kTauThreads>(scores + (int64_t)b * stride, L, k, h, tmp, res, s_mm);
  if (threadIdx.x == 0) ws.tau[b] = tau;
}

// (request, chunk) workgroups: every key >= tau goes to the chunk's slice of
// the candidate buffer in ascending token order, and the chunk's count and
// smallest and largest candidate keys to its metadata slot.  Key j of
// thread tid is token t0 + j*256 + tid, so token order is row j first: each
// wave ballots its selected keys row by row, and one wave scan over the 64
// (row, wave) counts gives every key its place.
__global__ __launch_bounds__(kTkThreads) void topk_collect_kernel(const float* __restrict__ scores, int64_t stride,
                                                                  const int32_t* __restrict__ lens, int64_t max_len,
                                                                  int32_t k, TopkWs ws) {
  __shared__ uint32_t res[2];
  __shared__ uint32_t s_mm[2];
  __shared__ uint32_t rw[kTkPer * (kTkThreads / 64)];  // (row, wave) counts, then their exclusive scan
  static_assert(kTkPer * (kTkThreads / 64) == 64, "one wave scans the (row, wave) counts");
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int b = logical / ws.chunks, chunk = logical % ws.chunks;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int n_act = (int)((L + kTkChunk - 1) / kTkChunk);
  if (chunk >= n_act) return;
  const float* s = scores + (int64_t)b * stride;
  const int64_t t0 = (int64_t)chunk * kTkChunk, t1 = min((int64_t)L, t0 + kTkChunk);
  uint32_t key[kTkPer];
  bool in[kTkPer];
  load_chunk(s, t0, t1, key, in);
  const uint32_t tau = ws.tau[b];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t rank[kTkPer];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const bool sel = in[j] && key[j] >= tau;
    const uint64_t m = __ballot(sel);
    rank[j] = (uint32_t)__popcll(m & below);
    if (lane == 0) rw[j * (kTkThreads / 64) + wv] = (uint32_t)__popcll(m);
    if (sel) { kmin = min(kmin, key[j]); kmax = max(kmax, key[j]); }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (threadIdx.x == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
  __syncthreads();
  if (lane == 0) { atomicMin(&s_mm[0], kmin); atomicMax(&s_mm[1], kmax); }
  if (wv == 0) {
    const uint32_t v = rw[lane];
    const uint32_t incl = wave_incl_scan(v);
    rw[lane] = incl - v;
    if (lane == 63) res[0] = incl;
  }
  __syncthreads();
  const int64_t slot = (int64_t)b * ws.chunks + chunk;
  if (threadIdx.x == 0) ws.meta[slot] = make_uint4(res[0], s_mm[0], s_mm[1], 0u);
  uint2* cb = ws.cand + slot * kTkChunk;
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const int64_t t = t0 + (int64_t)j * kTkThreads + threadIdx.x;
    if (in[j] && key[j] >= tau) cb[rw[j * (kTkThreads / 64) + wv] + rank[j]] = make_uint2(key[j], (uint32_t)t);
  }
}

// Exact selection of the k best of n_c candidates held in ascending token
// order -- the (key, index) list `lc` in LDS or, when `whole`, every key of
// the score row `srow` -- with their indices written to `out` in that order.
// [cmin, cmax] bounds the listed keys.  Called by all kFinThreads threads
// after a barrier that follows *bin_cnt = 0; barriers inside.
__device__ __forceinline__ void select_k_best(const uint2* lc, const float* __restrict__ srow, bool whole, uint32_t n_c,
                              uint32_t cmin, uint32_t cmax, int32_t k, int32_t* __restrict__ out, uint32_t* h,
                              uint32_t* tmp, uint32_t* res, uint2* bin_list, uint32_t* bin_cnt) {
  const int tid = threadIdx.x;
  auto cand = [&](uint32_t j) -> uint2 { return whole ? make_uint2(order_key(srow[j]), j) : lc[j]; };
  uint32_t need = (uint32_t)k;
  // Key rounds, 11 bits at a time from the highest bit in which the
  // candidates can differ (they lie in [smallest, largest collected key];
  // all 32 bits for the whole request).  After a round, a boundary bin of at
  // most 64 keys is finished by one wave ranking them instead of further
  // rounds.
  uint32_t kpre = 0, kmask = 0;  // determined high-bit prefix
  int hi0 = 32;
  if (!whole) hi0 = first_round_top(cmin, cmax, &kpre, &kmask);
  uint32_t T = 0, I = 0xFFFFFFFFu;  // selection: key > T, or key == T and index <= I
  bool done = false;
  for (int hi = hi0; hi > 0 && !done; hi -= 11) {
    const int lo = max(hi - 11, 0);
    const uint32_t wmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < kBins; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < n_c; j += kFinThreads) {
      const uint32_t key = cand(j).x;
      if ((key & kmask) == kpre) atomicAdd(&h[(key >> lo) & wmask], 1u);
    }
    __syncthreads();
    find_bin_desc<kBins, kFinThreads>(h, need, tmp, res);
    const uint32_t bin = res[0];
    kpre |= bin << lo;
    kmask |= wmask << lo;
    need -= res[1];
    const uint32_t in_bin = h[bin];
    __syncthreads();  // h and res are read before the next round rewrites them
    if (in_bin <= 64u) {
      // The keys of the boundary bin: the `need` best of them (by key, then
      // index; indices are distinct, so the order is total) complete the
      // selection.
      for (uint32_t j = tid; j < n_c; j += kFinThreads) {
        const uint2 e = cand(j);
        if ((e.x & kmask) == kpre) bin_list[atomicAdd(bin_cnt, 1u)] = e;
      }
      __syncthreads();
      if (tid < (int)in_bin) {
        // Rank of this lane's key among the bin's keys (larger key first,
        // then smaller index); the entry of rank need - 1 is the last one
        // selected.  Every lane reads the same LDS word at a time.
        const uint2 e = bin_list[tid];
        uint32_t rank = 0;
        for (uint32_t m = 0; m < in_bin; ++m) {
          const uint2 o = bin_list[m];
          rank += (o.x > e.x || (o.x == e.x && o.y < e.y)) ? 1u : 0u;
        }
        if (rank == need - 1) { res[0] = e.x; res[1] = e.y; }
      }
      __syncthreads();
      T = res[0];
      I = res[1];
      done = true;
    }
  }
  if (!done) {
    // T = kpre.  Among keys equal to T take the `need` lowest indices (index
    // threshold I, inclusive).
    T = kpre;
    for (int i = tid; i < kBins; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    uint32_t n_eq_local = 0;
    for (uint32_t j = tid; j < n_c; j += kFinThreads) n_eq_local += (cand(j).x == T) ? 1u : 0u;
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
          const uint2 e = cand(j);
          if (e.x == T && (e.y & imask) == ipre) atomicAdd(&h[(e.y >> lo) & wmask], 1u);
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
  // The candidates are in ascending token order, so the selected ones are
  // written in order by one block scan: thread tid takes a contiguous run.
  const uint32_t per = (n_c + kFinThreads - 1) / kFinThreads;
  const uint32_t j0 = min(n_c, tid * per), j1 = min(n_c, j0 + per);
  auto picked = [&](const uint2 e) { return e.x > T || (e.x == T && e.y <= I); };
  uint32_t mine = 0;
  for (uint32_t j = j0; j < j1; ++j) mine += picked(cand(j)) ? 1u : 0u;
  uint32_t pos = block_incl_scan<kFinThreads>(mine, tmp) - mine;
  for (uint32_t j = j0; j < j1 && pos < (uint32_t)k; ++j) {
    const uint2 e = cand(j);
    if (picked(e)) out[pos++] = (int32_t)e.y;
  }
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const float* __restrict__ scores, int64_t stride,
                                                                  const int32_t* __restrict__ lens, int64_t max_len,
                                                                  int32_t k, TopkWs ws, int32_t* __restrict__ out_idx,
                                                                  int32_t* __restrict__ status) {
  __shared__ uint32_t big[kFinLdsWords];   // gathered candidates (uint2)
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t tmp[kFinThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t coff[kFinThreads];  // chunk offsets in the gathered candidate list
  __shared__ uint32_t ccnt[kFinThreads];  // chunk candidate counts
  __shared__ uint32_t s_mm[2];
  __shared__ uint2 bin_list[64];           // members of the boundary bin, when few
  __shared__ uint32_t bin_cnt;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
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
  // Candidates: the chunks' keys >= tau gathered into LDS in token order, or,
  // should fewer than k or more than LDS holds have reached tau (or the
  // request have more chunks than this workgroup has threads), every key of
  // the request read from the scores.
  const int n_act = (int)((L + kTkChunk - 1) / kTkChunk);
  const int64_t slot0 = (int64_t)b * ws.chunks;
  const uint4 meta = (tid < n_act) ? ws.meta[slot0 + tid] : make_uint4(0u, 0xFFFFFFFFu, 0u, 0u);
  if (tid == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
  const uint32_t c_incl = block_incl_scan<kFinThreads>(meta.x, tmp);
  if (tid < n_act) { coff[tid] = c_incl - meta.x; ccnt[tid] = meta.x; }
  if (tid == kFinThreads - 1) res[0] = c_incl;
  {
    const uint32_t wmin = wave_min_u32(meta.y), wmax = wave_max_u32(meta.z);
    if (lane == 0) { atomicMin(&s_mm[0], wmin); atomicMax(&s_mm[1], wmax); }
  }
  __syncthreads();
  const uint32_t n_cand = res[0];
  const bool whole = n_cand < (uint32_t)k || n_cand > (uint32_t)kCandLds || n_act > kFinThreads;
  const uint32_t n_c = whole ? (uint32_t)L : n_cand;
  const float* srow = scores + (int64_t)b * stride;
  uint2* lc = reinterpret_cast<uint2*>(big);
  if (!whole) {
    // Wave w copies chunks w, w + 16, ...: each chunk's slice goes to its
    // offset in the gathered list.
    for (int c = tid >> 6; c < n_act; c += kFinThreads / 64) {
      const uint32_t n = ccnt[c], off = coff[c];
      const uint2* src = ws.cand + (slot0 + c) * kTkChunk;
      for (uint32_t i = lane; i < n; i += 64) lc[off + i] = src[i];
    }
  }
  const uint32_t cmin = s_mm[0], cmax = s_mm[1];
  if (tid == 0) bin_cnt = 0u;
  __syncthreads();
  select_k_best(lc, srow, whole, n_c, cmin, cmax, k, out, h, tmp, res, bin_list, &bin_cnt);
}

// Single-launch form for rows of up to kFusedMaxLen keys: one workgroup per
// request derives tau, gathers the request's keys >= tau into LDS in token
// order and selects.  Wave w streams the w-th of kFinThreads / 64 (16)
// equal token segments (multiples of 256 tokens that together cover the
// row; 4 consecutive keys per lane and 16-byte load, kFusedUnroll loads in
// flight) and appends its candidates, in token order, to its own
// kWaveCand-entry LDS region; the regions are then packed into one list.  Fewer than k candidates in all, or more than kWaveCand in one
// segment, make the selection run over the whole request read from the
// scores.  Score rows must be 16-byte aligned.
constexpr int kWaveCand = kCandLds / (kFinThreads / 64);
static_assert(kWaveCand % 64 == 0, "a wave packs its region in whole 64-entry rows");
constexpr int kFusedUnroll = 8;
// One CU streams a whole row here: past 64K keys (256 KB) the three launches,
// which spread a row over many CUs, are faster (c3f, rows to 128K: 41.6
// against 31.7 us; c4, rows to 64K: 28.0 against 35.1 us).
constexpr int64_t kFusedMaxLen = 65536;

__global__ __launch_bounds__(kFinThreads) void topk_fused_kernel(const float* __restrict__ scores, int64_t stride,
                                                                 const int32_t* __restrict__ lens, int64_t max_len,
                                                                 int32_t k, int32_t* __restrict__ out_idx,
                                                                 int32_t* __restrict__ status) {
  __shared__ uint32_t big[kFinLdsWords];   // wave regions, then the packed candidate list (uint2)
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t tmp[kFinThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t s_mm[2];
  __shared__ uint32_t c_mm[2];             // smallest and largest candidate key
  __shared__ uint32_t wcnt[kFinThreads / 64];
  __shared__ uint32_t ovf;
  __shared__ uint2 bin_list[64];
  __shared__ uint32_t bin_cnt;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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
  const float* srow = scores + (int64_t)b * stride;
  if (tid == 0) { c_mm[0] = 0xFFFFFFFFu; c_mm[1] = 0u; ovf = 0u; bin_cnt = 0u; }
  const uint32_t tau = request_tau<kFinThreads>(srow, L, k, h, tmp, res, s_mm);  // barriers inside

  constexpr int kWaves = kFinThreads / 64;  // one token segment per wave
  const int64_t seg = ((int64_t)(L + kWaves - 1) / kWaves + 255) / 256 * 256;
  const int64_t s0 = (int64_t)wv * seg, s1 = min((int64_t)L, s0 + seg);
  uint2* region = reinterpret_cast<uint2*>(big) + wv * kWaveCand;
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t cnt = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int64_t g = s0; g < s1; g += 256 * kFusedUnroll) {
    float4 v[kFusedUnroll];
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) {
      const int64_t t = g + u * 256 + lane * 4;
      v[u] = t < s1 ? *reinterpret_cast<const float4*>(srow + t) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) {
      const int64_t t = g + u * 256 + lane * 4;
      const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t key[4];
      bool sel[4];
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[e] = order_key(f[e]);
        sel[e] = t + e < s1 && key[e] >= tau;
        const uint64_t m = __ballot(sel[e]);
        before += (uint32_t)__popcll(m & below);
        total += (uint32_t)__popcll(m);
      }
      uint32_t pos = cnt + before;  // token order: lanes below first, then this lane's earlier keys
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (sel[e]) {
          if (pos < (uint32_t)kWaveCand) region[pos] = make_uint2(key[e], (uint32_t)(t + e));
          kmin = min(kmin, key[e]);
          kmax = max(kmax, key[e]);
          ++pos;
        }
      }
      cnt += total;
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    wcnt[wv] = cnt;
    atomicMin(&c_mm[0], kmin);
    atomicMax(&c_mm[1], kmax);
    if (cnt > (uint32_t)kWaveCand) ovf = 1u;
  }
  __syncthreads();
  uint32_t off = 0, n_cand = 0;
#pragma unroll
  for (int w = 0; w < kFinThreads / 64; ++w) {
    const uint32_t c = wcnt[w];
    off += w < wv ? c : 0u;
    n_cand += c;
  }
  const bool whole = ovf != 0u || n_cand < (uint32_t)k;
  uint2* lc = reinterpret_cast<uint2*>(big);
  if (!whole) {
    // Pack the regions: every wave takes its entries into registers, then
    // (after the barrier) writes them at its offset in the list.
    uint2 e[kWaveCand / 64];
#pragma unroll
    for (int r = 0; r < kWaveCand / 64; ++r) {
      const uint32_t i = (uint32_t)(r * 64 + lane);
      if (i < cnt) e[r] = region[i];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kWaveCand / 64; ++r) {
      const uint32_t i = (uint32_t)(r * 64 + lane);
      if (i < cnt) lc[off + i] = e[r];
    }
    __syncthreads();
  }
  select_k_best(lc, srow, whole, whole ? (uint32_t)L : n_cand, c_mm[0], c_mm[1], k, out, h, tmp, res, bin_list,
                &bin_cnt);
}

int launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  if (a.k > kMaxK || a.k < 1) return -2;
  if (a.max_len <= kFusedMaxLen && reinterpret_cast<uintptr_t>(a.scores) % 16 == 0 && a.score_stride % 4 == 0) {
    hipLaunchKernelGGL(topk_fused_kernel, dim3((unsigned)a.batch), dim3(kFinThreads), 0, s, a.scores,
                       a.score_stride, a.lens, a.max_len, a.k, a.out_idx, a.status);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
  TopkWs ws = carve(a.workspace, a.batch, a.max_len);
  const int64_t grid = (int64_t)a.batch * ws.chunks;
  if (grid > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL(topk_tau_kernel, dim3((unsigned)a.batch), dim3(kTauThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws);
  hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)grid), dim3(kTkThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws);
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.batch), dim3(kFinThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws, a.out_idx, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
