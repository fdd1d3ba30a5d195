// topk_select kernels: exact per-request Top-k by radix selection on an
// order-preserving 32-bit key, ties broken toward the lower token index.
//
// Key: NaN -> 0 (below everything), -0.0 -> +0.0, then the usual sign flip so
// that unsigned order equals numeric order.  The selection is the k_eff best
// entries under (key desc, index asc), a total order, so the result is unique
// whatever order atomics land in.
//
// Launches per call (both on the caller's stream):
//  1. collect: (request, 8192-key chunk) workgroups.  Each requests its
//     chunk's keys first (a row holds max_len entries, so the loads need not
//     wait for the request's length), then derives the request's threshold
//     key tau from a sample of its keys (all of them when the request has at
//     most 4096, else 16 evenly spread runs of 256): one histogram of the
//     sample over the 11 bits below the bits its keys share, and tau the
//     lower edge of the bin holding the sample key of rank r: k when the
//     sample is the whole request, else e + 4 sqrt(e) + 4 where
//     e = k * 4096 / L is the expected count of sampled keys at or above the
//     request's k-th largest key, so somewhat more than k keys of the
//     request reach tau (fewer only if the sample count falls four
//     deviations short).  Every chunk of a request draws the same sample, so
//     all of them find the same tau.  The chunk's keys >= tau go, with their
//     indices and in token order, to its own slice of the candidate buffer
//     (at most kTkSlice of them), and their count and smallest and largest
//     key to its metadata slot (no atomics, so nothing needs clearing
//     between calls).
//  2. finish: one workgroup per request gathers the chunks' candidates into
//     LDS (still in token order; every thread finds the chunk of each of
//     its list positions by binary search, so all the loads are in flight
//     at once) and selects the k_eff best exactly: 11-bit rounds over the
//     key from the highest bit in which the candidates differ; once the bin
//     holding the k-th best key has at most 64 keys, one wave ranks them by
//     (key, index) and the k-th best fixes the threshold; otherwise the
//     rounds go on and ties are split by rounds over the index.  The
//     selected indices are written in ascending order by one block scan over
//     the token-ordered candidates.  Should tau admit fewer than k keys (the
//     sample fell far short: vanishingly rare for any spread of scores, but
//     adversarial orders can do it), more than a chunk's slice holds or more
//     than fit in LDS (huge tie groups), the same steps run over the whole
//     request read from the scores, so the result is exact in every case.
//
// Rows of at most 64K keys (max_len), 16-byte aligned, take one launch
// instead (topk_fused_kernel): one workgroup per request does all three
// steps, with the candidates going straight to LDS; same candidates, same
// selection, same result.
#include "common.h"
#include "launch.h"
#include "topk_layout.h"

#include <algorithm>
#include <type_traits>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

namespace spmla {

constexpr int kBins = 2048;
constexpr int kFinThreads = 1024;
constexpr int kMaxK = 4096;
constexpr int kSampleRuns = 16, kSampleRun = 256;
constexpr int kSample = kSampleRuns * kSampleRun;  // keys sampled from a long request
constexpr int kFinLdsWords = 32768;              // 128 KiB of gathered candidates
constexpr int kCandLds = kFinLdsWords / 2;       // candidates that fit in LDS (uint2 each)
static_assert(kCandLds % kFinThreads == 0, "the gather gives every thread the same number of list positions");

struct TopkWs {
  unsigned long long* tau_pub;  // [B] (call tag << 32) | threshold key, published by the request's tau block
  uint4* meta;      // [B, chunks] (candidate count, threshold key used, largest key, 0) of each chunk
  uint2* cand;      // [B, chunks, kTkSlice] (score bits, index), chunk c's in its own slice, ascending index
  int32_t chunks;
  uint32_t tag;     // differs from call to call (see launch_topk)
};

static TopkWs carve(void* ws, int32_t batch, int64_t max_len, uint32_t tag) {
  TopkWs w;
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  w.chunks = n_chunks(max_len);
  w.tag = tag;
  const size_t bc = (size_t)batch * (size_t)w.chunks;
  w.tau_pub = reinterpret_cast<unsigned long long*>(p);
  p += align_up((size_t)batch * 8, 256);
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

// The smallest float whose key is at least `key` (key >= 1): every number
// when key is at most that of -inf, none (NaN) when it exceeds that of +inf.
// For such a key and every float f, order_key(f) >= key exactly when
// f >= key_floor(key) (NaN fails both).
__device__ __forceinline__ float key_floor(uint32_t key) {
  if (key <= 0x007FFFFFu) return -INFINITY;
  if (key > 0xFF800000u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__device__ __forceinline__ bool len_ok(int32_t L, int64_t max_len) { return L >= 0 && (int64_t)L <= max_len; }

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Block scan helpers (any block size that is a multiple of 64).
// Inclusive scan over the wave with DPP moves: shifts right by 1, 2, 4 and 8
// lanes within each row of 16 (lanes shifted in from outside the row read
// 0), then the last lane of row 0 added to row 1 and that of row 2 to row 3
// (row_bcast:15), then the last lane of row 1 added to rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  return v;
}
// Inclusive block scan; `tmp` holds one word per wave (16-byte aligned, NT /
// 64 a multiple of 4).  Contains barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* tmp) {
  constexpr int kW = NT / 64;
  static_assert(kW % 4 == 0, "the wave totals are read four at a time");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = v;
  __syncthreads();
  uint4 t[kW / 4];
#pragma unroll
  for (int i = 0; i < kW / 4; ++i) t[i] = reinterpret_cast<const uint4*>(tmp)[i];
  uint32_t pre = 0;
#pragma unroll
  for (int i = 0; i < kW / 4; ++i) {
    pre += 4 * i + 0 < wid ? t[i].x : 0u;
    pre += 4 * i + 1 < wid ? t[i].y : 0u;
    pre += 4 * i + 2 < wid ? t[i].z : 0u;
    pre += 4 * i + 3 < wid ? t[i].w : 0u;
  }
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

// Block-wide search over a histogram in LDS from the top bin down: the bin x
// with sum_{y > x} h[y] < need <= sum_{y >= x} h[y], and that sum above.
// NB a multiple of NT; need in [1, total].  Result in out[0..1]; barriers inside.
template <int NB, int NT>
__device__ void find_bin_desc(const uint32_t* h, uint32_t need, uint32_t* tmp, uint32_t* out) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  const int hi = NB - tid * PER;  // thread 0 owns the top PER bins
  uint32_t c[PER], mine = 0;      // the counts stay in registers for the search below
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = h[hi - 1 - j];
    mine += c[j];
  }
  if (tid == 0) { out[0] = 0u; out[1] = 0u; }
  const uint32_t incl = block_incl_scan<NT>(mine, tmp);
  const uint32_t excl = incl - mine;
  if (excl < need && need <= incl) {
    // the first j (from the top) whose running sum reaches need
    uint32_t run = excl, bin = 0, above = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!found && run + c[j] >= need) { bin = (uint32_t)(hi - 1 - j); above = run; found = true; }
      run += c[j];
    }
    out[0] = bin;
    out[1] = above;
  }
  __syncthreads();
}

// Same from the lowest bin up (smallest indices first).
template <int NB, int NT>
__device__ void find_bin_asc(const uint32_t* h, uint32_t need, uint32_t* tmp, uint32_t* out) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  const int lo = tid * PER;
  uint32_t c[PER], mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = h[lo + j];
    mine += c[j];
  }
  if (tid == 0) { out[0] = 0u; out[1] = 0u; }
  const uint32_t incl = block_incl_scan<NT>(mine, tmp);
  const uint32_t excl = incl - mine;
  if (excl < need && need <= incl) {
    uint32_t run = excl, bin = 0, below = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!found && run + c[j] >= need) { bin = (uint32_t)(lo + j); below = run; found = true; }
      run += c[j];
    }
    out[0] = bin;
    out[1] = below;
  }
  __syncthreads();
}

// Threshold from this thread's N keys (those with in[j]; `need` in [1, their
// count over the workgroup]): the lower edge of the bin holding the key of
// rank `need` from the top, in a histogram over the 11 bits below the bits
// all the keys share.  Called by all NT threads; barriers inside.  With
// kCleared the caller has already zeroed h and set s_mm to (~0, 0), with a
// barrier after.
template <int NT, int N, bool kCleared = false>
__device__ __forceinline__ uint32_t tau_of(const uint32_t (&key)[N], const bool (&in)[N], uint32_t need, uint32_t* h,
                                           uint32_t* tmp, uint32_t* res, uint32_t* s_mm) {
  const int tid = threadIdx.x;
  uint32_t lo_k = 0xFFFFFFFFu, hi_k = 0u;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    lo_k = min(lo_k, in[j] ? key[j] : 0xFFFFFFFFu);
    hi_k = max(hi_k, in[j] ? key[j] : 0u);
  }
  lo_k = wave_min_u32(lo_k);
  hi_k = wave_max_u32(hi_k);
  if constexpr (!kCleared) {
    if (tid == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
    for (int i = tid; i < kBins; i += NT) h[i] = 0u;
    __syncthreads();
  }
  if ((tid & 63) == 0) { atomicMin(&s_mm[0], lo_k); atomicMax(&s_mm[1], hi_k); }
  __syncthreads();
  uint32_t pre, mask;
  const int hi = first_round_top(s_mm[0], s_mm[1], &pre, &mask);
  const int lo = hi - 11;
#pragma unroll
  for (int j = 0; j < N; ++j)
    if (in[j]) atomicAdd(&h[(key[j] >> lo) & 2047u], 1u);
  __syncthreads();
  find_bin_desc<kBins, NT>(h, need, tmp, res);
  return pre | (res[0] << lo);
}

// Rank r of tau's bin in a sample of n_s of a request's L keys:
// e + 4 sqrt(e) + 4 with e = k * n_s / L, the expected count of sampled keys
// at or above the request's k-th largest key.
__device__ __forceinline__ uint32_t sample_need(int32_t k, uint32_t n_s, int32_t L) {
  const float e = (float)k * (float)n_s / (float)L;
  const float r = e + 4.f * sqrtf(e) + 4.f;
  return (uint32_t)min((int64_t)n_s, (int64_t)ceilf(r));
}

// Threshold key tau of a request whose length exceeds k, from kSample keys:
// the whole request when it has at most that many, else 16 runs of 256
// starting evenly over [0, L - 256].  Called by all NT threads; barriers
// inside.
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
  const uint32_t need = whole ? (uint32_t)k : sample_need(k, kSample, L);
  return tau_of<NT, PER>(key, in, need, h, tmp, res, s_mm);
}

// Collect launch: per request one tau block, then its (request, chunk)
// blocks.  Blocks run in the order tau blocks, chunk 0 of every request,
// chunk 1, ...: block index (c + 1) * B8 + b for chunk c of request b, where
// B8 is the batch rounded up to 8, so the tau blocks are dispatched first,
// the active chunks (low chunk numbers) next and spread evenly over the
// CUs, and all of a request's blocks run on XCD b % 8 and share its L2.
//
// tau block (requests longer than one chunk): derives tau from a sample
// placed by max_len, so that its loads need not wait for the request's
// length: 16 runs of 256 starting evenly over [0, max_len - 256], of which
// the keys below L count.  It publishes (tag << 32) | tau, tag being the
// call's own value.
//
// Chunk block: every key >= tau' = max(tau, 1) goes to the chunk's slice of
// the candidate buffer in ascending token order (as the score's bits and
// its index), and the chunk's count, tau' and its largest key to its
// metadata slot.  A request of at most one chunk has all its keys here and
// takes the exact threshold (rank k).  A longer one waits for its tau block
// (the chunk's own loads land meanwhile) and, should the tag not appear
// within a bounded wait, derives tau itself from the same sample.  Either
// way the result is exact: the finish checks that the k-th best candidate is
// at least every chunk's tau', and otherwise selects over the whole request.
// Key j of thread tid is token t0 + j*256 + tid, so token order is row j
// first: each wave ballots its selected keys row by row, and one block scan
// over the 128 (row, wave) counts gives every key its place.  The selection
// compares scores against the float key_floor(tau'), which admits the same
// keys; NaN scores are never candidates (should that leave fewer than k, the
// finish selects over the whole request).
constexpr int kTauSpin = 8000;  // polls of the published threshold (s_sleep 1 between them, four in flight)

template <int NT, bool kCleared = false>
__device__ __forceinline__ uint32_t sample_tau(const float (&sv)[kSampleRuns], int32_t ml, int32_t L, int32_t k, uint32_t* h,
                                               uint32_t* tmp, uint32_t* res, uint32_t* s_mm) {
  uint32_t skey[kSampleRuns];
  bool in[kSampleRuns];
  uint32_t n_s = 0;
#pragma unroll
  for (int j = 0; j < kSampleRuns; ++j) {
    const int32_t r0 = (int32_t)((int64_t)j * (ml - kSampleRun) / (kSampleRuns - 1));
    n_s += (uint32_t)min(max(L - r0, 0), kSampleRun);
    skey[j] = order_key(sv[j]);
    in[j] = r0 + (int)threadIdx.x < L;
  }
  return tau_of<NT, kSampleRuns, kCleared>(skey, in, sample_need(k, n_s, L), h, tmp, res, s_mm);  // barriers inside
}

__global__ __launch_bounds__(kTkThreads) void topk_collect_kernel(const float* __restrict__ scores, int64_t stride,
                                                                  const int32_t* __restrict__ lens, int32_t batch,
                                                                  int64_t max_len, int32_t k, TopkWs ws) {
  constexpr int kWaves = kTkThreads / 64;
  constexpr int kRows = kTkPer * kWaves;
  static_assert(kRows <= kTkThreads && kTkPer <= 64 && kTkPer % 4 == 0, "one block scan covers the (row, wave) counts");
  static_assert(kSampleRun == kTkThreads && kSample / kTkThreads == kSampleRuns,
                "thread tid holds key tid of every sample run");
  __shared__ uint32_t h[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t tmp[kWaves];
  __shared__ uint32_t res[2];
  __shared__ uint32_t s_mm[2];
  __shared__ __attribute__((aligned(16))) uint32_t rw[kRows];  // [wave][row] counts, then their offsets
  __shared__ uint32_t c_max;      // largest key of the chunk
  if (max_len <= 0) return;       // every length is then 0
  const int b8 = (batch + 7) & ~7;
  const int b = (int)blockIdx.x % b8, chunk = (int)blockIdx.x / b8 - 1;
  if (b >= batch) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* s = scores + (int64_t)b * stride;
  const int32_t ml = (int32_t)max_len;  // max_len < 2^31
  auto load_sample = [&](float (&sv)[kSampleRuns]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kSampleRuns; ++j)
      sv[j] = s[(int32_t)((int64_t)j * (ml - kSampleRun) / (kSampleRuns - 1)) + tid];
  };
  if (chunk < 0) {
    // tau block
    if (ml <= kTkChunk) return;  // every request fits one chunk
    float sv[kSampleRuns];
    load_sample(sv);
    // While the sample loads: clear the histogram (a barrier that waits
    // for LDS only, not for the loads in flight).
    for (int i = tid; i < kBins; i += kTkThreads) h[i] = 0u;
    if (tid == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int32_t L = lens[b];
    if (!len_ok(L, max_len) || L <= k || L <= kTkChunk) return;
    const uint32_t tau = sample_tau<kTkThreads, true>(sv, ml, L, k, h, tmp, res, s_mm);
    if (tid == 0)
      __hip_atomic_store(ws.tau_pub + b, ((unsigned long long)ws.tag << 32) | tau, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int32_t t0 = chunk * kTkChunk;
  // (In a block the compiler cannot fold: a plain run of loads whose values
  // only the active path uses gets moved below the length checks, so the
  // loads would wait for the length after all.)
  float v[kTkPer];
  int32_t always = 1;
  asm volatile("" : "+s"(always));
  if (always) {
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) v[j] = s[min(t0 + j * kTkThreads + tid, ml - 1)];
  }
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int n_act = (L + kTkChunk - 1) / kTkChunk;
  if (chunk >= n_act) return;
  if (tid == 0) c_max = 0u;
  if (t0 + kTkChunk > L) {
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) v[j] = t0 + j * kTkThreads + tid < L ? v[j] : __uint_as_float(0x7FC00000u);
  }
  uint32_t tau;
  if (L <= kTkChunk) {
    uint32_t key[kTkPer];
    bool in[kTkPer];
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
      key[j] = order_key(v[j]);
      in[j] = j * kTkThreads + tid < L;
    }
    tau = tau_of<kTkThreads, kTkPer>(key, in, (uint32_t)k, h, tmp, res, s_mm);  // barriers inside
  } else {
    if (tid == 0) {
      // The first polls' loads return after the chunk's loads (loads
      // complete in order), by when the tau block has usually published.
      // Four polls are kept in flight: each check waits for the oldest
      // only, and its slot is refilled at once, so a published word is seen
      // about one load latency after it lands instead of up to two.
      auto poll = [&]() { return __hip_atomic_load(ws.tau_pub + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      uint32_t got = 0, t = 0;
      auto check = [&](unsigned long long w) {
        if (!got && (uint32_t)(w >> 32) == ws.tag) {
          t = (uint32_t)w;
          got = 1;
        }
      };
      // Two sets of four slots take turns (one is checked while the other
      // is refilled), so no loaded value has to move between registers.
      unsigned long long wa[4], wb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) wa[q] = poll();
      for (int it = 0; it < kTauSpin / 8 && !got; ++it) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_s_sleep(1);
          wb[q] = poll();
          check(wa[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_s_sleep(1);
          wa[q] = poll();
          check(wb[q]);
        }
      }
      res[0] = t;
      res[1] = got;
    }
    __syncthreads();
    tau = res[0];
    if (!res[1]) {
      __syncthreads();  // res is read before sample_tau rewrites it
      float sv[kSampleRuns];
      load_sample(sv);
      tau = sample_tau<kTkThreads>(sv, ml, L, k, h, tmp, res, s_mm);
    }
  }
  tau = max(tau, 1u);
  const float ftau = key_floor(tau);
  // Count pass: lane j ends with the count of row j in this wave.
  uint32_t row_cnt = 0;
  float vmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const uint32_t c = (uint32_t)__popcll(__ballot(v[j] >= ftau));
    row_cnt = lane == j ? c : row_cnt;
    vmax = fmaxf(vmax, v[j]);
  }
  for (int o = 32; o > 0; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  if (lane < kTkPer) rw[wv * kTkPer + lane] = row_cnt;
  __syncthreads();  // c_max is cleared before any wave raises it
  if (lane == 0) atomicMax(&c_max, order_key(vmax));
  {
    // exclusive scan in token order: entry (row j, wave w) is thread j * kWaves + w
    const int j = tid / kWaves, w = tid % kWaves;
    const uint32_t cnt = tid < kRows ? rw[w * kTkPer + j] : 0u;
    const uint32_t incl = block_incl_scan<kTkThreads>(cnt, tmp);  // barriers inside
    if (tid < kRows) rw[w * kTkPer + j] = incl - cnt;
    if (tid == kTkThreads - 1) res[0] = incl;
  }
  __syncthreads();
  const uint32_t total = res[0];
  const int64_t slot = (int64_t)b * ws.chunks + chunk;
  if (tid == 0) ws.meta[slot] = make_uint4(total, tau, c_max, 0u);
  if (total > (uint32_t)kTkSlice) return;  // the finish reads the whole request instead
  uint2* cb = ws.cand + slot * kTkSlice;
  uint32_t base[kTkPer];
#pragma unroll
  for (int q = 0; q < kTkPer / 4; ++q) {
    const uint4 r = reinterpret_cast<const uint4*>(rw + wv * kTkPer)[q];
    base[4 * q] = r.x; base[4 * q + 1] = r.y; base[4 * q + 2] = r.z; base[4 * q + 3] = r.w;
  }
  // Write pass: the same ballots give each selected key its rank in its row.
  // (The selection is recomputed from a copy of the threshold the compiler
  // cannot see through: keeping the count pass's 32 lane masks alive
  // instead spills scalar registers.)
  float ftau_w = ftau;
  asm volatile("" : "+v"(ftau_w));
#pragma unroll
  for (int j = 0; j < kTkPer; ++j) {
    const bool sel = v[j] >= ftau_w;
    const uint64_t m = __ballot(sel);
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (sel) cb[base[j] + rank] = make_uint2(__float_as_uint(v[j]), (uint32_t)(t0 + j * kTkThreads + tid));
  }
}

// Exact selection of the k best of n_c candidates held in ascending token
// order -- the (key, index) list `lc` in LDS or, when `whole`, every key of
// the score row `srow` -- with their indices written to `out` in that order.
// [cmin, cmax] bounds the listed keys.  Called by all kFinThreads threads
// after a barrier that follows *bin_cnt = 0; barriers inside.
// Returns false, writing nothing, when the selection over a list comes out
// with a k-th best key below tau_max (the largest threshold a chunk
// collected with: keys between the two may be missing from the list).
__device__ __forceinline__ bool select_k_best(const uint2* lc, const float* __restrict__ srow, bool whole, uint32_t n_c,
                              uint32_t cmin, uint32_t cmax, uint32_t tau_max, int32_t k, int32_t* __restrict__ out,
                              uint32_t* h, uint32_t* tmp, uint32_t* res, uint2* bin_list, uint32_t* bin_cnt) {
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
      if (tid < 64) {
        // Wave 0 holds the bin's keys, one per lane; each lane ranks its own
        // among them (larger key first, then smaller index) from the other
        // lanes' registers; the entry of rank need - 1 is the last one
        // selected.
        const bool mine = tid < (int)in_bin;
        const uint2 e = mine ? bin_list[tid] : make_uint2(0u, 0u);
        uint32_t rank = 0;
        for (uint32_t m = 0; m < in_bin; ++m) {
          const uint32_t ox = (uint32_t)__builtin_amdgcn_readlane((int)e.x, (int)m);
          const uint32_t oy = (uint32_t)__builtin_amdgcn_readlane((int)e.y, (int)m);
          rank += (ox > e.x || (ox == e.x && oy < e.y)) ? 1u : 0u;
        }
        if (mine && rank == need - 1) { res[0] = e.x; res[1] = e.y; }
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
  if (!whole && T < tau_max) return false;  // uniform: T is the same in every thread
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
  return true;
}

// select_k_best over a list held in registers: thread tid holds list
// entries [j0, j0 + n_mine) in e[0 .. n_mine) (j0 = tid * per, per the same
// in every thread, so thread order is list order), each as (key, index).
// Same rounds, bin ranking, tie rounds, tau_max check and ordered output as
// select_k_best, without reading the list again from memory.  Called by all
// kFinThreads threads; barriers inside.
constexpr int kRegCand = kCandLds / kFinThreads;  // list entries a thread can hold
template <int P>
__device__ __forceinline__ bool select_regs(const uint2 (&e)[P], uint32_t n_mine, uint32_t cmin, uint32_t cmax,
                                            uint32_t tau_max, int32_t k, int32_t* __restrict__ out, uint32_t* h,
                                            uint32_t* tmp, uint32_t* res, uint2* bin_list, uint32_t* bin_cnt) {
  const int tid = threadIdx.x;
  uint32_t need = (uint32_t)k;
  uint32_t kpre = 0, kmask = 0;
  const int hi0 = first_round_top(cmin, cmax, &kpre, &kmask);
  uint32_t T = 0, I = 0xFFFFFFFFu;
  bool done = false;
  if (tid == 0) *bin_cnt = 0u;
  for (int hi = hi0; hi > 0 && !done; hi -= 11) {
    const int lo = max(hi - 11, 0);
    const uint32_t wmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < kBins; i += kFinThreads) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (i < (int)n_mine && (e[i].x & kmask) == kpre) atomicAdd(&h[(e[i].x >> lo) & wmask], 1u);
    __syncthreads();
    find_bin_desc<kBins, kFinThreads>(h, need, tmp, res);
    const uint32_t bin = res[0];
    kpre |= bin << lo;
    kmask |= wmask << lo;
    need -= res[1];
    const uint32_t in_bin = h[bin];
    __syncthreads();  // h and res are read before the next round rewrites them
    if (in_bin <= 64u) {
#pragma unroll
      for (int i = 0; i < P; ++i)
        if (i < (int)n_mine && (e[i].x & kmask) == kpre) bin_list[atomicAdd(bin_cnt, 1u)] = e[i];
      __syncthreads();
      if (tid < 64) {
        const bool mine = tid < (int)in_bin;
        const uint2 b = mine ? bin_list[tid] : make_uint2(0u, 0u);
        uint32_t rank = 0;
        for (uint32_t m = 0; m < in_bin; ++m) {
          const uint32_t ox = (uint32_t)__builtin_amdgcn_readlane((int)b.x, (int)m);
          const uint32_t oy = (uint32_t)__builtin_amdgcn_readlane((int)b.y, (int)m);
          rank += (ox > b.x || (ox == b.x && oy < b.y)) ? 1u : 0u;
        }
        if (mine && rank == need - 1) { res[0] = b.x; res[1] = b.y; }
      }
      __syncthreads();
      T = res[0];
      I = res[1];
      done = true;
    }
  }
  if (!done) {
    // T = kpre; among keys equal to T the `need` lowest indices are taken.
    T = kpre;
    uint32_t n_eq_local = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) n_eq_local += (i < (int)n_mine && e[i].x == T) ? 1u : 0u;
    const uint32_t n_eq = block_incl_scan<kFinThreads>(n_eq_local, tmp);
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
#pragma unroll
        for (int i = 0; i < P; ++i)
          if (i < (int)n_mine && e[i].x == T && (e[i].y & imask) == ipre) atomicAdd(&h[(e[i].y >> lo) & wmask], 1u);
        __syncthreads();
        find_bin_asc<kBins, kFinThreads>(h, need, tmp, res);
        ipre |= res[0] << lo;
        imask |= wmask << lo;
        need -= res[1];
      }
      I = ipre;
    }
  }
  if (T < tau_max) return false;  // uniform: T is the same in every thread
  auto picked = [&](const uint2 x) { return x.x > T || (x.x == T && x.y <= I); };
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) mine += (i < (int)n_mine && picked(e[i])) ? 1u : 0u;
  uint32_t pos = block_incl_scan<kFinThreads>(mine, tmp) - mine;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    if (i < (int)n_mine && picked(e[i]) && pos < (uint32_t)k) out[pos++] = (int32_t)e[i].y;
  }
  return true;
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const float* __restrict__ scores, int64_t stride,
                                                                  const int32_t* __restrict__ lens, int64_t max_len,
                                                                  int32_t k, TopkWs ws, int32_t* __restrict__ out_idx,
                                                                  int32_t* __restrict__ status) {
  __shared__ uint32_t h[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t tmp[kFinThreads / 64];
  __shared__ uint32_t res[2];
  __shared__ uint32_t coff[kFinThreads];  // chunk offsets in the gathered candidate list
  __shared__ uint32_t s_mm[2];
  __shared__ uint32_t ovf;                 // some chunk had more candidates than its slice
  __shared__ uint32_t s_tmax;              // largest threshold a chunk collected with
  __shared__ uint2 bin_list[64];           // members of the boundary bin, when few
  __shared__ uint32_t bin_cnt;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The request's chunk metadata is requested before its length is known
  // (slots past its last chunk hold stale values and are not used).
  const int64_t slot0 = (int64_t)b * ws.chunks;
  const uint4 meta_raw = tid < ws.chunks ? ws.meta[slot0 + tid] : make_uint4(0u, 0xFFFFFFFFu, 0u, 0u);
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
  // should fewer than k have reached tau, more than a slice or LDS holds (or
  // the request have more chunks than this workgroup has threads), every key
  // of the request read from the scores.
  const int n_act = (int)((L + kTkChunk - 1) / kTkChunk);
  const uint4 meta = tid < n_act ? meta_raw : make_uint4(0u, 0xFFFFFFFFu, 0u, 0u);
  if (tid == 0) { s_mm[0] = 0xFFFFFFFFu; s_mm[1] = 0u; ovf = 0u; s_tmax = 0u; }
  const uint32_t c_incl = block_incl_scan<kFinThreads>(meta.x, tmp);  // barriers inside
  if (tid < n_act) coff[tid] = c_incl - meta.x;
  if (tid == kFinThreads - 1) res[0] = c_incl;
  {
    const uint32_t wmin = wave_min_u32(meta.y), wmax = wave_max_u32(meta.z);
    const uint32_t tmax = wave_max_u32(tid < n_act ? meta.y : 0u);
    if (lane == 0) { atomicMin(&s_mm[0], wmin); atomicMax(&s_mm[1], wmax); atomicMax(&s_tmax, tmax); }
    if (meta.x > (uint32_t)kTkSlice) ovf = 1u;
  }
  __syncthreads();
  const uint32_t n_cand = res[0];
  const bool whole = ovf != 0u || n_cand < (uint32_t)k || n_cand > (uint32_t)kCandLds || n_act > kFinThreads;
  const float* srow = scores + (int64_t)b * stride;
  if (!whole) {
    // Thread tid takes list positions [j0, j0 + per) straight into
    // registers: the chunk of j0 by binary search over the chunk offsets
    // (chunks without candidates share their offset with the next chunk, so
    // the last chunk c with coff[c] <= j is the one that holds j), then on
    // through the following chunks.
    // The register arrays are sized to the run (4, 8 or 16 entries): each
    // pass of the selection runs every entry slot in every lane, and a
    // workgroup of 16 waves runs four of them on each SIMD.
    const uint32_t per = (n_cand + kFinThreads - 1) / kFinThreads;  // <= kRegCand
    const uint32_t j0 = min(n_cand, tid * per), n_mine = min(n_cand, j0 + per) - j0;
    const uint32_t cmin = s_mm[0], cmax = s_mm[1], tau_max = s_tmax;
    auto gather_select = [&](auto p_tag) __attribute__((always_inline)) -> bool {
      constexpr int P = decltype(p_tag)::value;
      uint2 e[P];
      int c = 0;
      {
        int lo = 0, hi = n_act - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (coff[mid] <= j0) lo = mid; else hi = mid - 1;
        }
        c = lo;
      }
      uint32_t next = c + 1 < n_act ? coff[c + 1] : n_cand;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        if (i < (int)n_mine) {
          const uint32_t j = j0 + i;
          while (j >= next) {
            ++c;
            next = c + 1 < n_act ? coff[c + 1] : n_cand;
          }
          e[i] = ws.cand[(slot0 + c) * kTkSlice + (j - coff[c])];
        }
      }
#pragma unroll
      for (int i = 0; i < P; ++i)
        if (i < (int)n_mine) e[i].x = order_key(__uint_as_float(e[i].x));
      return select_regs<P>(e, n_mine, cmin, cmax, tau_max, k, out, h, tmp, res, bin_list, &bin_cnt);
    };
    const bool done = per <= 4   ? gather_select(std::integral_constant<int, 4>{})
                      : per <= 8 ? gather_select(std::integral_constant<int, 8>{})
                                 : gather_select(std::integral_constant<int, kRegCand>{});
    if (done) return;
    __syncthreads();
  }
  // The whole request, read from the scores.
  if (tid == 0) bin_cnt = 0u;
  __syncthreads();
  select_k_best(nullptr, srow, true, (uint32_t)L, 0u, 0u, 0u, k, out, h, tmp, res, bin_list, &bin_cnt);

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
  __shared__ __attribute__((aligned(16))) uint32_t tmp[kFinThreads / 64];
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
  if (!whole) {
    // Each thread takes its run of the packed list into registers.
    const uint32_t per = (n_cand + kFinThreads - 1) / kFinThreads;  // <= kRegCand
    const uint32_t j0 = min(n_cand, tid * per), n_mine = min(n_cand, j0 + per) - j0;
    auto load_select = [&](auto p_tag) __attribute__((always_inline)) -> bool {
      constexpr int P = decltype(p_tag)::value;  // sized to the run, as in the finish
      uint2 e[P];
#pragma unroll
      for (int i = 0; i < P; ++i)
        if (i < (int)n_mine) e[i] = lc[j0 + i];
      return select_regs<P>(e, n_mine, c_mm[0], c_mm[1], tau, k, out, h, tmp, res, bin_list, &bin_cnt);
    };
    const bool done = per <= 4   ? load_select(std::integral_constant<int, 4>{})
                      : per <= 8 ? load_select(std::integral_constant<int, 8>{})
                                 : load_select(std::integral_constant<int, kRegCand>{});
    if (done) return;
    __syncthreads();
    if (tid == 0) bin_cnt = 0u;
    __syncthreads();
  }
  select_k_best(lc, srow, true, (uint32_t)L, 0u, 0u, 0u, k, out, h, tmp, res, bin_list, &bin_cnt);
}

// ---- allocation-free form (topk_select_noalloc): the workspace is this
// file-scope device array, which every GPU the library runs on holds until
// the process ends.  Host code never passes the array's name to a kernel
// (on the host it only stands for the symbol); the device address is
// resolved once per device with hipGetSymbolAddress and kept.
static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

int topk_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return -3;
  if (dev < 0 || dev >= kMaxDevices) return -2;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -3;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

// Tags for the published thresholds: a process-wide counter started at a
// random value, so a stale word in a reused workspace (a previous call, or
// memory a previous process left behind) is unlikely to carry the current
// call's tag; when one does, the stale threshold can only cost speed (see
// the collect launch).
static uint32_t next_tag() {
  static std::atomic<uint32_t> counter{[] {
    std::random_device rd;
    return rd() ^ (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count();
  }()};
  return counter.fetch_add(1, std::memory_order_relaxed) + 1u;
}

int launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  if (a.k > kMaxK || a.k < 1) return -2;
  if (a.max_len <= kFusedMaxLen && reinterpret_cast<uintptr_t>(a.scores) % 16 == 0 && a.score_stride % 4 == 0) {
    hipLaunchKernelGGL(topk_fused_kernel, dim3((unsigned)a.batch), dim3(kFinThreads), 0, s, a.scores,
                       a.score_stride, a.lens, a.max_len, a.k, a.out_idx, a.status);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
  TopkWs ws = carve(a.workspace, a.batch, a.max_len, next_tag());
  const int64_t grid8 = (int64_t)((a.batch + 7) & ~7) * (ws.chunks + 1);
  if (grid8 > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)grid8), dim3(kTkThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.batch, a.max_len, a.k, ws);
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.batch), dim3(kFinThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws, a.out_idx, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
