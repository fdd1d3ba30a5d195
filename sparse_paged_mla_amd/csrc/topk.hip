// topk_select kernels: exact per-request Top-k by radix selection on an
// order-preserving 32-bit key, with ties broken toward the lower token index.
//
// Key: NaN -> 0 (below everything), -0.0 -> +0.0, then the usual sign-flip so
// that unsigned order equals numeric order.  The selection is the k_eff best
// entries under (key desc, index asc), a total order, so the result is unique
// and does not depend on the order atomics land in.
//
// Launches per call (all on the caller's stream):
//  1. clear:  zero the per-request histogram and counters in the workspace.
//  2. hist:   (request, chunk) workgroups histogram the top 11 key bits in LDS
//             and add them into the request's global histogram.
//  3. filter: every workgroup finds the bin b0 holding the k-th best key (a
//             block scan of the 2048 bins), then streams its chunk again:
//             keys in bins above b0 are selected outright (their index goes to
//             the output row at an atomically reserved slot), keys in b0 go to
//             a candidate list.  Atomics are aggregated per wave with ballot +
//             mbcnt.
//  4. finish: one workgroup per request resolves the candidates: two more
//             histogram rounds over the low 21 key bits find the exact
//             threshold key T; keys above T are taken, and among keys equal to
//             T the lowest indices are taken (a radix select on the index when
//             there are more ties than places).  The k_eff indices are then
//             sorted ascending in LDS (bitonic) and written with -1 padding.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace spmla {

constexpr int kTkThreads = 256;
constexpr int kTkChunk = 4096;       // tokens per hist/filter workgroup
constexpr int kBins0 = 2048;         // top 11 key bits
constexpr int kFinThreads = 512;
constexpr int kMaxK = 4096;
constexpr int kCtrlWords = 8;        // out_count, cand_count, pad

struct TopkWs {
  uint32_t* hist;   // [B, 2048]
  uint32_t* ctrl;   // [B, 8]
  uint2* cand;      // [B, cap] (key, index)
  int64_t cap;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t topk_workspace_size(int32_t batch, int64_t max_len, int32_t k) {
  (void)k;
  if (batch <= 0 || max_len < 0) return 0;
  size_t hist = align_up((size_t)batch * kBins0 * 4, 256);
  size_t ctrl = align_up((size_t)batch * kCtrlWords * 4, 256);
  size_t cand = align_up((size_t)batch * (size_t)(max_len > 0 ? max_len : 1) * 8, 256);
  return hist + ctrl + cand;
}

static TopkWs carve(void* ws, int32_t batch, int64_t max_len) {
  TopkWs w;
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kBins0 * 4, 256);
  w.ctrl = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)batch * kCtrlWords * 4, 256);
  w.cand = reinterpret_cast<uint2*>(p);
  w.cap = max_len > 0 ? max_len : 1;
  return w;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN ranks lowest
  if (u == 0x80000000u) u = 0u;                     // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool len_ok(int32_t L, int64_t max_len) { return L >= 0 && (int64_t)L <= max_len; }

__global__ void topk_clear_kernel(uint32_t* __restrict__ hist, uint32_t* __restrict__ ctrl, int64_t n_hist,
                                  int64_t n_ctrl) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_hist; i += stride) hist[i] = 0u;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_ctrl; i += stride) ctrl[i] = 0u;
}

__global__ __launch_bounds__(kTkThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t stride,
                                                               const int32_t* __restrict__ lens, int64_t max_len,
                                                               int32_t k, uint32_t* __restrict__ ghist,
                                                               int32_t chunks_per_req) {
  __shared__ uint32_t h[kBins0];
  const int b = blockIdx.x / chunks_per_req;
  const int chunk = blockIdx.x % chunks_per_req;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int64_t t0 = (int64_t)chunk * kTkChunk;
  if (t0 >= L) return;
  const int64_t t1 = min((int64_t)L, t0 + kTkChunk);
  for (int i = threadIdx.x; i < kBins0; i += kTkThreads) h[i] = 0u;
  __syncthreads();
  const float* s = scores + (int64_t)b * stride;
  for (int64_t t = t0 + threadIdx.x; t < t1; t += kTkThreads) atomicAdd(&h[order_key(s[t]) >> 21], 1u);
  __syncthreads();
  uint32_t* gh = ghist + (int64_t)b * kBins0;
  for (int i = threadIdx.x; i < kBins0; i += kTkThreads) {
    const uint32_t c = h[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// Block-wide search over a histogram in LDS, from the top bin down: returns the
// bin x with sum_{y > x} h[y] < need <= sum_{y >= x} h[y], and that "above"
// count.  NB must be a multiple of the block size; `red` is scratch of
// blockDim.x words; `out` two words.  need >= 1 and <= total is required.
template <int NB, int NT>
__device__ void find_bin_desc(const uint32_t* h, uint32_t need, uint32_t* red, uint32_t* out) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  if (tid == 0) { out[0] = 0u; out[1] = 0u; }
  // Thread tid owns bins [NB - (tid+1)*PER, NB - tid*PER): thread 0 owns the top.
  const int hi = NB - tid * PER;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 1; j <= PER; ++j) mine += h[hi - j];
  red[tid] = mine;
  __syncthreads();
  // Inclusive scan over threads (Hillis-Steele in LDS).
  for (int off = 1; off < NT; off <<= 1) {
    uint32_t v = tid >= off ? red[tid - off] : 0u;
    __syncthreads();
    red[tid] += v;
    __syncthreads();
  }
  const uint32_t incl = red[tid];
  const uint32_t excl = incl - mine;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
    for (int j = 1; j <= PER; ++j) {
      const uint32_t c = h[hi - j];
      if (run + c >= need) {
        out[0] = (uint32_t)(hi - j);
        out[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

// Same, from the lowest bin up (used to take the smallest indices).
template <int NB, int NT>
__device__ void find_bin_asc(const uint32_t* h, uint32_t need, uint32_t* red, uint32_t* out) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  if (tid == 0) { out[0] = 0u; out[1] = 0u; }
  const int lo = tid * PER;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) mine += h[lo + j];
  red[tid] = mine;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    uint32_t v = tid >= off ? red[tid - off] : 0u;
    __syncthreads();
    red[tid] += v;
    __syncthreads();
  }
  const uint32_t incl = red[tid];
  const uint32_t excl = incl - mine;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
    for (int j = 0; j < PER; ++j) {
      const uint32_t c = h[lo + j];
      if (run + c >= need) {
        out[0] = (uint32_t)(lo + j);
        out[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

// Wave-aggregated append: lanes with `pred` get consecutive slots starting at
// a base reserved with one atomic per wave.  Returns the lane's slot.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0u;
  const uint32_t lane_rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  const int leader = __ffsll((long long)mask) - 1;
  uint32_t base = 0;
  if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __shfl(base, leader);
  return base + lane_rank;
}

__global__ __launch_bounds__(kTkThreads) void topk_filter_kernel(
    const float* __restrict__ scores, int64_t stride, const int32_t* __restrict__ lens, int64_t max_len, int32_t k,
    const uint32_t* __restrict__ ghist, uint32_t* __restrict__ ctrl, uint2* __restrict__ cand, int64_t cap,
    int32_t* __restrict__ out_idx, int32_t chunks_per_req) {
  __shared__ uint32_t h[kBins0];
  __shared__ uint32_t red[kTkThreads];
  __shared__ uint32_t res[2];
  const int b = blockIdx.x / chunks_per_req;
  const int chunk = blockIdx.x % chunks_per_req;
  const int32_t L = lens[b];
  if (!len_ok(L, max_len) || L <= k) return;
  const int64_t t0 = (int64_t)chunk * kTkChunk;
  if (t0 >= L) return;
  const int64_t t1 = min((int64_t)L, t0 + kTkChunk);
  const uint32_t* gh = ghist + (int64_t)b * kBins0;
  for (int i = threadIdx.x; i < kBins0; i += kTkThreads) h[i] = gh[i];
  __syncthreads();
  find_bin_desc<kBins0, kTkThreads>(h, (uint32_t)k, red, res);
  const uint32_t b0 = res[0];
  const float* s = scores + (int64_t)b * stride;
  uint32_t* c = ctrl + (int64_t)b * kCtrlWords;
  int32_t* out = out_idx + (int64_t)b * k;
  uint2* cb = cand + (int64_t)b * cap;
  // Every lane runs the same trip count so the wave-wide ballots stay uniform.
  for (int64_t base = t0; base < t1; base += kTkThreads) {
    const int64_t t = base + threadIdx.x;
    const bool in = t < t1;
    const uint32_t key = in ? order_key(s[t]) : 0u;
    const uint32_t bin = key >> 21;
    const bool sel = in && bin > b0;
    const bool cnd = in && bin == b0;
    const uint32_t ps = wave_append(sel, c + 0);
    if (sel) out[ps] = (int32_t)t;
    const uint32_t pc = wave_append(cnd, c + 1);
    if (cnd) cb[pc] = make_uint2(key, (uint32_t)t);
  }
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(const int32_t* __restrict__ lens, int64_t max_len,
                                                                  int32_t k, const uint32_t* __restrict__ ghist,
                                                                  const uint32_t* __restrict__ ctrl,
                                                                  const uint2* __restrict__ cand, int64_t cap,
                                                                  int32_t* __restrict__ out_idx,
                                                                  int32_t* __restrict__ status) {
  __shared__ uint32_t h[kBins0];
  __shared__ uint32_t red[kFinThreads];
  __shared__ uint32_t res[2];
  __shared__ uint32_t cnt;
  __shared__ int32_t sorted[kMaxK];
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
  // Threshold bin of the top 11 bits (as the filter pass found it).
  const uint32_t* gh = ghist + (int64_t)b * kBins0;
  for (int i = tid; i < kBins0; i += kFinThreads) h[i] = gh[i];
  __syncthreads();
  find_bin_desc<kBins0, kFinThreads>(h, (uint32_t)k, red, res);
  const uint32_t b0 = res[0];
  const uint32_t n_gt = ctrl[(int64_t)b * kCtrlWords + 0];
  const uint32_t n_c = ctrl[(int64_t)b * kCtrlWords + 1];
  const uint2* cb = cand + (int64_t)b * cap;
  uint32_t need = (uint32_t)k - n_gt;  // >= 1 places left for keys in bin b0

  // Round 1: key bits 20..10 among the candidates.
  for (int i = tid; i < kBins0; i += kFinThreads) h[i] = 0u;
  __syncthreads();
  for (uint32_t j = tid; j < n_c; j += kFinThreads) atomicAdd(&h[(cb[j].x >> 10) & 0x7FFu], 1u);
  __syncthreads();
  find_bin_desc<kBins0, kFinThreads>(h, need, red, res);
  const uint32_t d1 = res[0];
  need -= res[1];
  // Round 2: key bits 9..0 among candidates in bin d1.
  for (int i = tid; i < kBins0; i += kFinThreads) h[i] = 0u;
  __syncthreads();
  for (uint32_t j = tid; j < n_c; j += kFinThreads) {
    const uint32_t key = cb[j].x;
    if (((key >> 10) & 0x7FFu) == d1) atomicAdd(&h[key & 0x3FFu], 1u);
  }
  __syncthreads();
  find_bin_desc<1024, kFinThreads>(h, need, red, res);
  const uint32_t d2 = res[0];
  need -= res[1];
  const uint32_t T = (b0 << 21) | (d1 << 10) | d2;
  const uint32_t n_eq = h[d2];
  __syncthreads();

  // Among keys equal to T take the `need` lowest indices: find the index
  // threshold I (inclusive) by a 3-round radix select from the low end.
  uint32_t I = 0xFFFFFFFFu;
  if (n_eq > need) {
    uint32_t prefix = 0, pmask = 0;
    const int shifts[3] = {22, 11, 0};
    const uint32_t widths[3] = {0x1FFu, 0x7FFu, 0x7FFu};
    uint32_t need_i = need;
    for (int r = 0; r < 3; ++r) {
      for (int i = tid; i < kBins0; i += kFinThreads) h[i] = 0u;
      __syncthreads();
      for (uint32_t j = tid; j < n_c; j += kFinThreads) {
        const uint2 e = cb[j];
        if (e.x == T && (e.y & pmask) == prefix) atomicAdd(&h[(e.y >> shifts[r]) & widths[r]], 1u);
      }
      __syncthreads();
      find_bin_asc<kBins0, kFinThreads>(h, need_i, red, res);
      prefix |= res[0] << shifts[r];
      pmask |= widths[r] << shifts[r];
      need_i -= res[1];
    }
    I = prefix;
  }

  // Gather: the n_gt indices already in the output row, plus the resolved candidates.
  if (tid == 0) cnt = n_gt;
  for (uint32_t j = tid; j < n_gt; j += kFinThreads) sorted[j] = out[j];
  __syncthreads();
  for (uint32_t j = tid; j < n_c; j += kFinThreads) {
    const uint2 e = cb[j];
    if (e.x > T || (e.x == T && e.y <= I)) {
      const uint32_t p = atomicAdd(&cnt, 1u);
      if (p < (uint32_t)k) sorted[p] = (int32_t)e.y;
    }
  }
  __syncthreads();
  // Bitonic sort of the k entries (padded to a power of two with INT_MAX).
  int n2 = 1;
  while (n2 < k) n2 <<= 1;
  for (int j = k + tid; j < n2; j += kFinThreads) sorted[j] = 0x7FFFFFFF;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kFinThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t a = sorted[lo], c2 = sorted[hi];
        if ((a > c2) == up) {
          sorted[lo] = c2;
          sorted[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < k; j += kFinThreads) out[j] = sorted[j] == 0x7FFFFFFF ? -1 : sorted[j];
}

int launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  if (a.k > kMaxK || a.k < 1) return -2;
  TopkWs ws = carve(a.workspace, a.batch, a.max_len);
  const int64_t n_hist = (int64_t)a.batch * kBins0, n_ctrl = (int64_t)a.batch * kCtrlWords;
  hipLaunchKernelGGL(topk_clear_kernel, dim3((unsigned)std::min<int64_t>(1024, (n_hist + 255) / 256)), dim3(256), 0, s,
                     ws.hist, ws.ctrl, n_hist, n_ctrl);
  const int64_t chunks = a.max_len > 0 ? (a.max_len + kTkChunk - 1) / kTkChunk : 1;
  const int64_t grid = (int64_t)a.batch * chunks;
  if (grid > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)grid), dim3(kTkThreads), 0, s, a.scores, a.score_stride, a.lens,
                     a.max_len, a.k, ws.hist, (int32_t)chunks);
  hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)grid), dim3(kTkThreads), 0, s, a.scores, a.score_stride,
                     a.lens, a.max_len, a.k, ws.hist, ws.ctrl, ws.cand, ws.cap, a.out_idx, (int32_t)chunks);
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.batch), dim3(kFinThreads), 0, s, a.lens, a.max_len, a.k,
                     ws.hist, ws.ctrl, ws.cand, ws.cap, a.out_idx, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
