// lse_merge kernel: combine per-split (o, lse) partials of the same query into
// the result over the union of the splits (exact online-softmax algebra).
// One wave per (request, head) row: every lane reads the row's num_splits
// lse values, forms the weights exp(lse_s - lse), and streams float4 slices of
// the d-dim partials.  HBM-bound; the partial traffic is the whole cost, so
// the partials (read once) and the result (written once) go through
// non-temporal loads and stores.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kMergeThreads = 256;
constexpr int kMaxSplits = 64;

// SP > 0: exactly SP splits and d == 512, with each lane's partial slices
// loaded before (and so overlapping) the wait for the split lse values;
// SP == 0: any split count and d.
template <int SP>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const float* __restrict__ o_part,
                                                                  const float* __restrict__ lse_part, int32_t batch,
                                                                  int32_t splits, int32_t n_heads, int32_t d,
                                                                  float* __restrict__ o, float* __restrict__ lse) {
  __shared__ float wsh[kMergeThreads / 64][kMaxSplits];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * (kMergeThreads / 64) + wid;
  if (row >= (int64_t)batch * n_heads) return;
  const int64_t b = row / n_heads, h = row % n_heads;
  if constexpr (SP > 0) {
    splits = SP;
    d = 512;
  }
  // Partial slices of this lane (SP > 0): dims 4*lane + 256*i of split sp.
  f32x4 pv[SP > 0 ? SP : 1][2];
  if constexpr (SP > 0) {
#pragma unroll
    for (int sp = 0; sp < SP; ++sp)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        pv[sp][i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(o_part + ((b * SP + sp) * n_heads + h) * 512 + lane * 4 + 256 * i));
  }
  // Lane s < splits holds lse of split s.
  float my = -INFINITY;
  bool nan_seen = false;
  if (lane < splits) {
    my = lse_part[(b * splits + lane) * n_heads + h];
    nan_seen = my != my;
  }
  const bool any_nan = __any(nan_seen);
  float M = my;
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float* orow = o + row * d;
  const float kNaN = __uint_as_float(0x7FC00000u);
  if (any_nan || M == -INFINITY) {
    const float fill = any_nan ? kNaN : 0.f;
    for (int i = lane * 4; i < d; i += 256) *reinterpret_cast<float4*>(orow + i) = make_float4(fill, fill, fill, fill);
    if (lane == 0) lse[row] = any_nan ? kNaN : -INFINITY;
    return;
  }
  float e = (lane < splits && my > -INFINITY) ? expf(my - M) : 0.f;
  float sum = e;
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float L = M + logf(sum);
  wsh[wid][lane] = e / sum;  // = exp(lse_s - L); the wave's own slots only
  __builtin_amdgcn_wave_barrier();
  if constexpr (SP > 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < SP; ++sp) {
        const float ws = wsh[wid][sp];
        if (ws == 0.f) continue;  // an empty split: its partial (perhaps never written) is not used
        acc += ws * pv[sp][i];
      }
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(orow + lane * 4 + 256 * i));
    }
  } else {
    for (int i = lane * 4; i < d; i += 256) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int sp = 0; sp < splits; ++sp) {
        const float ws = wsh[wid][sp];
        if (ws == 0.f) continue;
        const float4 v = *reinterpret_cast<const float4*>(o_part + ((b * splits + sp) * n_heads + h) * d + i);
        acc.x += ws * v.x; acc.y += ws * v.y; acc.z += ws * v.z; acc.w += ws * v.w;
      }
      *reinterpret_cast<float4*>(orow + i) = acc;
    }
  }
  if (lane == 0) lse[row] = L;
}

int launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.n_heads;
  if (rows == 0) return 0;
  if (a.num_splits > kMaxSplits) return -2;
  const int64_t grid = (rows + (kMergeThreads / 64) - 1) / (kMergeThreads / 64);
  if (grid > 0x7FFFFFFF) return -2;
#define SPMLA_MERGE(SPN)                                                                                       \
  hipLaunchKernelGGL(lse_merge_kernel<SPN>, dim3((unsigned)grid), dim3(kMergeThreads), 0, s, a.o_part, a.lse_part, \
                     a.batch, a.num_splits, a.n_heads, a.d, a.o, a.lse)
  if (a.d == 512 && a.num_splits == 2) SPMLA_MERGE(2);
  else if (a.d == 512 && a.num_splits == 4) SPMLA_MERGE(4);
  else if (a.d == 512 && a.num_splits == 8) SPMLA_MERGE(8);
  else SPMLA_MERGE(0);
#undef SPMLA_MERGE
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
