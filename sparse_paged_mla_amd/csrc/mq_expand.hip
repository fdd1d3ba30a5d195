// mq_expand_requests kernel: the bookkeeping that lets a multi-query
// verification step (n_q new tokens per request, each attending causally)
// run through the single-query kernels.  Query i of request b becomes
// request v = b * n_q + i with the same block-table row and the length
// L_b - n_q + 1 + i (itself and every token before it); a request shorter
// than n_q gives its queries length -1, which every later call treats as a
// bad length.  One thread per (virtual request, block-table entry).
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kExpThreads = 256;

__global__ __launch_bounds__(kExpThreads) void mq_expand_kernel(const int32_t* __restrict__ bt, int32_t bt_stride,
                                                                const int32_t* __restrict__ lens, int32_t n_q,
                                                                int32_t chunks, int32_t* __restrict__ out_bt,
                                                                int32_t* __restrict__ out_lens) {
  const int v = blockIdx.x / chunks;
  const int b = v / n_q, i = v % n_q;
  const int64_t j = (int64_t)(blockIdx.x % chunks) * kExpThreads + threadIdx.x;
  if (j < bt_stride) out_bt[(int64_t)v * bt_stride + j] = bt[(int64_t)b * bt_stride + j];
  if (j == 0) {
    const int32_t L = lens[b];
    out_lens[v] = L >= n_q ? L - n_q + 1 + i : -1;
  }
}

int launch_mq_expand(const MqExpandArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  const int32_t chunks = (a.bt_stride + kExpThreads - 1) / kExpThreads;
  const int64_t grid = (int64_t)a.batch * a.n_q * chunks;
  if (grid > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL(mq_expand_kernel, dim3((unsigned)grid), dim3(kExpThreads), 0, s, a.bt, a.bt_stride, a.lens,
                     a.n_q, chunks, a.out_bt, a.out_lens);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
