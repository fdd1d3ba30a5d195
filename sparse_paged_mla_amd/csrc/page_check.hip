// kv_page_check kernel: the batched integrity check of every request's page
// mapping, run before the cache is read.  Each physical page carries a tag
// that changes on every reallocation; each block-table entry carries the tag
// its page had when it was given to the request.  A request whose length
// covers an entry with a bad page id or a stale tag is flagged, so that the
// caller can drop it instead of serving another request's data.
//
// One thread per block-table entry that some request's length covers: the
// entry, its recorded tag and the page's current tag are three loads (the
// last gathered through the first), and only a mismatch touches the status
// word.  The check reads a few bytes per page of context: its time is the
// launch and two dependent memory round trips.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace spmla {

constexpr int kChkThreads = 256;

__global__ __launch_bounds__(kChkThreads) void page_check_kernel(
    const int32_t* __restrict__ bt, const uint64_t* __restrict__ bt_tags, int32_t bt_stride,
    const int32_t* __restrict__ lens, int64_t max_len, const uint64_t* __restrict__ page_tags, int32_t num_pages,
    int32_t page_shift, int32_t chunks, int32_t* __restrict__ status) {
  const int b = blockIdx.x / chunks;
  const int64_t j = (int64_t)(blockIdx.x % chunks) * kChkThreads + threadIdx.x;
  const int32_t L = lens[b];
  const int64_t cap = (int64_t)bt_stride << page_shift;
  if (L < 0 || (int64_t)L > max_len || (int64_t)L > cap) {
    if (j == 0) atomicOr(status + b, kBadLen);
    return;
  }
  const int64_t pages = ((int64_t)L + (1 << page_shift) - 1) >> page_shift;
  if (j >= pages) return;
  const int64_t e = (int64_t)b * bt_stride + j;
  const int32_t page = bt[e];
  const uint64_t want = bt_tags[e];
  if (page < 0 || page >= num_pages) {
    atomicOr(status + b, kBadPage);
    return;
  }
  if (page_tags[page] != want) atomicOr(status + b, kBadTag);
}

int launch_page_check(const PageCheckArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  // Entries a valid length can cover: at most min(bt_stride, pages of max_len).
  const int64_t max_pages =
      std::min<int64_t>(a.bt_stride, (a.max_len + a.page_size - 1) >> page_shift);
  const int32_t chunks = (int32_t)std::max<int64_t>(1, (max_pages + kChkThreads - 1) / kChkThreads);
  const int64_t grid = (int64_t)a.batch * chunks;
  if (grid > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL(page_check_kernel, dim3((unsigned)grid), dim3(kChkThreads), 0, s, a.bt, a.bt_tags, a.bt_stride,
                     a.lens, a.max_len, a.page_tags, a.num_pages, page_shift, chunks, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
