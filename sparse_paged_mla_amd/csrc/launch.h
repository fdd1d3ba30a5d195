// Internal launcher declarations (host side).  Arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spmla {

struct IndexerArgs {
  const void* q_idx; int q_dtype; const float* w;
  const void* k_pool; const float* k_scale; int k_dtype;
  int32_t num_pages, page_size; const int32_t* bt; int32_t bt_stride;
  const int32_t* lens; int32_t batch; int64_t max_len; int32_t n_heads, d;
  float* scores; int64_t score_stride; int32_t* status;
  int32_t n_q = 1;  // queries per request scored per key read (1 or 2)
};
// Returns 0 on success, -2 unsupported combination, -3 launch failure.
int launch_indexer(const IndexerArgs& a, hipStream_t stream);

struct TopkArgs {
  const float* scores; int64_t score_stride; const int32_t* lens; int32_t batch; int64_t max_len;
  int32_t k; int32_t* out_idx; void* workspace; int32_t* status;
};
int launch_topk(const TopkArgs& a, hipStream_t stream);
// Device address of the static top-k workspace on the current device
// (resolved on the first call per device); 0, or -2 / -3 on failure.
int topk_scratch(void** ptr);

struct DecodeArgs {
  const void* q; int q_dtype; const void* kv; const float* kv_scale; int kv_dtype;
  int32_t num_pages, page_size; const int32_t* bt; int32_t bt_stride;
  const int32_t* lens; int32_t batch; int64_t max_len; const int32_t* indices; int32_t k;
  int32_t n_heads, d_latent, d_rope; float sm_scale; int32_t num_splits;
  int32_t split_tokens;  // 0: ceil(n / num_splits) rounded up to 32; else the fixed split length
  float* o_part; float* lse_part; int32_t* status;
};
int launch_decode(const DecodeArgs& a, hipStream_t stream);
// FP8 cache, bf16 query, 512 + 64 dims (mla_decode_f8.hip).
int launch_decode_f8(const DecodeArgs& a, hipStream_t stream);
// bf16 cache, bf16 query, 512 + 64 dims (mla_decode_bf16.hip).
int launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// Other shapes (mla_decode_generic.hip): latent and rope widths multiples of
// 8, latent >= 8, latent + rope <= kDecodeGenericMaxDim; fp32 or bf16
// queries; fp32, bf16 or FP8 caches, except bf16 queries over fp32 caches.
constexpr int kDecodeGenericMaxDim = 1024;
inline bool decode_generic_shape(int q_dtype, int kv_dtype, int d_latent, int d_rope) {
  constexpr int f32 = 0, bf16 = 1, fp8 = 2;  // the C ABI's dtype codes
  if (d_latent < 8 || d_latent % 8 != 0 || d_rope < 0 || d_rope % 8 != 0) return false;
  if (d_latent + d_rope > kDecodeGenericMaxDim) return false;
  if (q_dtype != f32 && q_dtype != bf16) return false;
  if (kv_dtype != f32 && kv_dtype != bf16 && kv_dtype != fp8) return false;
  return !(q_dtype == bf16 && kv_dtype == f32);
}
int launch_decode_generic(const DecodeArgs& a, hipStream_t stream);

struct MergeArgs {
  const float* o_part; const float* lse_part; int32_t batch, num_splits, n_heads, d; float* o; float* lse;
};
int launch_merge(const MergeArgs& a, hipStream_t stream);

struct AppendArgs {
  const void* rows; int row_dtype; int32_t batch, dim; void* pool; float* pool_scale; int pool_dtype;
  int32_t num_pages, page_size; const int32_t* bt; int32_t bt_stride; const int32_t* positions; int32_t* status;
  // A second pool with the same page ids, row and pool types (rows2 == nullptr: none).
  const void* rows2 = nullptr; int32_t dim2 = 0; void* pool2 = nullptr; float* pool_scale2 = nullptr;
};
int launch_cache_append(const AppendArgs& a, hipStream_t stream);

struct PageCheckArgs {
  const int32_t* bt; const uint64_t* bt_tags; int32_t bt_stride; const int32_t* lens; int32_t batch;
  int64_t max_len; const uint64_t* page_tags; int32_t num_pages, page_size; int32_t* status;
};
int launch_page_check(const PageCheckArgs& a, hipStream_t stream);

struct MqExpandArgs {
  const int32_t* bt; int32_t bt_stride; const int32_t* lens; int32_t batch, n_q; int32_t* out_bt; int32_t* out_lens;
};
int launch_mq_expand(const MqExpandArgs& a, hipStream_t stream);

}  // namespace spmla
