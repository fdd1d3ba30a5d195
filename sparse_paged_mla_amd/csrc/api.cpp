// C-ABI entry points of libsparse_mla.so: host-side validation, then launch.
// Validation touches no device memory and makes no HIP call, so a rejected
// call never enqueues anything.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/sparse_mla.h"
#include "launch.h"
#include "topk_layout.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SPMLA_OK;
}

bool is_pow2_page(int32_t p) { return p == 16 || p == 32 || p == 64 || p == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int map_launch(int rc, const char* what) {
  if (rc == 0) return ok();
  if (rc == -2) return fail(SPMLA_EUNSUPPORTED, "%s: unsupported dtype/shape combination", what);
  return fail(SPMLA_ELAUNCH, "%s: kernel launch failed (%s)", what, hipGetErrorString(hipGetLastError()));
}

int check_paging(const char* what, int32_t num_pages, int32_t page_size, const int32_t* bt, int32_t bt_stride,
                 const int32_t* lens, int32_t batch, int64_t max_len) {
  if (batch < 0) return fail(SPMLA_EINVAL, "%s: batch < 0", what);
  if (num_pages < 1) return fail(SPMLA_EINVAL, "%s: num_pages must be >= 1", what);
  if (!is_pow2_page(page_size)) return fail(SPMLA_EUNSUPPORTED, "%s: page_size must be 16, 32, 64 or 128", what);
  if (bt_stride < 1) return fail(SPMLA_EINVAL, "%s: bt_stride must be >= 1", what);
  if (max_len < 0 || max_len >= (int64_t)1 << 31) return fail(SPMLA_EINVAL, "%s: max_len out of [0, 2^31)", what);
  if (batch > 0 && (!bt || !lens)) return fail(SPMLA_EINVAL, "%s: null block_table or context_lens", what);
  return SPMLA_OK;
}

}  // namespace

extern "C" {

const char* spmla_last_error(void) { return g_err; }

int dsa_indexer_scores(const void* q_idx, int32_t q_dtype, const float* weights, const void* k_pool,
                       const float* k_scale, int32_t k_dtype, int32_t num_pages, int32_t page_size,
                       const int32_t* block_table, int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                       int64_t max_len, int32_t n_heads, int32_t d, float* scores, int64_t score_stride,
                       int32_t* req_status, void* stream) {
  const char* w = "dsa_indexer_scores";
  if (int rc = check_paging(w, num_pages, page_size, block_table, bt_stride, context_lens, batch, max_len)) return rc;
  if (q_dtype != SPMLA_F32 && q_dtype != SPMLA_BF16) return fail(SPMLA_EUNSUPPORTED, "%s: q_dtype must be F32 or BF16", w);
  if (k_dtype < SPMLA_F32 || k_dtype > SPMLA_FP8_E4M3) return fail(SPMLA_EINVAL, "%s: bad k_dtype", w);
  if (q_dtype == SPMLA_BF16 && k_dtype == SPMLA_F32)
    return fail(SPMLA_EUNSUPPORTED, "%s: bf16 queries need bf16 or FP8 keys", w);
  if (n_heads < 1 || n_heads > 128) return fail(SPMLA_EUNSUPPORTED, "%s: n_heads must be in [1, 128]", w);
  if (!(d == 16 || d == 32 || d == 64 || d == 128 || d == 256) || (q_dtype == SPMLA_BF16 && d < 32))
    return fail(SPMLA_EUNSUPPORTED, "%s: d must be 16/32/64/128/256 (>= 32 with bf16)", w);
  if (score_stride < max_len) return fail(SPMLA_EINVAL, "%s: score_stride < max_len", w);
  if (batch > 0) {
    if (!q_idx || !weights || !k_pool || !scores) return fail(SPMLA_EINVAL, "%s: null pointer", w);
    if (k_dtype == SPMLA_FP8_E4M3 && !k_scale) return fail(SPMLA_EINVAL, "%s: FP8 keys need k_scale", w);
    if (!aligned16(q_idx) || !aligned16(k_pool)) return fail(SPMLA_EINVAL, "%s: q_idx and k_pool must be 16-byte aligned", w);
    if (score_stride % 4 != 0 || !aligned16(scores))
      return fail(SPMLA_EINVAL, "%s: score rows must be 16-byte aligned (scores aligned, score_stride % 4 == 0)", w);
  }
  spmla::IndexerArgs a{q_idx, q_dtype, weights, k_pool, k_scale, k_dtype, num_pages, page_size, block_table,
                       bt_stride, context_lens, batch, max_len, n_heads, d, scores, score_stride, req_status};
  return map_launch(spmla::launch_indexer(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int dsa_indexer_scores_mq(const void* q_idx, int32_t q_dtype, const float* weights, const void* k_pool,
                          const float* k_scale, int32_t k_dtype, int32_t num_pages, int32_t page_size,
                          const int32_t* block_table, int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                          int64_t max_len, int32_t n_q, int32_t n_heads, int32_t d, float* scores,
                          int64_t score_stride, int32_t* req_status, void* stream) {
  const char* w = "dsa_indexer_scores_mq";
  if (n_q < 1 || n_q > 2) return fail(SPMLA_EUNSUPPORTED, "%s: n_q must be 1 or 2", w);
  if (n_q == 2 && ((n_heads != 16 && n_heads != 32 && n_heads != 64) || q_dtype != SPMLA_BF16))
    return fail(SPMLA_EUNSUPPORTED, "%s: two queries need bf16 queries and n_heads of 16, 32 or 64", w);
  if (int rc = check_paging(w, num_pages, page_size, block_table, bt_stride, context_lens, batch, max_len)) return rc;
  if (q_dtype != SPMLA_F32 && q_dtype != SPMLA_BF16) return fail(SPMLA_EUNSUPPORTED, "%s: q_dtype must be F32 or BF16", w);
  if (k_dtype < SPMLA_F32 || k_dtype > SPMLA_FP8_E4M3) return fail(SPMLA_EINVAL, "%s: bad k_dtype", w);
  if (q_dtype == SPMLA_BF16 && k_dtype == SPMLA_F32)
    return fail(SPMLA_EUNSUPPORTED, "%s: bf16 queries need bf16 or FP8 keys", w);
  if (n_heads < 1 || n_heads > 128) return fail(SPMLA_EUNSUPPORTED, "%s: n_heads must be in [1, 128]", w);
  if (!(d == 16 || d == 32 || d == 64 || d == 128 || d == 256) || (q_dtype == SPMLA_BF16 && d < 32))
    return fail(SPMLA_EUNSUPPORTED, "%s: d must be 16/32/64/128/256 (>= 32 with bf16)", w);
  if (score_stride < max_len) return fail(SPMLA_EINVAL, "%s: score_stride < max_len", w);
  if (batch > 0) {
    if (!q_idx || !weights || !k_pool || !scores) return fail(SPMLA_EINVAL, "%s: null pointer", w);
    if (k_dtype == SPMLA_FP8_E4M3 && !k_scale) return fail(SPMLA_EINVAL, "%s: FP8 keys need k_scale", w);
    if (!aligned16(q_idx) || !aligned16(k_pool)) return fail(SPMLA_EINVAL, "%s: q_idx and k_pool must be 16-byte aligned", w);
    if (score_stride % 4 != 0 || !aligned16(scores))
      return fail(SPMLA_EINVAL, "%s: score rows must be 16-byte aligned (scores aligned, score_stride % 4 == 0)", w);
  }
  spmla::IndexerArgs a{q_idx, q_dtype, weights, k_pool, k_scale, k_dtype, num_pages, page_size, block_table,
                       bt_stride, context_lens, batch, max_len, n_heads, d, scores, score_stride, req_status, n_q};
  return map_launch(spmla::launch_indexer(a, reinterpret_cast<hipStream_t>(stream)), w);
}

size_t topk_workspace_bytes(int32_t batch, int64_t max_len, int32_t k) {
  if (batch < 0 || max_len < 0 || max_len >= (int64_t)1 << 31 || k < 1 || k > 4096) return 0;
  return spmla::topk_workspace_size(batch, max_len, k);
}

int topk_select(const float* scores, int64_t score_stride, const int32_t* context_lens, int32_t batch,
                int64_t max_len, int32_t k, int32_t* out_idx, void* workspace, size_t workspace_bytes,
                int32_t* req_status, void* stream) {
  const char* w = "topk_select";
  if (batch < 0) return fail(SPMLA_EINVAL, "%s: batch < 0", w);
  if (k < 1 || k > 4096) return fail(SPMLA_EUNSUPPORTED, "%s: k must be in [1, 4096]", w);
  if (max_len < 0 || max_len >= (int64_t)1 << 31) return fail(SPMLA_EINVAL, "%s: max_len out of [0, 2^31)", w);
  if (score_stride < max_len) return fail(SPMLA_EINVAL, "%s: score_stride < max_len", w);
  if (batch == 0) return ok();
  if (!scores || !context_lens || !out_idx) return fail(SPMLA_EINVAL, "%s: null pointer", w);
  const size_t need = spmla::topk_workspace_size(batch, max_len, k);
  if (!workspace || workspace_bytes < need)
    return fail(SPMLA_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", w, need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(SPMLA_EINVAL, "%s: workspace must be 256-byte aligned", w);
  spmla::TopkArgs a{scores, score_stride, context_lens, batch, max_len, k, out_idx, workspace, req_status};
  return map_launch(spmla::launch_topk(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int topk_select_noalloc(const float* scores, int64_t score_stride, const int32_t* context_lens, int32_t batch,
                        int64_t max_len, int32_t k, int32_t* out_idx, int32_t* req_status, void* stream) {
  const char* w = "topk_select_noalloc";
  static_assert(SPMLA_TOPK_SCRATCH_BYTES == spmla::kTopkScratchBytes, "header and library agree on the scratch size");
  if (batch < 0) return fail(SPMLA_EINVAL, "%s: batch < 0", w);
  if (k < 1 || k > 4096) return fail(SPMLA_EUNSUPPORTED, "%s: k must be in [1, 4096]", w);
  if (max_len < 0 || max_len >= (int64_t)1 << 31) return fail(SPMLA_EINVAL, "%s: max_len out of [0, 2^31)", w);
  if (score_stride < max_len) return fail(SPMLA_EINVAL, "%s: score_stride < max_len", w);
  if (batch == 0) return ok();
  if (!scores || !context_lens || !out_idx) return fail(SPMLA_EINVAL, "%s: null pointer", w);
  const size_t need = spmla::topk_workspace_size(batch, max_len, k);
  if (need > spmla::kTopkScratchBytes)
    return fail(SPMLA_EWORKSPACE, "%s: batch %d, max_len %lld need %zu bytes of workspace; the static scratch holds %zu",
                w, batch, (long long)max_len, need, spmla::kTopkScratchBytes);
  void* ws = nullptr;
  if (spmla::topk_scratch(&ws) != 0)
    return fail(SPMLA_ELAUNCH, "%s: the static scratch has no address on the current device (%s)", w,
                hipGetErrorString(hipGetLastError()));
  spmla::TopkArgs a{scores, score_stride, context_lens, batch, max_len, k, out_idx, ws, req_status};
  return map_launch(spmla::launch_topk(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int mla_paged_decode(const void* q, int32_t q_dtype, const void* kv_pool, const float* kv_scale, int32_t kv_dtype,
                     int32_t num_pages, int32_t page_size, const int32_t* block_table, int32_t bt_stride,
                     const int32_t* context_lens, int32_t batch, int64_t max_len, const int32_t* indices, int32_t k,
                     int32_t n_heads, int32_t d_latent, int32_t d_rope, float sm_scale, int32_t num_splits,
                     int32_t split_tokens, float* o_part, float* lse_part, int32_t* req_status, void* stream) {
  const char* w = "mla_paged_decode";
  if (int rc = check_paging(w, num_pages, page_size, block_table, bt_stride, context_lens, batch, max_len)) return rc;
  if (q_dtype != SPMLA_F32 && q_dtype != SPMLA_BF16) return fail(SPMLA_EUNSUPPORTED, "%s: q_dtype must be F32 or BF16", w);
  if (kv_dtype < SPMLA_F32 || kv_dtype > SPMLA_FP8_E4M3) return fail(SPMLA_EINVAL, "%s: bad kv_dtype", w);
  if (n_heads < 1 || n_heads > 256) return fail(SPMLA_EUNSUPPORTED, "%s: n_heads must be in [1, 256]", w);
  if (d_latent < 1 || d_rope < 0) return fail(SPMLA_EINVAL, "%s: bad d_latent / d_rope", w);
  if (!spmla::decode_generic_shape(q_dtype, kv_dtype, d_latent, d_rope))
    return fail(SPMLA_EUNSUPPORTED,
                "%s: d_latent (>= 8) and d_rope must be multiples of 8 with d_latent + d_rope <= %d; bf16 queries "
                "need a bf16 or FP8 cache", w, spmla::kDecodeGenericMaxDim);
  if (num_splits < 1 || num_splits > 64) return fail(SPMLA_EUNSUPPORTED, "%s: num_splits must be in [1, 64]", w);
  if (split_tokens < 0 || split_tokens % 32 != 0)
    return fail(SPMLA_EINVAL, "%s: split_tokens must be 0 or a positive multiple of 32", w);
  if (indices && (k < 0 || k > 65536)) return fail(SPMLA_EUNSUPPORTED, "%s: k must be in [0, 65536]", w);
  if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(SPMLA_EINVAL, "%s: sm_scale must be positive and finite", w);
  if (batch > 0) {
    if (!q || !kv_pool || !o_part || !lse_part) return fail(SPMLA_EINVAL, "%s: null pointer", w);
    if (kv_dtype == SPMLA_FP8_E4M3 && !kv_scale) return fail(SPMLA_EINVAL, "%s: FP8 cache needs kv_scale", w);
    if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(o_part))
      return fail(SPMLA_EINVAL, "%s: q, kv_pool and o_part must be 16-byte aligned", w);
  }
  spmla::DecodeArgs a{q, q_dtype, kv_pool, kv_scale, kv_dtype, num_pages, page_size, block_table, bt_stride,
                      context_lens, batch, max_len, indices, indices ? k : 0, n_heads, d_latent, d_rope, sm_scale,
                      num_splits, split_tokens, o_part, lse_part, req_status};
  return map_launch(spmla::launch_decode(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int lse_merge(const float* o_part, const float* lse_part, int32_t batch, int32_t num_splits, int32_t n_heads,
              int32_t d, float* o, float* lse, void* stream) {
  const char* w = "lse_merge";
  if (batch < 0 || n_heads < 0) return fail(SPMLA_EINVAL, "%s: negative size", w);
  if (num_splits < 1 || num_splits > 64) return fail(SPMLA_EUNSUPPORTED, "%s: num_splits must be in [1, 64]", w);
  if (d < 4 || d % 4 != 0) return fail(SPMLA_EUNSUPPORTED, "%s: d must be a positive multiple of 4", w);
  if (batch == 0 || n_heads == 0) return ok();
  if (!o_part || !lse_part || !o || !lse) return fail(SPMLA_EINVAL, "%s: null pointer", w);
  if (!aligned16(o_part) || !aligned16(o)) return fail(SPMLA_EINVAL, "%s: o_part and o must be 16-byte aligned", w);
  spmla::MergeArgs a{o_part, lse_part, batch, num_splits, n_heads, d, o, lse};
  return map_launch(spmla::launch_merge(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int kv_cache_append(const void* rows, int32_t row_dtype, int32_t batch, int32_t row_dim, void* pool,
                    float* pool_scale, int32_t pool_dtype, int32_t num_pages, int32_t page_size,
                    const int32_t* block_table, int32_t bt_stride, const int32_t* positions, int32_t* req_status,
                    void* stream) {
  const char* w = "kv_cache_append";
  if (batch < 0) return fail(SPMLA_EINVAL, "%s: batch < 0", w);
  if (row_dtype != SPMLA_F32 && row_dtype != SPMLA_BF16)
    return fail(SPMLA_EUNSUPPORTED, "%s: row_dtype must be F32 or BF16", w);
  if (pool_dtype < SPMLA_F32 || pool_dtype > SPMLA_FP8_E4M3) return fail(SPMLA_EINVAL, "%s: bad pool_dtype", w);
  if (row_dim < 8 || row_dim > 4096 || row_dim % 8 != 0)
    return fail(SPMLA_EUNSUPPORTED, "%s: row_dim must be a multiple of 8 in [8, 4096]", w);
  if (num_pages < 1) return fail(SPMLA_EINVAL, "%s: num_pages must be >= 1", w);
  if (!is_pow2_page(page_size)) return fail(SPMLA_EUNSUPPORTED, "%s: page_size must be 16, 32, 64 or 128", w);
  if (bt_stride < 1) return fail(SPMLA_EINVAL, "%s: bt_stride must be >= 1", w);
  if (batch == 0) return ok();
  if (!rows || !pool || !block_table || !positions) return fail(SPMLA_EINVAL, "%s: null pointer", w);
  if (pool_dtype == SPMLA_FP8_E4M3 && !pool_scale) return fail(SPMLA_EINVAL, "%s: an FP8 pool needs pool_scale", w);
  if (!aligned16(rows) || !aligned16(pool)) return fail(SPMLA_EINVAL, "%s: rows and pool must be 16-byte aligned", w);
  spmla::AppendArgs a{rows, row_dtype, batch, row_dim, pool, pool_scale, pool_dtype, num_pages, page_size,
                      block_table, bt_stride, positions, req_status};
  return map_launch(spmla::launch_cache_append(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int kv_cache_append_pair(const void* kv_rows, int32_t kv_dim, void* kv_pool, float* kv_scale, const void* idx_rows,
                         int32_t idx_dim, void* idx_pool, float* idx_scale, int32_t row_dtype, int32_t pool_dtype,
                         int32_t batch, int32_t num_pages, int32_t page_size, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* positions, int32_t* req_status, void* stream) {
  const char* w = "kv_cache_append_pair";
  if (batch < 0) return fail(SPMLA_EINVAL, "%s: batch < 0", w);
  if (row_dtype != SPMLA_F32 && row_dtype != SPMLA_BF16)
    return fail(SPMLA_EUNSUPPORTED, "%s: row_dtype must be F32 or BF16", w);
  if (pool_dtype < SPMLA_F32 || pool_dtype > SPMLA_FP8_E4M3) return fail(SPMLA_EINVAL, "%s: bad pool_dtype", w);
  for (int32_t d : {kv_dim, idx_dim})
    if (d < 8 || d > 4096 || d % 8 != 0)
      return fail(SPMLA_EUNSUPPORTED, "%s: row dims must be multiples of 8 in [8, 4096]", w);
  if (num_pages < 1) return fail(SPMLA_EINVAL, "%s: num_pages must be >= 1", w);
  if (!is_pow2_page(page_size)) return fail(SPMLA_EUNSUPPORTED, "%s: page_size must be 16, 32, 64 or 128", w);
  if (bt_stride < 1) return fail(SPMLA_EINVAL, "%s: bt_stride must be >= 1", w);
  if (batch == 0) return ok();
  if (!kv_rows || !kv_pool || !idx_rows || !idx_pool || !block_table || !positions)
    return fail(SPMLA_EINVAL, "%s: null pointer", w);
  if (pool_dtype == SPMLA_FP8_E4M3 && (!kv_scale || !idx_scale))
    return fail(SPMLA_EINVAL, "%s: FP8 pools need their scales", w);
  if (!aligned16(kv_rows) || !aligned16(kv_pool) || !aligned16(idx_rows) || !aligned16(idx_pool))
    return fail(SPMLA_EINVAL, "%s: rows and pools must be 16-byte aligned", w);
  spmla::AppendArgs a{kv_rows, row_dtype, batch, kv_dim, kv_pool, kv_scale, pool_dtype, num_pages, page_size,
                      block_table, bt_stride, positions, req_status, idx_rows, idx_dim, idx_pool, idx_scale};
  return map_launch(spmla::launch_cache_append(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int kv_page_check(const int32_t* block_table, const uint64_t* bt_tags, int32_t bt_stride, const int32_t* context_lens,
                  int32_t batch, int64_t max_len, const uint64_t* page_tags, int32_t num_pages, int32_t page_size,
                  int32_t* req_status, void* stream) {
  const char* w = "kv_page_check";
  if (int rc = check_paging(w, num_pages, page_size, block_table, bt_stride, context_lens, batch, max_len)) return rc;
  if (batch == 0) return ok();
  if (!bt_tags || !page_tags || !req_status) return fail(SPMLA_EINVAL, "%s: null pointer", w);
  if ((reinterpret_cast<uintptr_t>(bt_tags) | reinterpret_cast<uintptr_t>(page_tags)) & 7u)
    return fail(SPMLA_EINVAL, "%s: tag arrays must be 8-byte aligned", w);
  spmla::PageCheckArgs a{block_table, bt_tags, bt_stride, context_lens, batch, max_len, page_tags, num_pages,
                         page_size, req_status};
  return map_launch(spmla::launch_page_check(a, reinterpret_cast<hipStream_t>(stream)), w);
}

int mq_expand_requests(const int32_t* block_table, int32_t bt_stride, const int32_t* context_lens, int32_t batch,
                       int32_t n_q, int32_t* out_block_table, int32_t* out_lens, void* stream) {
  const char* w = "mq_expand_requests";
  if (batch < 0) return fail(SPMLA_EINVAL, "%s: batch < 0", w);
  if (n_q < 1 || n_q > 65536) return fail(SPMLA_EUNSUPPORTED, "%s: n_q must be in [1, 65536]", w);
  if (bt_stride < 1) return fail(SPMLA_EINVAL, "%s: bt_stride must be >= 1", w);
  if (batch == 0) return ok();
  if (!block_table || !context_lens || !out_block_table || !out_lens) return fail(SPMLA_EINVAL, "%s: null pointer", w);
  spmla::MqExpandArgs a{block_table, bt_stride, context_lens, batch, n_q, out_block_table, out_lens};
  return map_launch(spmla::launch_mq_expand(a, reinterpret_cast<hipStream_t>(stream)), w);
}

}  // extern "C"
