/*
 * sparse_mla.h -- C ABI of the sparse paged MLA decode library (libsparse_mla.so,
 * HIP for gfx950 / MI355X).
 *
 * One decode step of one attention layer, as the pages describe it: a DSA-style
 * indexer scores every history token of a request and attention keeps only the
 * Top-k of them, over MLA's compressed latent cache (cKV), a single row per
 * token shared by every head [KW 5.1.1, 5.1.2].  The cache is paged: a pool of
 * fixed-size pages plus a per-request block table from logical to physical
 * page, read through the table [EG, "PagedAttention's two primitives"], which
 * is what lets continuous batching run ragged, scattered requests [EG,
 * "implementation cost checklist", item 1].  Rows are stored bf16 or FP8 e4m3
 * and converted on read [WA section 1], with per-token scales [EG, "engineering
 * constraints of FP8 KV"].  Each request keeps its own latent rows, history and
 * index state [KW 5.1.3]; here the index state is a second pool of indexer keys
 * that shares the latent pool's page ids.  Split results are combined with the
 * online-softmax (m, l, O) algebra, which gives the same result as unsplit
 * attention [KW 5.2.2].
 *
 * Sources (page title -- site):
 *  [KW] "快手万擎大模型推理成本和性能优化实践" (Kuaishou Wanqing LLM inference cost
 *       and performance practice) -- 6aiq.com
 *  [EG] "推論エンジンの実践：Continuous Batching・Prefix Cache・Speculative Decoding"
 *       (inference-engine practice guide) -- deepseekmodel.com
 *  [WA] "より小さく、高速で、安全に：Kimi と GLM を大規模に展開するための実行方法"
 *       (Workers AI: smaller, faster, safer serving of Kimi and GLM) -- socker-news
 *
 * Conventions shared by every entry point
 *  - Pointers: every array pointer is DEVICE memory unless stated otherwise.
 *    The caller owns all memory; the library never allocates, frees or keeps a
 *    pointer beyond the work it enqueues (topk_select_noalloc's static
 *    workspace aside).  Buffers must stay alive until that work completes on
 *    `stream`.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream).  Every entry
 *    point only enqueues work; none synchronises the host.
 *  - Layouts: row-major, last dimension contiguous.  Pools and row arrays must
 *    be 16-byte aligned; every row length in bytes must be a multiple of 8.
 *  - Return value: SPMLA_OK, or a negative spmla_status when host-side
 *    validation rejects the call (null pointer, unsupported dtype or shape,
 *    workspace too small) -- then nothing is enqueued -- or when the launch
 *    itself fails (SPMLA_ELAUNCH).  spmla_last_error() gives a message.
 *  - Device-side faults in the data (a page id outside [0, num_pages), a
 *    context length outside [0, min(max_len, bt_stride * page_size)], an index
 *    outside [0, L) other than -1) never cause an out-of-bounds access: the
 *    offending request's bits are OR-ed into req_status[b] (when req_status is
 *    not NULL; the caller zeroes it) and that request's affected outputs are
 *    NaN (or not written, for a bad length).  Other requests are unaffected.
 *    The caller decides what to do with a flagged request, in the spirit of
 *    aborting a request rather than returning wrong data [WA section 3].
 *  - Reentrancy: stateless and thread-safe; calls on different streams may
 *    overlap (except topk_select_noalloc calls on one GPU, which share its
 *    static workspace).
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPMLA_OK = 0,
  SPMLA_EINVAL = -1,       /* null pointer, negative size, inconsistent arguments */
  SPMLA_EUNSUPPORTED = -2, /* valid but not implemented (dtype pair, shape) */
  SPMLA_ELAUNCH = -3,      /* the HIP launch failed */
  SPMLA_EWORKSPACE = -4    /* workspace missing or smaller than *_workspace_bytes */
} spmla_status;

typedef enum {
  SPMLA_F32 = 0,
  SPMLA_BF16 = 1,
  SPMLA_FP8_E4M3 = 2 /* OCP e4m3fn: bias 7, largest finite 448, no infinities */
} spmla_dtype;

/* Per-request status bits written to req_status[b]. */
enum { SPMLA_REQ_BAD_PAGE = 1, SPMLA_REQ_BAD_LEN = 2, SPMLA_REQ_BAD_INDEX = 4, SPMLA_REQ_BAD_TAG = 8 };

/*
 * dsa_indexer_scores -- indexer score of every history token of every request
 * (the ranking DSA uses to pick the Top-k tokens [KW 5.1.1]):
 *
 *   scores[b, t] = sum_h weights[b, h] * max(0, sum_i q_idx[b, h, i] * key(b, t)[i])
 *
 * for t < context_lens[b], where key(b, t) is row (block_table[b, t / page_size],
 * t % page_size) of k_pool, times k_scale of that row when FP8.  One key per
 * token is shared by all indexer heads.  Entries t >= context_lens[b] are not
 * written.
 *
 *  q_idx        [batch, n_heads, d], q_dtype F32 or BF16.  The arithmetic
 *               follows q_dtype: F32 -> fp32 products and sums (k_pool F32);
 *               BF16 -> bf16 products with fp32 sums (k_pool BF16 or FP8,
 *               widened exactly).
 *  weights      [batch, n_heads] fp32, any sign.
 *  k_pool       [num_pages, page_size, d] of k_dtype; k_scale [num_pages,
 *               page_size] fp32 when k_dtype is FP8, else ignored (may be NULL).
 *  block_table  [batch, bt_stride] int32 physical page ids.
 *  context_lens [batch] int32; max_len (host value) bounds every context_lens[b].
 *  scores       [batch, score_stride] fp32, score_stride >= max_len, rows
 *               16-byte aligned (scores aligned, score_stride a multiple of 4).
 *  req_status   [batch] int32 or NULL.
 * Supported: n_heads <= 128; d in {16, 32, 64, 128, 256} (bf16: d >= 32);
 * page_size in {16, 32, 64, 128}.
 */
int dsa_indexer_scores(const void* q_idx, int32_t q_dtype, const float* weights,
                       const void* k_pool, const float* k_scale, int32_t k_dtype,
                       int32_t num_pages, int32_t page_size,
                       const int32_t* block_table, int32_t bt_stride,
                       const int32_t* context_lens, int32_t batch, int64_t max_len,
                       int32_t n_heads, int32_t d,
                       float* scores, int64_t score_stride,
                       int32_t* req_status, void* stream);

/*
 * dsa_indexer_scores_mq -- the indexer for a multi-query verification step
 * (see mq_expand_requests): all n_q queries of a request are scored against
 * each key as it is read, so the key pool is read once for all of them.
 * Same arguments and arithmetic as dsa_indexer_scores, except:
 *  arithmetic with n_q = 2, FP8 keys and d = 128: each query row is held as
 *          2^(E-7) * (hi + lo/16), hi and lo e4m3 codes and E the exponent
 *          of the row's largest |q| (exact for every element within 2^14 of
 *          it, off by less than 2^-22 of it otherwise), and the products run
 *          on the scaled FP8 MFMA over the stored key codes: the scores agree
 *          with dsa_indexer_scores' to fp32 rounding, not bit for bit (with
 *          bf16 keys they are equal bit for bit);
 *  q_idx   [batch, n_q, n_heads, d], weights [batch, n_q, n_heads];
 *  scores  [batch * n_q, score_stride]: row b * n_q + i holds query i's
 *          scores for every t < context_lens[b] (the tokens that query may
 *          not see are computed too and must be ignored: the expanded
 *          lengths of mq_expand_requests bound what the top-k reads);
 *  req_status [batch * n_q] or NULL: a request's bits go to all its entries.
 * Supported: n_q = 1, or n_q = 2 with bf16 queries and n_heads 16, 32 or 64.
 */
int dsa_indexer_scores_mq(const void* q_idx, int32_t q_dtype, const float* weights,
                          const void* k_pool, const float* k_scale, int32_t k_dtype,
                          int32_t num_pages, int32_t page_size,
                          const int32_t* block_table, int32_t bt_stride,
                          const int32_t* context_lens, int32_t batch, int64_t max_len,
                          int32_t n_q, int32_t n_heads, int32_t d,
                          float* scores, int64_t score_stride,
                          int32_t* req_status, void* stream);

/*
 * topk_workspace_bytes -- device workspace topk_select needs for these sizes
 * (host function, no device work).  Returns 0 for invalid sizes.
 */
size_t topk_workspace_bytes(int32_t batch, int64_t max_len, int32_t k);

/*
 * topk_select -- the k_eff = min(k, L_b) best tokens of each request by score
 * [KW 5.1.1: attention keeps the Top-k history tokens].  Order: larger score
 * first; -0.0 equals +0.0; NaN ranks below every number; equal scores go to
 * the lower token index.  out_idx[b, 0 .. k_eff) lists the chosen token
 * indices in ascending order; out_idx[b, k_eff .. k) = -1.
 *
 *  scores       [batch, score_stride] fp32; only t < context_lens[b] is read.
 *  context_lens [batch] int32, each in [0, max_len] (else SPMLA_REQ_BAD_LEN and
 *               an all -1 row).
 *  out_idx      [batch, k] int32.
 *  workspace    device buffer of at least topk_workspace_bytes(batch, max_len, k)
 *               bytes; contents on entry are ignored (the call clears what it
 *               uses).  Calls that share a workspace must not overlap.
 *  req_status   [batch] int32 or NULL.
 * Supported: 1 <= k <= 4096; max_len < 2^31.
 * Launches: one when max_len <= 65536 and the score rows are 16-byte aligned
 * (scores aligned, score_stride a multiple of 4), else three; the result is
 * the same either way.
 */
int topk_select(const float* scores, int64_t score_stride,
                const int32_t* context_lens, int32_t batch, int64_t max_len, int32_t k,
                int32_t* out_idx, void* workspace, size_t workspace_bytes,
                int32_t* req_status, void* stream);

/*
 * topk_select_noalloc -- topk_select for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): same arguments, result, errors and launches, without the
 * workspace.  Its workspace is a static device array of
 * SPMLA_TOPK_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call itself allocates nothing.  Sizes for which
 * topk_workspace_bytes(batch, max_len, k) exceeds that array are rejected with
 * SPMLA_EWORKSPACE and nothing is enqueued.  The first call on a device
 * resolves the array's address there (call with that device current).  Every
 * call on one GPU shares the array, which keeps the last call's contents
 * (nothing in it needs clearing between calls): calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.
 */
#define SPMLA_TOPK_SCRATCH_BYTES ((size_t)32 << 20)
int topk_select_noalloc(const float* scores, int64_t score_stride,
                        const int32_t* context_lens, int32_t batch, int64_t max_len, int32_t k,
                        int32_t* out_idx, int32_t* req_status, void* stream);

/*
 * mla_paged_decode -- split-KV attention of every query head over a token set
 * of the paged latent cache.  For request b, head h and split s:
 *
 *   z_t   = sm_scale * sum_{i < d_latent + d_rope} q[b, h, i] * row(b, t)[i]
 *   o_part[b, s, h, :]  = sum_t softmax(z)_t * row(b, t)[0 .. d_latent)
 *   lse_part[b, s, h]   = ln sum_t exp(z_t)
 *
 * over the split's tokens; every head reads the same shared latent row
 * [KW 5.1.2], and the value of a token is its first d_latent dims.  The token
 * set is indices[b, 0 .. k) (entries -1 are skipped) or, with indices == NULL,
 * every t < context_lens[b].  Split s takes list positions [s*c, (s+1)*c)
 * (n = k, or context_lens[b] when dense), with
 *   split_tokens == 0: c = ceil(n / num_splits) rounded up to a multiple of
 *     32, the same number of splits for every request; a split with no
 *     tokens gives o_part = 0 and lse_part = -inf;
 *   split_tokens > 0 (a multiple of 32): c = split_tokens for every request,
 *     the last split (s = num_splits - 1) taking all positions from s*c to n:
 *     a long request spreads over more splits than a short one, so that a
 *     ragged batch gives every split about the same work.  Splits that start
 *     at or past n write lse_part = -inf and leave o_part unwritten
 *     (lse_merge gives them weight 0 and never reads their o_part).
 * With num_splits == 1 the partials are the final result; otherwise combine
 * them with lse_merge.
 *
 *  q            [batch, n_heads, d_latent + d_rope], q_dtype F32 or BF16 (the
 *               arithmetic follows it, as for dsa_indexer_scores).
 *  kv_pool      [num_pages, page_size, d_latent + d_rope] of kv_dtype;
 *               kv_scale [num_pages, page_size] fp32 iff FP8.
 *  o_part       [batch, num_splits, n_heads, d_latent] fp32.
 *  lse_part     [batch, num_splits, n_heads] fp32, natural log.
 *  split_tokens 0, or a positive multiple of 32 (else SPMLA_EINVAL): see above.
 * Supported: d_latent >= 8 and d_rope >= 0 multiples of 8 with
 * d_latent + d_rope <= 1024; q F32 over any cache, q BF16 over a bf16 or FP8
 * cache; n_heads <= 256; 1 <= num_splits <= 64; page_size in
 * {16, 32, 64, 128}; 0 <= k <= 65536.  Tuned kernels serve q BF16 with
 * 512 + 64 (bf16 or FP8 cache) and q F32 with 64 + 16; other shapes run a
 * plain fp32 kernel with the same results (to rounding) and status bits.
 */
int mla_paged_decode(const void* q, int32_t q_dtype,
                     const void* kv_pool, const float* kv_scale, int32_t kv_dtype,
                     int32_t num_pages, int32_t page_size,
                     const int32_t* block_table, int32_t bt_stride,
                     const int32_t* context_lens, int32_t batch, int64_t max_len,
                     const int32_t* indices, int32_t k,
                     int32_t n_heads, int32_t d_latent, int32_t d_rope, float sm_scale,
                     int32_t num_splits, int32_t split_tokens,
                     float* o_part, float* lse_part,
                     int32_t* req_status, void* stream);

/*
 * lse_merge -- combine split partials into the result over the union of the
 * splits, the online-softmax state algebra [KW 5.2.2]:
 *
 *   M = max_s lse_part[b, s, h] over splits with lse > -inf
 *   lse[b, h] = M + ln sum_s exp(lse_part[b, s, h] - M)
 *   o[b, h, :] = sum_s exp(lse_part[b, s, h] - lse[b, h]) * o_part[b, s, h, :]
 *
 * All splits empty: o = 0, lse = -inf.  Any NaN lse_part: o and lse NaN.
 *  o_part [batch, num_splits, n_heads, d], lse_part [batch, num_splits, n_heads]
 *  o      [batch, n_heads, d], lse [batch, n_heads] (fp32; may not alias inputs).
 * Supported: d a multiple of 4, 1 <= num_splits <= 64.
 */
int lse_merge(const float* o_part, const float* lse_part,
              int32_t batch, int32_t num_splits, int32_t n_heads, int32_t d,
              float* o, float* lse, void* stream);

/*
 * kv_cache_append -- write each request's new token row into its page slot,
 * quantising on write for an FP8 pool: the counterpart of dequant-on-read.
 * Every decode step appends the token it produced to its sequence, whose
 * cache sits in pages reached through the block table [EG, "Continuous
 * Batching": the per-step loop]; an FP8 cache holds e4m3 codes [WA section 1].
 * Called once for the latent pool (row_dim = d_latent + d_rope) and once for
 * the indexer-key pool (row_dim = d) with the same block table.
 *
 *  rows       [batch, row_dim] row_dtype F32 or BF16: the new rows.
 *  pool       [num_pages, page_size, row_dim] pool_dtype F32, BF16 or FP8_E4M3,
 *             written in place; pool_scale [num_pages, page_size] fp32 (FP8
 *             only, else may be NULL).
 *  positions  [batch] int32: the slot of request b is token positions[b]
 *             (page block_table[b][t / page_size], slot t mod page_size);
 *             t < 0 appends nothing for that request.  With context lengths
 *             that already count the new token, t = context_lens[b] - 1.
 *             Distinct requests must name distinct slots.
 *
 * FP8 pool: scale s = absmax(row) / 448 computed in fp32 (1 for an all-zero
 * row), stored in pool_scale; element i becomes the e4m3 code nearest to the
 * fp32 quotient x_i / s, ties to the even code.  BF16 pool: x rounded to
 * nearest even.  F32 pool: x.  Rows must be finite.  A position at or past
 * bt_stride * page_size sets SPMLA_REQ_BAD_LEN, a page id outside
 * [0, num_pages) sets SPMLA_REQ_BAD_PAGE; such a request writes nothing.
 * Supported: row_dim a multiple of 8 in [8, 4096]; page_size 16/32/64/128;
 * rows and pool 16-byte aligned.  Nothing is read from the pool.
 */
int kv_cache_append(const void* rows, int32_t row_dtype, int32_t batch, int32_t row_dim,
                    void* pool, float* pool_scale, int32_t pool_dtype,
                    int32_t num_pages, int32_t page_size,
                    const int32_t* block_table, int32_t bt_stride,
                    const int32_t* positions, int32_t* req_status, void* stream);

/*
 * kv_cache_append_pair -- kv_cache_append for the latent pool and the
 * indexer-key pool of the same new tokens in one launch: the two pools share
 * page ids, so one block table, one positions array and one num_pages serve
 * both.  kv_rows [batch, kv_dim] go to kv_pool (scales kv_scale), idx_rows
 * [batch, idx_dim] to idx_pool (scales idx_scale); both use row_dtype and
 * pool_dtype.  Same arithmetic, status bits and limits as kv_cache_append.
 */
int kv_cache_append_pair(const void* kv_rows, int32_t kv_dim, void* kv_pool, float* kv_scale,
                         const void* idx_rows, int32_t idx_dim, void* idx_pool, float* idx_scale,
                         int32_t row_dtype, int32_t pool_dtype, int32_t batch,
                         int32_t num_pages, int32_t page_size,
                         const int32_t* block_table, int32_t bt_stride,
                         const int32_t* positions, int32_t* req_status, void* stream);

/*
 * kv_page_check -- the KV-page integrity check, a separate batched pass run
 * before a step reads the cache.  Every physical page carries a tag that is
 * new on each reallocation; before decode reads the cache the mapping of
 * requests to pages is verified, and a request whose tags or mapping do not
 * match is aborted rather than served wrong data [WA section 3].  The check
 * is kept out of the attention kernels, as the pages keep it.
 *
 *  block_table [batch, bt_stride] int32 and bt_tags [batch, bt_stride]
 *              uint64: entry j of request b and the tag its page had when it
 *              was given to the request.
 *  page_tags   [num_pages] uint64: each page's current tag.
 *  req_status  [batch] int32 (required): for every entry j <
 *              ceil(context_lens[b] / page_size), a page id outside
 *              [0, num_pages) ORs SPMLA_REQ_BAD_PAGE and a tag that differs
 *              from page_tags[page] ORs SPMLA_REQ_BAD_TAG; a length outside
 *              [0, min(max_len, bt_stride * page_size)] ORs SPMLA_REQ_BAD_LEN.
 *              Entries past a request's pages are not read.
 *
 * The outputs that the other calls produce for a flagged request must not be
 * used.  Supported: page_size 16/32/64/128; tag arrays 8-byte aligned.
 */
int kv_page_check(const int32_t* block_table, const uint64_t* bt_tags, int32_t bt_stride,
                  const int32_t* context_lens, int32_t batch, int64_t max_len,
                  const uint64_t* page_tags, int32_t num_pages, int32_t page_size,
                  int32_t* req_status, void* stream);

/*
 * mq_expand_requests -- bookkeeping for a multi-query verification step.  A
 * speculative step verifies the gamma+1 drafted positions of each request
 * in one parallel forward, each position seeing only itself and what
 * precedes it [EG, "Speculative Decoding"; KW 5.3].  With the n_q new tokens
 * already in the cache (context_lens counts them), query i of request b is
 * run as request v = b * n_q + i of an expanded batch: block-table row v is
 * a copy of row b and its length is L_b - n_q + 1 + i.  The indexer, top-k,
 * decode and merge calls then take the expanded batch unchanged (queries
 * laid out [batch, n_q, ...] are already [batch * n_q, ...]), so every query
 * gets its own scores, its own top-k and its own attention.
 *
 *  block_table [batch, bt_stride], context_lens [batch]: the real requests.
 *  out_block_table [batch * n_q, bt_stride], out_lens [batch * n_q]: written.
 *  A request with L_b < n_q gets length -1 for all its queries, which the
 *  later calls flag as SPMLA_REQ_BAD_LEN.  Supported: 1 <= n_q <= 65536.
 *
 * The same expansion serves a prefill chunk of n_q new tokens attending
 * densely and causally: mla_paged_decode with indices = NULL over the
 * expanded batch computes, for every query, one partial per KV split (a
 * block of the context), and lse_merge combines the blocks with the online
 * softmax state, the single-GPU form of blockwise ring attention [KW 5.2.2].
 */
int mq_expand_requests(const int32_t* block_table, int32_t bt_stride, const int32_t* context_lens,
                       int32_t batch, int32_t n_q, int32_t* out_block_table, int32_t* out_lens,
                       void* stream);

/* Message of the last failing call on this thread (host memory, valid until
 * the next call on this thread). */
const char* spmla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
