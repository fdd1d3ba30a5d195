/*
 * fp64 CPU oracle for the sparse paged MLA decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the bench's CPU
 * baseline use it.  It shares no code with the HIP library (its own FP8 and
 * bf16 decoders, its own page lookup, its own softmax); the only thing the two
 * sides share is the seeded input generator, which holds none of this
 * arithmetic.
 *
 * It is deliberately plain: straight loops in the order the definitions read,
 * double precision throughout, no blocking, no fusion, no reordering.
 *
 * Sources (page title -- where on the page):
 *  [KW] "快手万擎大模型推理成本和性能优化实践" (Kuaishou Wanqing: LLM inference
 *       cost and performance practice), 6aiq.com.
 *  [EG] "推論エンジンの実践：Continuous Batching・Prefix Cache・Speculative
 *       Decoding" (inference-engine practice guide), deepseekmodel.com.
 *  [WA] "より小さく、高速で、安全に：Kimi と GLM を大規模に展開するための実行方法"
 *       (Workers AI: KV quantisation, weight compression, cache integrity),
 *       socker-news summary.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Indexer score of token t: s_t = sum_h w_h * max(0, q_h . k_t), one key per
 *    token shared by all indexer heads, no extra scale.  The pages only say
 *    that DSA ranks history tokens and attention keeps the Top-k [KW 5.1.1].
 *  - Top-k: the min(k, L) largest scores; equal scores go to the lower token
 *    index; -0 equals +0; NaN ranks below every number; output ascending,
 *    padded with -1.
 *  - Attention: z_t = sm_scale * (q_h . c_t) over all d_latent + d_rope dims;
 *    the value of token t is its first d_latent dims; o = softmax(z) . V;
 *    lse = natural log of sum_t exp(z_t).  An empty token set gives o = 0,
 *    lse = -inf.
 *  - FP8 rows: OCP e4m3fn code times the row's fp32 scale, one scale per token
 *    over the whole row.
 *  - Cache append (quantise on write): scale = absmax / 448 in fp32 (1 for a
 *    zero row), each code the nearest e4m3 value of the fp32 quotient x / scale
 *    with ties to the even code; the pages name e4m3 [WA section 1] but not
 *    the scale rule or the rounding.
 *
 * Parity pins for every function live in the tests (brute force on tiny
 * inputs, closed forms, invariants, library routines); see the test files.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2 };
enum { OR_BAD_PAGE = 1, OR_BAD_LEN = 2, OR_BAD_INDEX = 4, OR_BAD_TAG = 8 };

/* ---------------------------------------------------------------- decoders */

/* OCP FP8 e4m3fn: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no
 * infinities, so exponent field 15 with mantissa 0..6 is an ordinary normal
 * number (largest finite: 1.75 * 2^8 = 448).  The pages name the e4m3 format
 * for the FP8 KV cache [WA section 1]. */
double oracle_fp8_e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* base, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  if (dtype == OR_BF16) return oracle_bf16_value(((const uint16_t*)base)[i]);
  return oracle_fp8_e4m3_value(((const uint8_t*)base)[i]);
}

/* ----------------------------------------------------------- paged lookup */

/* Token t of request b lives in physical page block_table[b][t / P], slot
 * t mod P: the block table maps logical blocks to physical blocks of a
 * fixed-size pool and every read goes through it [EG, "PagedAttention's two
 * primitives"].  Returns the flat row number (page * P + slot) or -1 when the
 * page id is out of [0, num_pages). */
static int64_t row_of(const int32_t* bt, int32_t bt_stride, int32_t b, int64_t t,
                      int32_t page_size, int32_t num_pages) {
  int32_t page = bt[(int64_t)b * bt_stride + t / page_size];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_size + t % page_size;
}

/* Dequantise one cached row into out[0 .. dim): exact widening for fp32/bf16;
 * FP8 code times the token's scale for e4m3 [WA section 1: FP8 values are
 * converted on read]. */
static void load_row(const void* pool, const float* scale, int dtype, int64_t row, int32_t dim, double* out) {
  double s = (dtype == OR_FP8) ? (double)scale[row] : 1.0;
  for (int32_t i = 0; i < dim; ++i) out[i] = elem(pool, dtype, row * dim + i) * s;
}

static int len_ok(int32_t len, int32_t bt_stride, int32_t page_size, int64_t max_len) {
  return len >= 0 && (int64_t)len <= max_len && (int64_t)len <= (int64_t)bt_stride * page_size;
}

/* Status check of one request's mapping: every page its length needs must
 * be a valid pool page. */
static int32_t check_request(const int32_t* bt, int32_t bt_stride, const int32_t* lens, int32_t b,
                             int32_t page_size, int32_t num_pages, int64_t max_len) {
  int32_t len = lens[b];
  if (!len_ok(len, bt_stride, page_size, max_len)) return OR_BAD_LEN;
  int64_t pages = ((int64_t)len + page_size - 1) / page_size;
  for (int64_t j = 0; j < pages; ++j) {
    int32_t p = bt[(int64_t)b * bt_stride + j];
    if (p < 0 || p >= num_pages) return OR_BAD_PAGE;
  }
  return 0;
}

/* ------------------------------------------------------------------ indexer */

/* Score of token t of request b (reading above):
 *   s = sum_h w[b,h] * max(0, sum_i q_idx[b,h,i] * k_t[i]),
 * and the magnitude A = sum_h |w[b,h]| * sum_i |q_idx[b,h,i] * k_t[i]| that
 * bounds the rounding of any accumulation order. */
static void score_one(const void* q_idx, int q_dtype, const float* w, const double* krow,
                      int32_t b, int32_t n_heads, int32_t d, double* s_out, double* a_out) {
  double s = 0.0, a = 0.0;
  for (int32_t h = 0; h < n_heads; ++h) {
    double dot = 0.0, mag = 0.0;
    int64_t qo = ((int64_t)b * n_heads + h) * d;
    for (int32_t i = 0; i < d; ++i) {
      double p = elem(q_idx, q_dtype, qo + i) * krow[i];
      dot += p;
      mag += fabs(p);
    }
    double wh = (double)w[(int64_t)b * n_heads + h];
    s += wh * (dot > 0.0 ? dot : 0.0);
    a += fabs(wh) * mag;
  }
  *s_out = s;
  *a_out = a;
}

/* Full scores for every request: scores[b, t] for t < lens[b]; entries at
 * t >= lens[b] are left as they are.  status[b] gets the request's mapping
 * flags; a flagged request's scores are NaN. */
int oracle_indexer_scores(const void* q_idx, int q_dtype, const float* w,
                          const void* k_pool, const float* k_scale, int k_dtype,
                          int32_t num_pages, int32_t page_size,
                          const int32_t* bt, int32_t bt_stride, const int32_t* lens, int32_t batch,
                          int64_t max_len, int32_t n_heads, int32_t d,
                          double* scores, double* mags, int64_t score_stride, int32_t* status) {
  double* krow = (double*)malloc(sizeof(double) * (size_t)d);
  if (!krow) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    int32_t st = check_request(bt, bt_stride, lens, b, page_size, num_pages, max_len);
    if (status) status[b] = st;
    int64_t len = lens[b];
    if (st & OR_BAD_LEN) continue;
    for (int64_t t = 0; t < len; ++t) {
      double s, a;
      if (st) {
        s = NAN;
        a = NAN;
      } else {
        load_row(k_pool, k_scale, k_dtype, row_of(bt, bt_stride, b, t, page_size, num_pages), d, krow);
        score_one(q_idx, q_dtype, w, krow, b, n_heads, d, &s, &a);
      }
      scores[(int64_t)b * score_stride + t] = s;
      if (mags) mags[(int64_t)b * score_stride + t] = a;
    }
  }
  free(krow);
  return 0;
}

/* Scores at sampled (request, token) positions only; for checks at sizes
 * where the full pass is too slow.  Positions must be valid. */
int oracle_indexer_scores_at(const void* q_idx, int q_dtype, const float* w,
                             const void* k_pool, const float* k_scale, int k_dtype,
                             int32_t num_pages, int32_t page_size,
                             const int32_t* bt, int32_t bt_stride,
                             int32_t n_heads, int32_t d,
                             const int32_t* sb, const int64_t* stok, int64_t n,
                             double* s_out, double* a_out) {
  double* krow = (double*)malloc(sizeof(double) * (size_t)d);
  if (!krow) return -1;
  for (int64_t j = 0; j < n; ++j) {
    int64_t row = row_of(bt, bt_stride, sb[j], stok[j], page_size, num_pages);
    if (row < 0) { s_out[j] = NAN; a_out[j] = NAN; continue; }
    load_row(k_pool, k_scale, k_dtype, row, d, krow);
    score_one(q_idx, q_dtype, w, krow, sb[j], n_heads, d, &s_out[j], &a_out[j]);
  }
  free(krow);
  return 0;
}

/* -------------------------------------------------------------------- top-k */

typedef struct { double s; int64_t t; } scored;

/* Rank order: numbers descending (-0 and +0 compare equal), every NaN after
 * every number, equal keys by ascending token index. */
static int before(const scored* a, const scored* b) {
  int an = isnan(a->s), bn = isnan(b->s);
  if (an != bn) return bn;          /* a number ranks before a NaN */
  if (!an && a->s != b->s) return a->s > b->s;
  return a->t < b->t;
}

static int cmp_rank(const void* x, const void* y) {
  const scored* a = (const scored*)x;
  const scored* b = (const scored*)y;
  if (before(a, b)) return -1;
  if (before(b, a)) return 1;
  return 0;
}

static int cmp_i32(const void* x, const void* y) {
  int32_t a = *(const int32_t*)x, b = *(const int32_t*)y;
  return (a > b) - (a < b);
}

/* The k_eff = min(k, L_b) best tokens of each request under the rank order,
 * listed ascending by token index, padded with -1 up to k.  DSA keeps the
 * Top-k history tokens for attention [KW 5.1.1]. */
int oracle_topk(const double* scores, int64_t score_stride, const int32_t* lens, int32_t batch,
                int32_t k, int32_t* out_idx) {
  for (int32_t b = 0; b < batch; ++b) {
    int64_t len = lens[b];
    int32_t* out = out_idx + (int64_t)b * k;
    for (int32_t j = 0; j < k; ++j) out[j] = -1;
    if (len <= 0) continue;
    scored* v = (scored*)malloc(sizeof(scored) * (size_t)len);
    if (!v) return -1;
    for (int64_t t = 0; t < len; ++t) { v[t].s = scores[(int64_t)b * score_stride + t]; v[t].t = t; }
    qsort(v, (size_t)len, sizeof(scored), cmp_rank);
    int64_t keff = len < k ? len : k;
    for (int64_t j = 0; j < keff; ++j) out[j] = (int32_t)v[j].t;
    qsort(out, (size_t)keff, sizeof(int32_t), cmp_i32);
    free(v);
  }
  return 0;
}

/* ---------------------------------------------------------------- attention */

/* Attention of every query head of every request over a token set: the
 * tokens listed in indices[b, 0..k) (entries -1 are padding), or, with
 * indices == NULL, every token t < L_b.  All heads read the same cached
 * latent row (MLA's compressed cKV is shared by all heads and cannot be split
 * by head [KW 5.1.2]).  Per head h:
 *   z_t = sm_scale * sum_{i < d_latent + d_rope} q[b,h,i] * c_t[i]
 *   m = max_t z_t,  l = sum_t exp(z_t - m)
 *   o[b,h,:] = sum_t exp(z_t - m) * c_t[0 .. d_latent) / l,  lse[b,h] = m + ln l.
 * Index entries outside [0, L_b) other than -1 flag OR_BAD_INDEX; a flagged
 * request's outputs are NaN. */
int oracle_mla_attention(const void* q, int q_dtype, const void* kv, const float* kv_scale, int kv_dtype,
                         int32_t num_pages, int32_t page_size,
                         const int32_t* bt, int32_t bt_stride, const int32_t* lens, int32_t batch,
                         int64_t max_len, const int32_t* indices, int32_t k,
                         int32_t n_heads, int32_t d_latent, int32_t d_rope, double sm_scale,
                         double* o, double* lse, int32_t* status) {
  const int32_t D = d_latent + d_rope;
  for (int32_t b = 0; b < batch; ++b) {
    int32_t st = check_request(bt, bt_stride, lens, b, page_size, num_pages, max_len);
    int64_t len = lens[b];
    int64_t n_tok = indices ? k : len;
    if (!(st & OR_BAD_LEN) && indices) {
      for (int64_t j = 0; j < n_tok; ++j) {
        int32_t t = indices[(int64_t)b * k + j];
        if (t < -1 || t >= len) st |= OR_BAD_INDEX;
      }
    }
    if (status) status[b] = st;
    if (st) {
      for (int32_t h = 0; h < n_heads; ++h) {
        for (int32_t i = 0; i < d_latent; ++i) o[((int64_t)b * n_heads + h) * d_latent + i] = NAN;
        lse[(int64_t)b * n_heads + h] = NAN;
      }
      continue;
    }
    /* Gather the set's rows once (dequantised). */
    int64_t n_valid = 0;
    for (int64_t j = 0; j < n_tok; ++j)
      if (!indices || indices[(int64_t)b * k + j] >= 0) ++n_valid;
    double* rows = (double*)malloc(sizeof(double) * (size_t)(n_valid > 0 ? n_valid : 1) * (size_t)D);
    double* z = (double*)malloc(sizeof(double) * (size_t)(n_valid > 0 ? n_valid : 1));
    if (!rows || !z) { free(rows); free(z); return -1; }
    int64_t r = 0;
    for (int64_t j = 0; j < n_tok; ++j) {
      int64_t t = indices ? indices[(int64_t)b * k + j] : j;
      if (t < 0) continue;
      load_row(kv, kv_scale, kv_dtype, row_of(bt, bt_stride, b, t, page_size, num_pages), D, rows + r * D);
      ++r;
    }
    for (int32_t h = 0; h < n_heads; ++h) {
      double* oh = o + ((int64_t)b * n_heads + h) * d_latent;
      int64_t qo = ((int64_t)b * n_heads + h) * D;
      if (n_valid == 0) {
        for (int32_t i = 0; i < d_latent; ++i) oh[i] = 0.0;
        lse[(int64_t)b * n_heads + h] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int64_t j = 0; j < n_valid; ++j) {
        double dot = 0.0;
        for (int32_t i = 0; i < D; ++i) dot += elem(q, q_dtype, qo + i) * rows[j * D + i];
        z[j] = sm_scale * dot;
        if (z[j] > m) m = z[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < n_valid; ++j) l += exp(z[j] - m);
      for (int32_t i = 0; i < d_latent; ++i) oh[i] = 0.0;
      for (int64_t j = 0; j < n_valid; ++j) {
        double p = exp(z[j] - m) / l;
        for (int32_t i = 0; i < d_latent; ++i) oh[i] += p * rows[j * D + i];
      }
      lse[(int64_t)b * n_heads + h] = m + log(l);
    }
    free(rows);
    free(z);
  }
  return 0;
}

/* --------------------------------------------------------------- LSE merge */

/* Combine per-split partial results (o_j, lse_j) of the same query into the
 * result over the union of the splits' disjoint token sets.  This is the
 * online-softmax state carried across KV blocks, which reproduces full
 * attention exactly [KW 5.2.2; KW 5.2.3 notes that the blockwise schedule
 * does not change the mathematical result]:
 *   M = max_j lse_j over splits with lse_j > -inf
 *   lse = M + ln sum_j exp(lse_j - M)
 *   o = sum_j exp(lse_j - lse) * o_j
 * If every split is empty (lse_j = -inf for all j): o = 0, lse = -inf.
 * Layout: o_part [B, S, H, d], lse_part [B, S, H]; o [B, H, d], lse [B, H]. */
int oracle_lse_merge(const double* o_part, const double* lse_part, int32_t batch, int32_t splits,
                     int32_t n_heads, int32_t d, double* o, double* lse) {
  for (int32_t b = 0; b < batch; ++b) {
    for (int32_t h = 0; h < n_heads; ++h) {
      double* oh = o + ((int64_t)b * n_heads + h) * d;
      double M = -INFINITY;
      int any_nan = 0;
      for (int32_t j = 0; j < splits; ++j) {
        double v = lse_part[((int64_t)b * splits + j) * n_heads + h];
        if (isnan(v)) any_nan = 1;
        if (v > M) M = v;
      }
      if (any_nan) {
        for (int32_t i = 0; i < d; ++i) oh[i] = NAN;
        lse[(int64_t)b * n_heads + h] = NAN;
        continue;
      }
      if (M == -INFINITY) {
        for (int32_t i = 0; i < d; ++i) oh[i] = 0.0;
        lse[(int64_t)b * n_heads + h] = -INFINITY;
        continue;
      }
      double sum = 0.0;
      for (int32_t j = 0; j < splits; ++j) {
        double v = lse_part[((int64_t)b * splits + j) * n_heads + h];
        if (v > -INFINITY) sum += exp(v - M);
      }
      double L = M + log(sum);
      for (int32_t i = 0; i < d; ++i) oh[i] = 0.0;
      for (int32_t j = 0; j < splits; ++j) {
        double v = lse_part[((int64_t)b * splits + j) * n_heads + h];
        if (!(v > -INFINITY)) continue;
        double wgt = exp(v - L);
        const double* oj = o_part + (((int64_t)b * splits + j) * n_heads + h) * d;
        for (int32_t i = 0; i < d; ++i) oh[i] += wgt * oj[i];
      }
      lse[(int64_t)b * n_heads + h] = L;
    }
  }
  return 0;
}

/* ------------------------------------------------------------ cache append */

/* OCP e4m3fn code of a binary32 value: the finite code nearest to |q|, ties
 * going to the code with an even mantissa, chosen by looking at all 127
 * non-negative finite codes; magnitudes past 448 take the largest code
 * (saturation, the generator's convention for the FP8 cache).  The sign bit
 * is q's own, so -0 and negative values that round to zero give 0x80.  NaN
 * gives the NaN code. */
uint8_t oracle_fp8_e4m3_encode(float q) {
  if (isnan(q)) return signbit(q) ? 0xFF : 0x7F;
  if (isinf(q)) return signbit(q) ? 0xFE : 0x7E;
  double a = fabs((double)q);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(oracle_fp8_e4m3_value((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best_d = d;
      best = c;
    }
  }
  return (uint8_t)(signbit(q) ? (best | 0x80) : best);
}

void oracle_fp8_e4m3_encode_array(const float* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_e4m3_encode(q[i]);
}

/* bf16 bits of a binary32 value, round to nearest with ties to even (the
 * upper 16 bits, incremented when the dropped half exceeds one half ulp or
 * equals it with an odd kept part); NaN stays a quiet NaN. */
uint16_t oracle_bf16_encode(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040);
  uint32_t kept = u >> 16, dropped = u & 0xFFFF;
  if (dropped > 0x8000 || (dropped == 0x8000 && (kept & 1))) kept += 1;
  return (uint16_t)kept;
}

void oracle_bf16_encode_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_encode(x[i]);
}

/* Append one new token row per request to its page slot.  Each decode step
 * appends the token just produced to its sequence, whose cache lives in
 * blocks reached through the block table [EG, "Continuous Batching": the
 * per-step loop]; an FP8 cache stores e4m3 codes [WA section 1].  Token
 * positions[b] of request b goes to page block_table[b][t / P], slot t mod P
 * (t < 0: the request appends nothing).  FP8 pool (reading): one fp32 scale
 * per token, s = absmax / 448 computed in fp32 (1 for an all-zero row), and
 * code_i = e4m3(x_i / s) with the quotient rounded to fp32 first; bf16 pool:
 * x rounded to nearest even; fp32 pool: x.  A position past the mapped pages
 * flags BAD_LEN and a page id outside [0, num_pages) flags BAD_PAGE; such a
 * request writes nothing. */
int oracle_cache_append(const void* rows, int row_dtype, int32_t batch, int32_t dim, void* pool, float* pool_scale,
                        int pool_dtype, int32_t num_pages, int32_t page_size, const int32_t* bt, int32_t bt_stride,
                        const int32_t* positions, int32_t* status) {
  float* x = (float*)malloc(sizeof(float) * (size_t)(dim > 0 ? dim : 1));
  if (!x) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    int32_t t = positions[b];
    if (t < 0) continue;
    if ((int64_t)t >= (int64_t)bt_stride * page_size) {
      status[b] |= OR_BAD_LEN;
      continue;
    }
    int64_t row = row_of(bt, bt_stride, b, t, page_size, num_pages);
    if (row < 0) {
      status[b] |= OR_BAD_PAGE;
      continue;
    }
    for (int32_t i = 0; i < dim; ++i) x[i] = (float)elem(rows, row_dtype, (int64_t)b * dim + i);
    if (pool_dtype == OR_FP8) {
      float amax = 0.0f;
      for (int32_t i = 0; i < dim; ++i)
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      pool_scale[row] = sc;
      for (int32_t i = 0; i < dim; ++i) {
        float q = x[i] / sc;
        ((uint8_t*)pool)[row * dim + i] = oracle_fp8_e4m3_encode(q);
      }
    } else if (pool_dtype == OR_BF16) {
      for (int32_t i = 0; i < dim; ++i) ((uint16_t*)pool)[row * dim + i] = oracle_bf16_encode(x[i]);
    } else {
      for (int32_t i = 0; i < dim; ++i) ((float*)pool)[row * dim + i] = x[i];
    }
  }
  free(x);
  return 0;
}

/* ------------------------------------------------------- page integrity */

/* Integrity check of every request's page mapping before the cache is read.
 * Each physical page carries a tag that is new on every reallocation, and
 * before decode reads the cache the server checks which request uses which
 * page; on a mismatch the request is aborted rather than served wrong data
 * [WA section 3: tag management, mapping verification].  Reading: the tag
 * each request expects for its logical page j is recorded beside its block
 * table entry (bt_tags[b][j], written when the page was given to it), and
 * the check compares it with the page's current tag page_tags[bt[b][j]] for
 * every page the request's length covers.  A length outside
 * [0, min(max_len, bt_stride * page_size)] flags BAD_LEN (nothing else is
 * checked); a page id outside [0, num_pages) flags BAD_PAGE; a tag that
 * differs flags BAD_TAG.  Entries past a request's pages are not looked at. */
int oracle_page_check(const int32_t* bt, const uint64_t* bt_tags, int32_t bt_stride, const int32_t* lens,
                      int32_t batch, int64_t max_len, const uint64_t* page_tags, int32_t num_pages,
                      int32_t page_size, int32_t* status) {
  for (int32_t b = 0; b < batch; ++b) {
    int32_t len = lens[b];
    if (!len_ok(len, bt_stride, page_size, max_len)) {
      status[b] |= OR_BAD_LEN;
      continue;
    }
    int64_t pages = ((int64_t)len + page_size - 1) / page_size;
    for (int64_t j = 0; j < pages; ++j) {
      int32_t p = bt[(int64_t)b * bt_stride + j];
      if (p < 0 || p >= num_pages) status[b] |= OR_BAD_PAGE;
      else if (page_tags[p] != bt_tags[(int64_t)b * bt_stride + j]) status[b] |= OR_BAD_TAG;
    }
  }
  return 0;
}

/* ---------------------------------------------------------- cache accounting */

/* KV-cache bytes per token of a standard multi-head model: 2 (K and V) x
 * layers x KV heads x head dim x bytes per element [EG, memory-wall section:
 * the KV-size formula and its 60-layer, 48-head, 128-dim FP16 example]. */
double oracle_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim, double bytes_per_elem) {
  return 2.0 * layers * kv_heads * head_dim * bytes_per_elem;
}

/* MLA analogue for one layer: one shared latent row of d_latent + d_rope
 * elements per token, no separate K and V (the compressed cKV is one state
 * shared across heads [KW 5.1.2]), plus the per-token scale bytes when FP8.
 * The pages only say MLA shrinks the heads x head-dim term [EG, ledger
 * section]; this accounting is the reading used for the pools. */
double oracle_mla_bytes_per_token(int32_t d_latent, int32_t d_rope, double bytes_per_elem, double scale_bytes) {
  return (double)(d_latent + d_rope) * bytes_per_elem + scale_bytes;
}
