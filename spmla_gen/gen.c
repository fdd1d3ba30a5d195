/*
 * Seeded synthetic-input generator shared by the HIP path's tests/bench and
 * by the fp64 oracle's tests.  It holds none of the attention method's
 * arithmetic: it only draws numbers and stores them in the storage formats
 * the cache uses (fp32, bf16, FP8 e4m3fn with a per-token scale).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw i of stream key K is mix64(K + (i + 1) * GAMMA), where
 * mix64 is SplitMix64's output finaliser.  A stream key is derived from
 * (seed, tensor id, sub-stream) by chaining mix64, so every element of every
 * tensor can be regenerated on its own.  Normals use the Box-Muller
 * transform (cosine branch) on draws 2i and 2i+1.
 *
 * Storage encoders: bf16 is round-to-nearest-even of the fp32 value.  FP8 is
 * the OCP 8-bit e4m3fn format (4 exponent bits, bias 7, 3 mantissa bits,
 * largest finite 448, no infinities, S.1111.111 is NaN); values are divided
 * by a per-row scale absmax/448 (scale 1 for an all-zero row), rounded to
 * nearest even and saturated to +-448.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t spmla_gen_stream_key(uint64_t seed, uint64_t tensor_id, uint64_t sub) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ (tensor_id + 1) * GAMMA);
  k = mix64(k ^ (sub + 1) * GAMMA);
  return k;
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* Uniform in [0, 1) with 53 random bits. */
static inline double unif01(uint64_t key, uint64_t i) { return (double)(draw(key, i) >> 11) * 0x1.0p-53; }

/* Standard normal for element i: Box-Muller on draws 2i, 2i+1; u1 in (0, 1]. */
static inline double normal(uint64_t key, uint64_t i) {
  double u1 = (double)((draw(key, 2 * i) >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(draw(key, 2 * i + 1) >> 11) * 0x1.0p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP e4m3fn encode of a finite double, round-to-nearest-even, saturating. */
static inline uint8_t encode_e4m3(double v) {
  uint8_t sign = 0;
  if (v < 0) { sign = 0x80; v = -v; }
  if (!(v == v)) return 0x7F;
  if (v >= 448.0) return sign | 0x7E;
  /* Subnormal range: step 2^-9 below 2^-6. Code m (0..8) for m*2^-9; m == 8 is exactly 2^-6 = code 0x08. */
  if (v < 0x1.0p-6) {
    double q = v * 512.0;
    double r = nearbyint(q); /* default rounding mode: nearest-even */
    return sign | (uint8_t)r;
  }
  int e;
  double fr = frexp(v, &e);  /* v = fr * 2^e, fr in [0.5, 1) */
  int ex = e - 1;            /* v = (2 fr) * 2^ex, 2fr in [1, 2) */
  double mant = (2.0 * fr - 1.0) * 8.0;
  double mr = nearbyint(mant);
  if (mr >= 8.0) { mr = 0.0; ex += 1; }
  int code = ((ex + 7) << 3) | (int)mr;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

void spmla_gen_normal_f32(uint64_t key, uint64_t i0, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = (float)normal(key, i0 + (uint64_t)j);
}

void spmla_gen_uniform_f64(uint64_t key, uint64_t i0, int64_t n, double* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = unif01(key, i0 + (uint64_t)j);
}

void spmla_gen_normal_f64(uint64_t key, uint64_t i0, int64_t n, double* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = normal(key, i0 + (uint64_t)j);
}

void spmla_gen_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = f32_to_bf16_rne(x[j]);
}

/* Encode rows [rows, dim] of fp32 into e4m3fn with one scale per row. */
void spmla_gen_rows_to_fp8(const float* x, int64_t rows, int32_t dim, uint8_t* out, float* scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * dim;
    float amax = 0.f;
    for (int32_t d = 0; d < dim; ++d) { float a = fabsf(xr[d]); if (a > amax) amax = a; }
    float s = amax > 0.f ? amax / 448.0f : 1.0f;
    scale[r] = s;
    for (int32_t d = 0; d < dim; ++d) out[r * dim + d] = encode_e4m3((double)xr[d] / (double)s);
  }
}

/*
 * Fill a paged pool with per-token rows.  Token t of request b (t < lens[b])
 * gets dim normals drawn from stream (seed, tensor_id, sub=b) at counters
 * t*dim .. t*dim+dim-1, stored in the requested format at physical page
 * block_table[b*bt_stride + t/page_size], slot t % page_size.
 * dtype: 0 fp32 (out is float*), 1 bf16 (uint16*), 2 fp8 e4m3fn (uint8*, with
 * per-token scale written to scale[page*page_size + slot]).
 * Slots that no token maps to are left untouched (the caller pre-fills them).
 */
int spmla_gen_fill_pool(uint64_t seed, uint64_t tensor_id, int32_t batch, const int32_t* lens,
                        int32_t page_size, int32_t dim, const int32_t* block_table, int32_t bt_stride,
                        int32_t dtype, void* out, float* scale, int32_t poison_tail) {
  if (dim > 4096 || dim <= 0 || page_size <= 0) return -1;
  int64_t total_pages = 0;
  for (int32_t b = 0; b < batch; ++b) total_pages += (lens[b] + page_size - 1) / page_size;
  /* Flatten (request, logical page) so the parallel loop balances ragged lengths. */
  int64_t* starts = (int64_t*)__builtin_alloca(sizeof(int64_t) * (size_t)(batch + 1));
  starts[0] = 0;
  for (int32_t b = 0; b < batch; ++b) starts[b + 1] = starts[b] + (lens[b] + page_size - 1) / page_size;
#pragma omp parallel
  {
    float row[4096];
#pragma omp for schedule(dynamic, 16)
    for (int64_t g = 0; g < total_pages; ++g) {
      int32_t b = 0;
      { int32_t lo = 0, hi = batch - 1;
        while (lo < hi) { int32_t mid = (lo + hi + 1) / 2; if (starts[mid] <= g) lo = mid; else hi = mid - 1; }
        b = lo; }
      int64_t lp = g - starts[b];
      uint64_t key = spmla_gen_stream_key(seed, tensor_id, (uint64_t)b);
      int64_t page = block_table[(int64_t)b * bt_stride + lp];
      for (int32_t s = 0; s < page_size; ++s) {
        int64_t t = lp * page_size + s;
        int tail = t >= lens[b];
        /* Slots past the context length hold either more draws of the same
           stream (plausible-looking garbage) or NaN, so that a reader that
           strays past the length is caught. */
        if (tail && poison_tail) {
          for (int32_t d = 0; d < dim; ++d) row[d] = NAN;
        } else {
          for (int32_t d = 0; d < dim; ++d) row[d] = (float)normal(key, (uint64_t)t * (uint64_t)dim + (uint64_t)d);
        }
        int64_t slot = page * page_size + s;
        if (tail && poison_tail && dtype == 2) {
          scale[slot] = NAN;
          memset((uint8_t*)out + slot * dim, 0x7F, (size_t)dim);
          continue;
        }
        if (dtype == 0) {
          memcpy((float*)out + slot * dim, row, sizeof(float) * (size_t)dim);
        } else if (dtype == 1) {
          uint16_t* o = (uint16_t*)out + slot * dim;
          for (int32_t d = 0; d < dim; ++d) o[d] = f32_to_bf16_rne(row[d]);
        } else {
          float amax = 0.f;
          for (int32_t d = 0; d < dim; ++d) { float a = fabsf(row[d]); if (a > amax) amax = a; }
          float sc = amax > 0.f ? amax / 448.0f : 1.0f;
          scale[slot] = sc;
          uint8_t* o = (uint8_t*)out + slot * dim;
          for (int32_t d = 0; d < dim; ++d) o[d] = encode_e4m3((double)row[d] / (double)sc);
        }
      }
    }
  }
  return 0;
}

/* Fill every element of a buffer of n elements with "garbage" normals of stream key (formats as above; fp8 gets codes only). */
void spmla_gen_fill_garbage(uint64_t key, int64_t n, int32_t dtype, void* out, int32_t poison) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    float v = poison ? NAN : (float)normal(key, (uint64_t)j);
    if (dtype == 0) ((float*)out)[j] = v;
    else if (dtype == 1) ((uint16_t*)out)[j] = f32_to_bf16_rne(v);
    else ((uint8_t*)out)[j] = encode_e4m3((double)v);
  }
}
