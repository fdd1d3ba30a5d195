// mla_paged_decode for the shapes the tuned kernels do not take: any latent
// and rope widths that are multiples of 8 (latent + rope <= 1024), fp32 or
// bf16 queries, fp32 / bf16 / FP8 caches.  Split-KV MLA decode with the
// exact online softmax (running max and sum, the accumulator rescaled when
// the max grows), in fp32 on the vector units: it covers the shapes of the
// interface rather than a workload, so it is plain rather than fast.
//
// Workgroup = (request b, split s, group of 16 heads), 256 threads.  The
// group's query sits in LDS as fp32.  The split's positions go 16 at a time:
// threads 0..15 resolve a position to its cache row (index -> block table ->
// row, with the same checks and status bits as the other decode kernels),
// the 16 rows are widened to fp32 into LDS, thread (h, t) (h = tid / 16,
// t = tid % 16) forms the logit of head h for token t, each head's 16
// threads (one 16-lane group of a wave) update that head's running max and
// sum with shuffles, and thread (h, j) then adds the tile's weighted value
// rows to output dims j, j + 16, ... of head h.
#include "common.h"
#include "launch.h"

namespace spmla {
namespace {

constexpr int kGThreads = 256;
constexpr int kGHeads = 16;
constexpr int kGTok = 16;
constexpr int kGMaxD = kDecodeGenericMaxDim;
constexpr int kGMaxOut = kGMaxD / 16;  // output dims per thread at most

__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <int QDT, int KDT>
__global__ __launch_bounds__(kGThreads) void mla_decode_generic_kernel(
    const void* __restrict__ q, const uint8_t* __restrict__ kv, const float* __restrict__ kv_scale, int32_t num_pages,
    int32_t page_shift, const int32_t* __restrict__ bt, int32_t bt_stride, const int32_t* __restrict__ lens,
    int64_t max_len, const int32_t* __restrict__ indices, int32_t k, int32_t n_heads, int32_t d_latent, int32_t d_rope,
    float sm_scale, int32_t num_splits, int32_t split_tok, int32_t n_hg, float* __restrict__ o_part,
    float* __restrict__ lse_part,
    int32_t* __restrict__ status) {
  extern __shared__ __attribute__((aligned(16))) float gsm[];
  const int D = d_latent + d_rope;
  const int DS = D + 1;                   // LDS row stride (odd: heads read at one dim fall on distinct banks)
  float* qs = gsm;                        // [16][DS] the group's query
  float* kt = qs + kGHeads * DS;          // [16][DS] the tile's rows
  float* ps = kt + kGTok * DS;            // [16][16] weights
  float* rsc = ps + kGHeads * kGTok;      // [16] rescale of each head's accumulator
  int32_t* trow = reinterpret_cast<int32_t*>(rsc + kGHeads);  // [16] cache row of each tile token, -1 masked
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int hi = tid >> 4, ti = tid & 15;  // (head, token) for the logits; (head, dim lane) for the values
  const int hg = (int)(blockIdx.x % n_hg);
  const int s = (int)((blockIdx.x / n_hg) % num_splits);
  const int b = (int)(blockIdx.x / (n_hg * num_splits));
  const int h = hg * kGHeads + hi;
  const int page_size = 1 << page_shift;
  const float kNaN = __uint_as_float(0x7FC00000u);
  auto out_o = [&](int hh, int dim) -> float* {
    return o_part + ((((int64_t)b * num_splits + s) * n_heads + hh) * d_latent + dim);
  };
  auto out_lse = [&](int hh) -> float* { return lse_part + (((int64_t)b * num_splits + s) * n_heads + hh); };

  const int32_t L = lens[b];
  if (L < 0 || (int64_t)L > max_len || (int64_t)L > (int64_t)bt_stride * page_size) {
    if (tid == 0 && status) atomicOr(status + b, kBadLen);
    for (int i = tid; i < kGHeads * d_latent; i += kGThreads) {
      const int hh = hg * kGHeads + i / d_latent;
      if (hh < n_heads) *out_o(hh, i % d_latent) = kNaN;
    }
    if (tid < kGHeads && hg * kGHeads + tid < n_heads) *out_lse(hg * kGHeads + tid) = kNaN;
    return;
  }
  // The group's query, widened to fp32 (heads past the last one: zeros).
  for (int i = tid; i < kGHeads * D; i += kGThreads) {
    const int hh = hg * kGHeads + i / D, d = i % D;
    float v = 0.f;
    if (hh < n_heads) {
      const int64_t e = ((int64_t)b * n_heads + hh) * D + d;
      v = QDT == kF32 ? reinterpret_cast<const float*>(q)[e]
                      : bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q)[e]);
    }
    qs[(i / D) * DS + d] = v;
  }
  if (tid == 0) bad_flag = 0;

  const bool sparse = indices != nullptr;
  const int64_t n = sparse ? (int64_t)k : (int64_t)L;
  const int64_t per = split_tok > 0 ? (int64_t)split_tok : ((n + num_splits - 1) / num_splits + 31) / 32 * 32;
  const int64_t p_begin = (int64_t)s * per;
  const int64_t p_end = split_tok > 0 && s == num_splits - 1 ? n : min(n, p_begin + per);
  if (split_tok > 0 && p_begin >= p_end) {  // past the request's last token: only lse -inf
    if (tid < kGHeads && hg * kGHeads + tid < n_heads) *out_lse(hg * kGHeads + tid) = -INFINITY;
    return;
  }
  const int32_t* btb = bt + (int64_t)b * bt_stride;
  const int n_out = (d_latent - ti + 15) / 16;  // output dims of this thread: ti, ti + 16, ...

  float m_run = -INFINITY, l_run = 0.f;
  float o[kGMaxOut];
#pragma unroll
  for (int c = 0; c < kGMaxOut; ++c) o[c] = 0.f;
  __syncthreads();

  for (int64_t p0 = p_begin; p0 < p_end; p0 += kGTok) {
    // Resolve the tile's positions.
    if (tid < kGTok) {
      const int64_t p = p0 + tid;
      int32_t row = -1;
      if (p < p_end) {
        const int64_t t = sparse ? (int64_t)indices[(int64_t)b * k + p] : p;
        if (t < -1 || t >= L) {
          bad_flag = 1;
          if (status) atomicOr(status + b, kBadIndex);
        } else if (t >= 0) {
          const int32_t page = btb[t >> page_shift];
          if (page < 0 || page >= num_pages) {
            bad_flag = 1;
            if (status) atomicOr(status + b, kBadPage);
          } else {
            row = (int32_t)(((int64_t)page << page_shift) + (t & (page_size - 1)));
          }
        }
      }
      trow[tid] = row;
    }
    __syncthreads();
    // The tile's rows, widened to fp32 (masked tokens: zeros).
    for (int i = tid; i < kGTok * D; i += kGThreads) {
      const int tt = i / D, d = i % D;
      const int32_t row = trow[tt];
      float v = 0.f;
      if (row >= 0) {
        const int64_t e = (int64_t)row * D + d;
        if constexpr (KDT == kF32) {
          v = reinterpret_cast<const float*>(kv)[e];
        } else if constexpr (KDT == kBF16) {
          v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(kv)[e]);
        } else {
          const uint32_t word = kv[e];
          v = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false)[0] * kv_scale[row];
        }
      }
      kt[tt * DS + d] = v;
    }
    __syncthreads();
    // Logit of head hi for token ti, then the head's running max and sum.
    float z = 0.f;
    for (int d = 0; d < D; ++d) z = __builtin_fmaf(qs[hi * DS + d], kt[ti * DS + d], z);
    z = trow[ti] >= 0 ? z * sm_scale : -INFINITY;
    const float m_new = fmaxf(m_run, max16(z));
    const float pz = m_new == -INFINITY ? 0.f : expf(z - m_new);
    const float scale = m_run == -INFINITY ? 0.f : expf(m_run - m_new);
    l_run = l_run * scale + sum16(pz);
    m_run = m_new;
    ps[hi * kGTok + ti] = pz;
    if (ti == 0) rsc[hi] = scale;
    __syncthreads();
    // Output dims ti, ti + 16, ... of head hi.
    const float sc = rsc[hi];
#pragma unroll
    for (int c = 0; c < kGMaxOut; ++c) {
      if (c < n_out) {
        const int j = ti + 16 * c;
        float acc = o[c] * sc;
#pragma unroll
        for (int tt = 0; tt < kGTok; ++tt) acc = __builtin_fmaf(ps[hi * kGTok + tt], kt[tt * DS + j], acc);
        o[c] = acc;
      }
    }
    __syncthreads();  // the next tile rewrites kt, ps and rsc
  }
  const bool bad = bad_flag != 0;
  if (h < n_heads) {
    const float inv = bad ? kNaN : (l_run > 0.f ? 1.f / l_run : 0.f);
#pragma unroll
    for (int c = 0; c < kGMaxOut; ++c)
      if (c < n_out) *out_o(h, ti + 16 * c) = o[c] * inv;
    if (ti == 0) *out_lse(h) = bad ? kNaN : (l_run > 0.f ? m_run + logf(l_run) : -INFINITY);
  }
}

template <int QDT, int KDT>
int launch_generic_t(const DecodeArgs& a, hipStream_t stream) {
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  const int n_hg = (a.n_heads + kGHeads - 1) / kGHeads;
  const int64_t grid = (int64_t)a.batch * a.num_splits * n_hg;
  if (grid == 0) return 0;
  if (grid > 0x7FFFFFFF) return -2;
  const int D = a.d_latent + a.d_rope;
  const size_t lds = ((size_t)(kGHeads + kGTok) * (D + 1) + kGHeads * kGTok + kGHeads) * 4 + kGTok * 4;
  // LDS past the default 64 KiB of dynamic shared memory needs the kernel's
  // limit raised (gfx950 has 160 KiB per workgroup).
  if (lds > 65536 && hipFuncSetAttribute(reinterpret_cast<const void*>(&mla_decode_generic_kernel<QDT, KDT>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return -3;
  hipLaunchKernelGGL((mla_decode_generic_kernel<QDT, KDT>), dim3((unsigned)grid), dim3(kGThreads), lds, stream, a.q,
                     reinterpret_cast<const uint8_t*>(a.kv), a.kv_scale, a.num_pages, page_shift, a.bt, a.bt_stride,
                     a.lens, a.max_len, a.indices, a.k, a.n_heads, a.d_latent, a.d_rope, a.sm_scale, a.num_splits, a.split_tokens, n_hg,
                     a.o_part, a.lse_part, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace

int launch_decode_generic(const DecodeArgs& a, hipStream_t stream) {
  if (!decode_generic_shape(a.q_dtype, a.kv_dtype, a.d_latent, a.d_rope)) return -2;
  if (a.q_dtype == kF32) {
    if (a.kv_dtype == kF32) return launch_generic_t<kF32, kF32>(a, stream);
    if (a.kv_dtype == kBF16) return launch_generic_t<kF32, kBF16>(a, stream);
    return launch_generic_t<kF32, kFP8>(a, stream);
  }
  if (a.kv_dtype == kBF16) return launch_generic_t<kBF16, kBF16>(a, stream);
  return launch_generic_t<kBF16, kFP8>(a, stream);
}

}  // namespace spmla
