// mla_paged_decode kernel: split-KV MLA decode over the selected tokens of the
// paged latent cache, both contractions on MFMA.
//
// Workgroup = (request b, split s, group of 64 query heads); 4 waves, 16 heads
// each.  Per 32-token tile:
//  1. Stage (all 256 threads): resolve each token through the block table,
//     load its row (FP8 codes widened exactly to bf16 on the way, fp32 kept
//     as is), store it twice in LDS -- row-major K[token][dim] for the score
//     contraction and transposed V^T[dim][token] (first d_latent dims) for the
//     value contraction.  The FP8 per-token scale is kept apart.
//  2. Scores on MFMA as S^T[token x head] = K . Q^T: tokens on M, the wave's 16
//     heads on N, the query held in registers as the B operand for the whole
//     split.  The 16x16 result puts 4 tokens x 1 head in each lane.
//  3. Online softmax per head (running max m, running sum l) in fp32, exp2
//     domain; a column max/sum needs only two xor shuffles.
//  4. Values on MFMA as O[head x dim] += P[head x token] . V[token x dim].  The
//     probabilities are already where the A operand wants them: the 8 values a
//     lane holds for its head (tokens 4g..4g+3 and 16+4g..16+4g+3) form its
//     k-slots, and V^T is read from LDS with the same token permutation.  The
//     FP8 scale of token t multiplies its score and its probability.
// The output accumulator is 16 heads x d_latent fp32 per wave, in registers.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kDecThreads = 256;
constexpr int kTile = 32;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWg = 64;

template <class Op, int KDT, int KSTEPS, int NT>
__global__ __launch_bounds__(kDecThreads, 2) void mla_decode_kernel(
    const void* __restrict__ q, const uint8_t* __restrict__ kv, const float* __restrict__ kv_scale,
    int32_t num_pages, int32_t page_shift, const int32_t* __restrict__ bt, int32_t bt_stride,
    const int32_t* __restrict__ lens, int64_t max_len, const int32_t* __restrict__ indices, int32_t k,
    int32_t n_heads, float sm_scale_log2, int32_t num_splits, int32_t n_hg, float* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ status) {
  typedef typename Op::elem E;
  constexpr int KPL = Op::KPL;
  constexpr int D = KSTEPS * 4 * KPL;
  constexpr int DC = NT * 16;
  constexpr bool kBf = std::is_same<Op, OpBF16>::value;
  constexpr int KPAD = kBf ? 8 : 4;
  constexpr int VPAD = kBf ? 8 : 4;
  constexpr int DS = D + KPAD;        // K row stride (elements)
  constexpr int VS = kTile + VPAD;    // V^T row stride (elements)
  constexpr int ROW_BYTES = D * Storage<KDT>::bytes;
  constexpr int CH_BYTES = 8 * Storage<KDT>::bytes;  // 8 elements per staging chunk
  constexpr int NCH = D / 8;
  static_assert(D % 8 == 0 && DC % 8 == 0 && DC <= D, "shape");

  __shared__ __attribute__((aligned(16))) E Kt[kTile * DS];
  __shared__ __attribute__((aligned(16))) E Vt[DC * VS];
  __shared__ float tok_scale[kTile];
  __shared__ int tok_state[kTile];  // 0 valid, 1 masked, 2 unreadable (bad page / index)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int page_size = 1 << page_shift;

  const int hg = blockIdx.x % n_hg;
  const int s = (blockIdx.x / n_hg) % num_splits;
  const int b = blockIdx.x / (n_hg * num_splits);
  const int head0 = hg * kHeadsPerWg + wv * kHeadsPerWave;  // first head of this wave
  const bool wave_active = head0 < n_heads;
  const float kNaN = __uint_as_float(0x7FC00000u);

  auto out_o = [&](int h, int dim) -> float* {
    return o_part + ((((int64_t)b * num_splits + s) * n_heads + h) * DC + dim);
  };
  auto out_lse = [&](int h) -> float* { return lse_part + (((int64_t)b * num_splits + s) * n_heads + h); };

  const int32_t L = lens[b];
  if (L < 0 || (int64_t)L > max_len || (int64_t)L > (int64_t)bt_stride * page_size) {
    if (tid == 0 && status) atomicOr(status + b, kBadLen);
    if (wave_active) {
      for (int i = lane; i < kHeadsPerWave * DC; i += 64) {
        const int h = head0 + i / DC;
        if (h < n_heads) *out_o(h, i % DC) = kNaN;
      }
      if (lane < kHeadsPerWave && head0 + lane < n_heads) *out_lse(head0 + lane) = kNaN;
    }
    return;
  }
  const int64_t n = indices ? (int64_t)k : (int64_t)L;
  const int64_t per = ((n + num_splits - 1) / num_splits + kTile - 1) / kTile * kTile;
  const int64_t p_begin = (int64_t)s * per;
  const int64_t p_end = min(n, p_begin + per);

  // Query fragments: B operand of S^T = K . Q^T (column = head r16).
  typename Op::frag qb[KSTEPS];
  {
    const int h = head0 + r16;
    if (wave_active && h < n_heads) {
      const E* qh = reinterpret_cast<const E*>(q) + ((int64_t)b * n_heads + h) * D;
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        if constexpr (kBf) {
          uint4 v = *reinterpret_cast<const uint4*>(qh + st * 4 * KPL + g * KPL);
          qb[st] = __builtin_bit_cast(bf16x8, v);
        } else {
          qb[st] = qh[st * 4 * KPL + g * KPL];
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) qb[st] = zero_frag<Op>();
    }
  }

  f32x4 acc_o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc_o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head r16
  float l_run = 0.f;        // running sum of head r16
  bool unreadable = false;

  const int32_t* btb = bt + (int64_t)b * bt_stride;
  const int32_t* idxb = indices ? indices + (int64_t)b * k : nullptr;
  const int srow = tid >> 3;  // staging token slot
  const int sj = tid & 7;     // staging chunk lane

  for (int64_t p0 = p_begin; p0 < p_end; p0 += kTile) {
    // ---- 1. stage the tile
    {
      const int64_t p = p0 + srow;
      int state = 1;
      int64_t row = 0;
      if (p < p_end) {
        const int64_t t = idxb ? (int64_t)idxb[p] : p;
        if (t == -1) {
          state = 1;
        } else if (t < -1 || t >= L) {
          state = 2;
          if (sj == 0 && status) atomicOr(status + b, kBadIndex);
        } else {
          const int32_t page = btb[t >> page_shift];
          if (page < 0 || page >= num_pages) {
            state = 2;
            if (sj == 0 && status) atomicOr(status + b, kBadPage);
          } else {
            state = 0;
            row = ((int64_t)page << page_shift) + (t & (page_size - 1));
          }
        }
      }
      if (sj == 0) {
        tok_state[srow] = state;
        tok_scale[srow] = (KDT == kFP8 && state == 0) ? kv_scale[row] : 1.f;
      }
      const uint8_t* src = kv + row * ROW_BYTES;
      for (int c = sj; c < NCH; c += 8) {
        E v8[8];
        if (state == 0) {
          uint32_t raw[(CH_BYTES + 3) / 4];
          load_raw<CH_BYTES>(src + c * CH_BYTES, raw);
          if constexpr (kBf) {
            bf16x8 f;
            raw_to_frags<OpBF16, KDT, 1>(raw, &f);
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = f[e];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = raw_elem_f32<KDT>(raw, e);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = (E)0.f;
        }
        E* kd = Kt + srow * DS + c * 8;
        if constexpr (kBf) {
          *reinterpret_cast<bf16x8*>(kd) = bf16x8{v8[0], v8[1], v8[2], v8[3], v8[4], v8[5], v8[6], v8[7]};
        } else {
          *reinterpret_cast<float4*>(kd) = make_float4(v8[0], v8[1], v8[2], v8[3]);
          *reinterpret_cast<float4*>(kd + 4) = make_float4(v8[4], v8[5], v8[6], v8[7]);
        }
        if (c * 8 < DC) {
#pragma unroll
          for (int e = 0; e < 8; ++e) Vt[(c * 8 + e) * VS + srow] = v8[e];
        }
      }
    }
    __syncthreads();

    if (wave_active) {
      // ---- 2. scores S^T[token][head] for the tile's two 16-token halves
      f32x4 sc[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        sc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        const E* krow = Kt + (m * 16 + r16) * DS + g * KPL;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
          typename Op::frag a;
          if constexpr (kBf) {
            a = *reinterpret_cast<const bf16x8*>(krow + st * 4 * KPL);
          } else {
            a = krow[st * 4 * KPL];
          }
          sc[m] = Op::mma(a, qb[st], sc[m]);
        }
      }
      // ---- 3. online softmax (log2 domain) for head r16
      float z[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = m * 16 + g * 4 + i;
          const int st = tok_state[tk];
          unreadable |= (st == 2);
          float v = sc[m][i] * (sm_scale_log2 * tok_scale[tk]);
          v = st == 0 ? v : -INFINITY;
          z[m][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = wave_max_xor16_32(mx);
      const float m_new = fmaxf(m_run, mx);
      float alpha = 1.f;
      float psum = 0.f;
      float pv[2][4];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[m][i] = 0.f;
      } else {
        alpha = exp2f(m_run - m_new);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pp = exp2f(z[m][i] - m_new);
            psum += pp;
            pv[m][i] = pp * tok_scale[m * 16 + g * 4 + i];
          }
        }
      }
      psum = wave_sum_xor16_32(psum);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // Rescale the accumulator rows (heads 4g+i) by their heads' alpha.
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, g * 4 + i);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[nt][i] *= ai[i];
      }
      // ---- 4. O += P . V
      if constexpr (kBf) {
        bf16x8 pa = {(__bf16)pv[0][0], (__bf16)pv[0][1], (__bf16)pv[0][2], (__bf16)pv[0][3],
                     (__bf16)pv[1][0], (__bf16)pv[1][1], (__bf16)pv[1][2], (__bf16)pv[1][3]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const E* vrow = Vt + (nt * 16 + r16) * VS;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + g * 4);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + g * 4);
          const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          acc_o[nt] = Op::mma(pa, vb, acc_o[nt]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const E* vrow = Vt + (nt * 16 + r16) * VS;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_o[nt] = Op::mma(pv[m][i], vrow[m * 16 + g * 4 + i], acc_o[nt]);
          }
        }
      }
    }
    __syncthreads();
  }

  if (!wave_active) return;
  // ---- finalize: o = O / l, lse = (m + log2 l) * ln 2
  const bool bad = __any(unreadable);
  float li[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) li[i] = __shfl(l_run, g * 4 + i);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + g * 4 + i;
      if (h < n_heads) {
        float v = li[i] > 0.f ? acc_o[nt][i] / li[i] : 0.f;
        if (bad) v = kNaN;
        *out_o(h, nt * 16 + r16) = v;
      }
    }
  }
  if (g == 0 && head0 + r16 < n_heads) {
    float lse = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
    if (bad) lse = kNaN;
    *out_lse(head0 + r16) = lse;
  }
}

template <class Op, int KDT, int KSTEPS, int NT>
static int launch_one(const DecodeArgs& a, hipStream_t stream) {
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  const int n_hg = (a.n_heads + kHeadsPerWg - 1) / kHeadsPerWg;
  const int64_t grid = (int64_t)a.batch * a.num_splits * n_hg;
  if (grid == 0) return 0;
  if (grid > 0x7FFFFFFF) return -2;
  const float sm_log2 = a.sm_scale * 1.44269504088896340736f;
  hipLaunchKernelGGL((mla_decode_kernel<Op, KDT, KSTEPS, NT>), dim3((unsigned)grid), dim3(kDecThreads), 0, stream,
                     a.q, reinterpret_cast<const uint8_t*>(a.kv), a.kv_scale, a.num_pages, page_shift, a.bt,
                     a.bt_stride, a.lens, a.max_len, a.indices, a.k, a.n_heads, sm_log2, a.num_splits, n_hg,
                     a.o_part, a.lse_part, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int D = a.d_latent + a.d_rope;
  if (a.q_dtype == kBF16 && D == 576 && a.d_latent == 512) {
    if (a.kv_dtype == kBF16) return launch_one<OpBF16, kBF16, 18, 32>(a, s);
    if (a.kv_dtype == kFP8) return launch_one<OpBF16, kFP8, 18, 32>(a, s);
    return -2;
  }
  if (a.q_dtype == kF32 && D == 80 && a.d_latent == 64) {
    if (a.kv_dtype == kF32) return launch_one<OpF32, kF32, 20, 4>(a, s);
    if (a.kv_dtype == kBF16) return launch_one<OpF32, kBF16, 20, 4>(a, s);
    if (a.kv_dtype == kFP8) return launch_one<OpF32, kFP8, 20, 4>(a, s);
    return -2;
  }
  return -2;
}

}  // namespace spmla
