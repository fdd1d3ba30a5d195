// mla_paged_decode kernel: split-KV MLA decode over the selected tokens of the
// paged latent cache, both contractions on MFMA.
//
// Workgroup = (request b, split s, group of 64 query heads); 4 waves, 16 heads
// each.  The split's token list is resolved (index -> block table -> cache
// row, plus the FP8 scale) into LDS 1024 positions at a time, so row loads
// never wait on a table lookup.  Per 32-token tile:
//  1. Stage (all 256 threads): the tile's rows, loaded ahead into registers,
//     are widened (FP8 codes exactly to bf16, fp32 kept as is) and stored
//     once in LDS, row-major K[token][dim], in one of two buffers so that the
//     next tile is staged while this one is on the matrix cores.
//  2. Scores on MFMA as S^T[token x head] = K . Q^T: tokens on M, the wave's 16
//     heads on N, the query held in registers as the B operand for the whole
//     split.  The 16x16 result puts 4 tokens x 1 head in each lane.
//  3. Softmax weights per head against a fixed reference (see below) in fp32,
//     exp2 domain; a column max/sum needs only two xor shuffles.
//  4. Values on MFMA as O[head x dim] += P[head x token] . V[token x dim].  The
//     probabilities are already where the A operand wants them: the 8 values a
//     lane holds for its head (tokens 4g..4g+3 and 16+4g..16+4g+3) form its
//     k-slots, and the V operand comes from the same row-major tile through
//     gfx950's transposing LDS read with that token permutation.  The FP8
//     scale of token t multiplies its score and its probability.
// The output accumulator is 16 heads x d_latent fp32 per wave, in registers.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kDecThreads = 256;
constexpr int kTile = 32;
constexpr int kSeg = 512;   // token positions whose rows are resolved at once
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWg = 64;
constexpr float kHeadroom = 16.f;  // log2 headroom of the fixed softmax reference

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

template <class Op, int KDT, int KSTEPS, int NT>
__global__ __launch_bounds__(kDecThreads) void mla_decode_kernel(
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
  constexpr int DS = D + KPAD;        // K row stride (elements)
  constexpr int ROW_BYTES = D * Storage<KDT>::bytes;
  constexpr int CH_BYTES = 8 * Storage<KDT>::bytes;  // 8 elements per staging chunk
  constexpr int CH_DW = (CH_BYTES + 3) / 4;
  constexpr int NCH = D / 8;
  constexpr int CPT = (NCH + 15) / 16;  // chunks per staging thread (16 threads per row pair)
  static_assert(D % 8 == 0 && DC % 8 == 0 && DC <= D, "shape");

  __shared__ __attribute__((aligned(16))) E Kbuf[2][kTile * DS];
  __shared__ int32_t seg_row[kSeg];   // >= 0 cache row, -1 masked, -2 unreadable
  __shared__ float seg_scale[kSeg];
  __shared__ int redo_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int page_size = 1 << page_shift;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = logical % n_hg;
  const int s = (logical / n_hg) % num_splits;
  const int b = logical / (n_hg * num_splits);
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

  // Softmax with a fixed reference per head instead of a running max: the
  // reference of head r16 is the max of the first tile in which the head sees
  // a valid token (its accumulator is still zero then, so setting it is free);
  // later weights are exp2(z - m_ref) <= 2^kHeadroom unless a tile's max
  // exceeds m_ref by more than kHeadroom.  If that happens anywhere in the
  // workgroup the split is recomputed once with the true max as reference,
  // so the accumulator is never rescaled inside the loop.  Same result as the
  // running-max form: o and l share the reference, which cancels in o / l.
  f32x4 acc_o[NT];
  float m_ref = -INFINITY;   // reference (log2 domain) of head r16
  float m_true = -INFINITY;  // running true max of head r16
  float l_run = 0.f;         // sum of weights of head r16
  bool unreadable = false;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc_o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  l_run = 0.f;
  if (pass == 1) m_ref = m_true;
  bool over = false;
  if (tid == 0) redo_flag = 0;

  const int32_t* btb = bt + (int64_t)b * bt_stride;
  const int32_t* idxb = indices ? indices + (int64_t)b * k : nullptr;
  const int spair = tid >> 4;  // staging: token rows 2*spair, 2*spair+1 of the tile
  const int sj = tid & 15;     // staging: chunks sj, sj+16, ...
  uint32_t raw[CPT][2][CH_DW];
  bool raw_ok[2];

  // Issue the global loads of the tile at tile0.  Every lane issues the same
  // loads whatever its row (a masked row reads row 0, a spare chunk slot
  // re-reads the last chunk), so the compiler can count them and keep them in
  // flight across the tile's math; stage() zeroes what is masked.
  auto issue = [&](int64_t seg_begin, int64_t seg_end, int64_t tile0) __attribute__((always_inline)) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t p = tile0 + 2 * spair + rr;
      const int32_t row = p < seg_end ? seg_row[p - seg_begin] : -1;
      raw_ok[rr] = row >= 0;
      const uint8_t* src = kv + (int64_t)(row >= 0 ? row : 0) * ROW_BYTES;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = min(sj + 16 * i, NCH - 1);
        load_raw<CH_BYTES>(src + c * CH_BYTES, raw[i][rr]);
      }
    }
  };
  // Widen the staged registers into the LDS tile (row-major K[token][dim]; the
  // value operand is read from the same rows with transposing LDS reads).
  auto stage = [&](E* __restrict__ Kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = sj + 16 * i;
      if (c < NCH) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
          for (int w = 0; w < CH_DW; ++w) raw[i][rr][w] = raw_ok[rr] ? raw[i][rr][w] : 0u;
          E* kd = Kt + (2 * spair + rr) * DS + c * 8;
          if constexpr (kBf) {
            bf16x8 f;
            raw_to_frags<OpBF16, KDT, 1>(raw[i][rr], &f);
            *reinterpret_cast<bf16x8*>(kd) = f;
          } else {
            float v8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = raw_elem_f32<KDT>(raw[i][rr], e);
            *reinterpret_cast<float4*>(kd) = make_float4(v8[0], v8[1], v8[2], v8[3]);
            *reinterpret_cast<float4*>(kd + 4) = make_float4(v8[4], v8[5], v8[6], v8[7]);
          }
        }
      }
    }
  };

  for (int64_t seg = p_begin; seg < p_end; seg += kSeg) {
    const int64_t seg_end = min(p_end, seg + kSeg);
    __syncthreads();  // previous segment's tiles are done with seg_row / LDS
    // ---- resolve the segment's rows (index -> page -> row) once
    for (int64_t p = seg + tid; p < seg_end; p += kDecThreads) {
      const int64_t t = idxb ? (int64_t)idxb[p] : p;
      int32_t row = -1;
      float sc = 1.f;
      if (t == -1) {
        row = -1;
      } else if (t < -1 || t >= L) {
        row = -2;
        if (status) atomicOr(status + b, kBadIndex);
      } else {
        const int32_t page = btb[t >> page_shift];
        if (page < 0 || page >= num_pages) {
          row = -2;
          if (status) atomicOr(status + b, kBadPage);
        } else {
          row = (int32_t)(((int64_t)page << page_shift) + (t & (page_size - 1)));
          if (KDT == kFP8) sc = kv_scale[row];
        }
      }
      seg_row[p - seg] = row;
      seg_scale[p - seg] = sc;
    }
    __syncthreads();
    issue(seg, seg_end, seg);
    stage(Kbuf[0]);
    issue(seg, seg_end, seg + kTile);
    __syncthreads();
    int buf = 0;
    for (int64_t p0 = seg; p0 < seg_end; p0 += kTile, buf ^= 1) {
      const E* Kt = Kbuf[buf];
      {
        const int64_t tb = p0 - seg;  // tile base within the segment
        // ---- scores S^T[token][head] for the tile's two 16-token halves
        f32x4 sc[2], sc2[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          sc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
          sc2[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // K fragments are read from LDS one k-step ahead of the MFMAs that use
        // them (two fragments per k-step, double-buffered), so LDS latency
        // hides behind the matrix cores even with one wave per SIMD.
        typename Op::frag ka[2][2];
        auto kfrag = [&](int st, int m) __attribute__((always_inline)) -> typename Op::frag {
          const E* krow = Kt + (m * 16 + r16) * DS + g * KPL + st * 4 * KPL;
          if constexpr (kBf) {
            return *reinterpret_cast<const bf16x8*>(krow);
          } else {
            return *krow;
          }
        };
        ka[0][0] = kfrag(0, 0);
        ka[0][1] = kfrag(0, 1);
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
          const int cur = st & 1;
          if (st + 1 < KSTEPS) {
            ka[cur ^ 1][0] = kfrag(st + 1, 0);
            ka[cur ^ 1][1] = kfrag(st + 1, 1);
          }
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            if (st & 1) sc2[m] = Op::mma(ka[cur][m], qb[st], sc2[m]);
            else sc[m] = Op::mma(ka[cur][m], qb[st], sc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) sc[m] += sc2[m];
        // ---- online softmax (log2 domain) for head r16
        float z[2][4], tsc[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t pp = tb + m * 16 + g * 4 + i;
            const bool inside = p0 + m * 16 + g * 4 + i < seg_end;
            const int32_t row = inside ? seg_row[pp] : -1;
            tsc[m][i] = inside ? seg_scale[pp] : 1.f;
            unreadable |= (row == -2);
            float v = sc[m][i] * (sm_scale_log2 * tsc[m][i]);
            v = row >= 0 ? v : -INFINITY;
            z[m][i] = v;
            mx = fmaxf(mx, v);
          }
        }
        mx = wave_max_xor16_32(mx);
        m_true = fmaxf(m_true, mx);
        if (m_ref == -INFINITY) m_ref = mx;  // first valid tile of this head (accumulator still zero)
        over |= mx > m_ref + kHeadroom;
        float psum = 0.f;
        float pv[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pp = m_ref == -INFINITY ? 0.f : exp2f(z[m][i] - m_ref);
            psum += pp;
            pv[m][i] = pp * tsc[m][i];
          }
        }
        psum = wave_sum_xor16_32(psum);
        l_run += psum;
        // ---- O += P . V, with V read straight from the row-major tile.
        if constexpr (kBf) {
          bf16x8 pa = {(__bf16)pv[0][0], (__bf16)pv[0][1], (__bf16)pv[0][2], (__bf16)pv[0][3],
                       (__bf16)pv[1][0], (__bf16)pv[1][1], (__bf16)pv[1][2], (__bf16)pv[1][3]};
          // A transposing LDS read hands lane i of each 16-lane group column
          // i % 4 of rows {i/4, 4 + i/4, 8 + i/4, 12 + i/4} of the 16 x 4
          // matrix of 16-bit values its group's lanes point at.  Source lane j
          // of group g points at 4 consecutive dims of token 4g + j/4 (and
          // 16 + 4g + j/4), so lane (dim r16, group g) receives that dim for
          // tokens 4g..4g+3 (and 16+4g..16+4g+3): the k-slots the softmax
          // weights already sit in.
          typedef __attribute__((address_space(3))) v4bf16_t lds_v4bf16;
          const E* vsrc = Kt + (g * 4 + (r16 >> 2)) * DS + 4 * (r16 & 3);
          auto vfrag = [&](int nt) __attribute__((always_inline)) -> bf16x8 {
            const v4bf16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(vsrc + nt * 16));
            const v4bf16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(vsrc + 16 * DS + nt * 16));
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          };
          bf16x8 vb[2];
          vb[0] = vfrag(0);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (nt + 1 < NT) vb[(nt + 1) & 1] = vfrag(nt + 1);
            acc_o[nt] = Op::mma(pa, vb[nt & 1], acc_o[nt]);
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc_o[nt] = Op::mma(pv[m][i], Kt[(m * 16 + g * 4 + i) * DS + nt * 16 + r16], acc_o[nt]);
            }
          }
        }
      }
      // Stage the next tile into the other buffer while this tile's MFMAs
      // drain, then send the loads of the tile after it.
      if (p0 + kTile < seg_end) {
        stage(Kbuf[buf ^ 1]);
        issue(seg, seg_end, p0 + 2 * kTile);
      }
      __syncthreads();
    }
  }

  // Recompute the split once if any head of the workgroup outgrew its reference.
  if (__any(over) && (tid & 63) == 0) atomicOr(&redo_flag, 1);
  __syncthreads();
  const bool redo = redo_flag != 0;
  __syncthreads();
  if (!redo) break;
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
    float lse = l_run > 0.f ? (m_ref + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
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
