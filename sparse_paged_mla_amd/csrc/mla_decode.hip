// mla_paged_decode kernels: split-KV MLA decode over the selected tokens of
// the paged latent cache, both contractions on MFMA.  mla_decode_kernel
// (the fp32 query with 64 + 16 dims, over fp32, bf16 or FP8 caches) widens
// each tile once into LDS; a bf16 query with 576-dim rows goes to the
// role-specialised kernels of mla_decode_f8.hip (FP8 cache, the tile kept in
// LDS as codes) and mla_decode_bf16.hip (bf16 cache).
//
// Workgroup = (request b, split s, group of 64 query heads); 8 waves.  A pair
// of waves shares 16 heads: each wave of the pair contracts half of the row
// dims for the scores and accumulates half of the output dims, so per wave
// the query (half of 16 x 576 bf16) and the accumulator (16 x 256 fp32) fit
// in half the registers and two waves run per SIMD.  The split's token list is
// resolved (index -> block table -> cache row, plus the FP8 scale) into LDS
// 1024 positions at a time, so row loads never wait on a table lookup.
// Per 32-token tile:
//  1. Stage (all 512 threads): the tile's rows, loaded ahead into registers,
//     are widened (FP8 codes exactly to bf16, fp32 kept as is) and stored
//     once in LDS, row-major K[token][dim].  Three buffers rotate: a tile is
//     staged two tiles ahead of the one on the matrix cores, so each tile
//     needs one barrier.
//  2. Scores on MFMA as S^T[token x head] = K . Q^T over the wave's half of
//     the dims: tokens on M, the 16 heads on N, the query half in registers
//     (B operand).  The two halves are exchanged through LDS and added by
//     both waves, which therefore hold identical scores.
//  3. Softmax weights per head against a fixed reference (below) in fp32,
//     exp2 domain; no cross-lane reduction in the steady state.
//  4. Values on MFMA as O[head x dim] += P[head x token] . V[token x dim] for
//     the wave's half of the output dims.  The weights already sit where the
//     A operand wants them (the 8 values a lane holds for its head, tokens
//     4g..4g+3 and 16+4g..16+4g+3, are its k-slots), and the V operand comes
//     from the same row-major tile through gfx950's transposing LDS read with
//     that token permutation.  The FP8 scale of token t multiplies its score
//     and its weight.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kDecThreads = 512;   // 8 waves: 4 head groups x 2 dim halves
constexpr int kTile = 32;          // tokens per tile
constexpr int kBufs = 3;           // LDS tile buffers (one barrier per tile)
constexpr int kSeg = 1024;         // token positions whose rows are resolved at once
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
    int32_t n_heads, float sm_scale_log2, int32_t num_splits, int32_t split_tok, int32_t n_hg,
    float* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ status) {
  typedef typename Op::elem E;
  constexpr int KPL = Op::KPL;
  constexpr int D = KSTEPS * 4 * KPL;
  constexpr int DC = NT * 16;
  constexpr int KS_H = KSTEPS / 2;     // score k-steps per dim half
  constexpr int NT_H = NT / 2;         // output 16-dim tiles per half
  constexpr bool kBf = std::is_same<Op, OpBF16>::value;
  // LDS row stride (elements).  bf16 rows are padded to an odd multiple of
  // 32 bytes modulo 256, and rows 8..15 of every 16 swap the two 16-byte
  // chunks of each 32-byte pair (sw() below): with that, the 16 rows a score
  // fragment read touches and the 8 rows of a transposing value read each
  // fall on distinct LDS banks.
  constexpr int DS = kBf ? D + 16 : D + 4;
  static_assert(!kBf || ((DS * 2 / 32) % 2 == 1 && (DS * 2) % 32 == 0), "bf16 row stride");
  constexpr int ROW_BYTES = D * Storage<KDT>::bytes;
  constexpr int CH_BYTES = 8 * Storage<KDT>::bytes;  // 8 elements per staging chunk
  constexpr int CH_DW = (CH_BYTES + 3) / 4;
  constexpr int NCH = D / 8;
  constexpr int CPT = (NCH + 31) / 32;  // chunks per staging thread (32 threads per row pair)
  static_assert(D % 8 == 0 && DC % 8 == 0 && DC <= D && KSTEPS % 2 == 0 && NT % 2 == 0, "shape");

  __shared__ __attribute__((aligned(16))) E Kbuf[kBufs][kTile * DS];
  __shared__ __attribute__((aligned(16))) int32_t seg_row[kSeg];   // cache row, or -1 when masked
  __shared__ __attribute__((aligned(16))) float seg_zsc[kSeg];     // softmax scale (log2) x FP8 scale
  __shared__ __attribute__((aligned(16))) float seg_tsc[kSeg];     // FP8 scale of the row
  __shared__ __attribute__((aligned(16))) float seg_bias[kSeg];    // 0, or -inf when masked
  __shared__ f32x4 sx[2][kDecThreads / 64][2][64];  // score halves exchanged between the waves of a pair
  __shared__ int redo_flag;
  __shared__ int bad_flag;  // some selected token could not be read

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int half = wv & 1;   // dim half of this wave
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int page_size = 1 << page_shift;
  // Element offset of 16-byte chunk c of tile row `row`.
  auto sw = [](int row, int c) -> int { return row * DS + (kBf ? (c ^ ((row >> 3) & 1)) : c) * 8; };

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = logical % n_hg;
  const int s = (logical / n_hg) % num_splits;
  const int b = logical / (n_hg * num_splits);
  const int head0 = hg * kHeadsPerWg + (wv >> 1) * kHeadsPerWave;  // first head of this wave
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
      for (int i = lane; i < kHeadsPerWave * (DC / 2); i += 64) {
        const int h = head0 + i / (DC / 2);
        if (h < n_heads) *out_o(h, half * (DC / 2) + i % (DC / 2)) = kNaN;
      }
      if (half == 0 && lane < kHeadsPerWave && head0 + lane < n_heads) *out_lse(head0 + lane) = kNaN;
    }
    return;
  }
  const int64_t n = indices ? (int64_t)k : (int64_t)L;
  const int64_t per = split_tok > 0 ? (int64_t)split_tok : ((n + num_splits - 1) / num_splits + kTile - 1) / kTile * kTile;
  const int64_t p_begin = (int64_t)s * per;
  const int64_t p_end = split_tok > 0 && s == num_splits - 1 ? n : min(n, p_begin + per);
  if (split_tok > 0 && p_begin >= p_end) {  // past the request's last token: only lse -inf
    if (wave_active && half == 0 && lane < kHeadsPerWave && head0 + lane < n_heads) *out_lse(head0 + lane) = -INFINITY;
    return;
  }

  // Query fragments for this wave's half of the dims: B operand of S^T = K . Q^T
  // (column = head r16).
  typename Op::frag qb[KS_H];
  {
    const int h = head0 + r16;
    if (wave_active && h < n_heads) {
      const E* qh = reinterpret_cast<const E*>(q) + ((int64_t)b * n_heads + h) * D;
#pragma unroll
      for (int st = 0; st < KS_H; ++st) {
        const int e0 = (half * KS_H + st) * 4 * KPL + g * KPL;
        if constexpr (kBf) {
          qb[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qh + e0));
        } else {
          qb[st] = qh[e0];
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < KS_H; ++st) qb[st] = zero_frag<Op>();
    }
  }

  const int32_t* btb = bt + (int64_t)b * bt_stride;
  const int32_t* idxb = indices ? indices + (int64_t)b * k : nullptr;
  const int spair = tid >> 5;  // staging: token rows 2*spair, 2*spair+1 of the tile
  const int sj = tid & 31;     // staging: chunks sj, sj+32, ...
  uint32_t raw[CPT][2][CH_DW];
  bool raw_ok[2];

  // Issue the global loads of the tile whose first row is seg_row[tb].  Every
  // lane issues the same loads whatever its row (a masked row reads row 0, a
  // spare chunk slot re-reads the last chunk), so the compiler can count them
  // and keep them in flight across the tile's math; stage() zeroes what is
  // masked.
  auto issue = [&](int tb) __attribute__((always_inline)) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int32_t row = seg_row[tb + 2 * spair + rr];
      raw_ok[rr] = row >= 0;
      const uint8_t* src = kv + (int64_t)(row >= 0 ? row : 0) * ROW_BYTES;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = min(sj + 32 * i, NCH - 1);
        load_raw<CH_BYTES>(src + c * CH_BYTES, raw[i][rr]);
      }
    }
  };
  // Widen the staged registers into an LDS tile (row-major K[token][dim]; the
  // value operand is read from the same rows with transposing LDS reads).
  auto stage = [&](E* __restrict__ Kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = sj + 32 * i;
      if (c < NCH) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
          for (int w = 0; w < CH_DW; ++w) raw[i][rr][w] = raw_ok[rr] ? raw[i][rr][w] : 0u;
          E* kd = Kt + sw(2 * spair + rr, c);
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

  // Partial scores S^T[token x head] over this wave's half of the dims for
  // the tile in Kt: row r16 (+16), chunk half*KS_H*4*KPL/8 + st*4*KPL/8 + g
  // (bf16); the chunk swizzle only flips bit 0, which st's even stride
  // leaves alone.
  auto qk_partial = [&](const E* __restrict__ Kt, f32x4 (&out)[2]) __attribute__((always_inline)) {
    f32x4 sc2[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      out[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc2[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const E* kbase = kBf ? Kt + sw(r16, half * KS_H * 4 + g) : Kt + r16 * DS + half * KS_H * 4 + g;
#pragma unroll
    for (int st = 0; st < KS_H; ++st) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const E* krow = kbase + m * 16 * DS + st * 4 * KPL;
        typename Op::frag a;
        if constexpr (kBf) {
          a = *reinterpret_cast<const bf16x8*>(krow);
        } else {
          a = *krow;
        }
        if (st & 1) sc2[m] = Op::mma(a, qb[st], sc2[m]);
        else out[m] = Op::mma(a, qb[st], out[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) out[m] += sc2[m];
  };

  // Softmax with a fixed reference per head instead of a running max: the
  // reference of head r16 is the max of the first tile in which the split has
  // a valid token (every head's accumulator is still zero then, so setting it
  // is free); later weights are exp2(z - m_ref) <= 2^kHeadroom unless a
  // tile's max exceeds m_ref by more than kHeadroom.  If that happens anywhere
  // in the workgroup the split is recomputed once with the true max as
  // reference, so the accumulator is never rescaled inside the loop.  Same
  // result as the running-max form: o and l share the reference, which
  // cancels in o / l.  Between those points each lane keeps its own partial
  // max and sum (over its 8 tokens of each tile); they are combined across the
  // lanes of a head once, at the end.
  f32x4 acc_o[NT_H];
  float m_ref = -INFINITY;   // reference (log2 domain) of head r16, equal in its 4 lanes
  float m_lane = -INFINITY;  // this lane's running max
  float l_lane = 0.f;        // this lane's sum of weights
  if (tid == 0) bad_flag = 0;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int nt = 0; nt < NT_H; ++nt) acc_o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_lane = 0.f;
    if (pass == 1) m_ref = wave_max_xor16_32(m_lane);
    bool over = false;
    if (tid == 0) redo_flag = 0;

    for (int64_t seg = p_begin; seg < p_end; seg += kSeg) {
      const int64_t seg_end = min(p_end, seg + kSeg);
      const int ntiles = (int)((seg_end - seg + kTile - 1) / kTile);
      __syncthreads();  // previous segment's tiles are done with seg_row / LDS
      // ---- resolve the segment's rows (index -> page -> row) once; entries
      // past the segment's end are masked, so the tail tile needs no bounds test
      for (int e = tid; e < kSeg; e += kDecThreads) {
        const int64_t p = seg + e;
        int32_t row = -1;
        float sc = 1.f;
        if (p < seg_end) {
          const int64_t t = idxb ? (int64_t)idxb[p] : p;
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
              if (KDT == kFP8) sc = kv_scale[row];
            }
          }
        }
        seg_row[e] = row;
        seg_zsc[e] = sm_scale_log2 * sc;
        seg_tsc[e] = sc;
        seg_bias[e] = row >= 0 ? 0.f : -INFINITY;
      }
      __syncthreads();
      // Tile i lives in Kbuf[i % 3].  Tiles 0 and 1 are staged up front; tile
      // i + 2 is staged in iteration i, after every wave has passed the
      // barrier that ends tile i - 1, whose buffer it reuses.  The partial
      // scores of tile i + 1 are computed in iteration i as well, so the
      // matrix cores have them to work on while the softmax of tile i runs.
      issue(0);
      stage(Kbuf[0]);
      if (ntiles > 1) {
        issue(kTile);
        stage(Kbuf[1]);
      }
      if (ntiles > 2) issue(2 * kTile);
      __syncthreads();
      f32x4 sc_own[2];
      qk_partial(Kbuf[0], sc_own);
#pragma unroll
      for (int m = 0; m < 2; ++m) sx[0][wv][m][lane] = sc_own[m];
      __syncthreads();
      int cur = 0;
      for (int i = 0; i < ntiles; ++i) {
        const int nxt = cur == 2 ? 0 : cur + 1;
        const E* Kt = Kbuf[cur];
        const int tb = i * kTile;  // tile base within the segment
        // ---- full scores of tile i: own half + other half (a two-term sum is
        // commutative, so both waves of the pair hold identical scores)
        f32x4 sc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const f32x4 other = sx[i & 1][wv ^ 1][m][lane];
          sc[m] = sc_own[m] + other;
        }
        // Per-token factors of this lane's 8 tokens (tb + m*16 + g*4 + j).
        f32x4 zsc[2], tsc[2], zb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          zsc[m] = *reinterpret_cast<const f32x4*>(seg_zsc + tb + m * 16 + g * 4);
          tsc[m] = *reinterpret_cast<const f32x4*>(seg_tsc + tb + m * 16 + g * 4);
          zb[m] = *reinterpret_cast<const f32x4*>(seg_bias + tb + m * 16 + g * 4);
        }
        // ---- partial scores of tile i + 1 (after the last tile this reads a
        // stale buffer; the result is never used)
        qk_partial(Kbuf[nxt], sc_own);
        // ---- softmax weights (log2 domain) for head r16
        // A masked row was staged as zeros, so its score is 0 and z = -inf.
        float z[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            z[m][j] = __builtin_fmaf(sc[m][j], zsc[m][j], zb[m][j]);
            mx = fmaxf(mx, z[m][j]);
          }
        }
        m_lane = fmaxf(m_lane, mx);
        // First tile with a valid token: every head takes that tile's max as
        // its reference (all heads see the same tokens, so this branch is
        // taken by the whole wave at once).
        if (__builtin_expect(__any(m_ref == -INFINITY), 0)) {
          const float full = wave_max_xor16_32(mx);
          if (m_ref == -INFINITY) m_ref = full;
        }
        over |= mx > m_ref + kHeadroom;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;  // all z are -inf while unset
        float pv[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pp = __builtin_amdgcn_exp2f(z[m][j] - m_use);
            l_lane += pp;
            pv[m][j] = pp * tsc[m][j];
          }
        }
        // ---- O += P . V over this wave's half of the output dims
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
          // Row 4g + r16/4 (bit 3 of it is g/2), dims half*DC/2 + 4*(r16&3)
          // onwards: chunk half*DC/16 + (r16&3)/2, swizzled; nt's stride of
          // two chunks leaves the swizzle bit alone.
          const int vrow = g * 4 + (r16 >> 2);
          const E* vsrc = Kt + sw(vrow, half * (DC / 16) + ((r16 & 3) >> 1)) + 4 * (r16 & 1);
#pragma unroll
          for (int nt = 0; nt < NT_H; ++nt) {
            const v4bf16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(vsrc + nt * 16));
            const v4bf16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(vsrc + 16 * DS + nt * 16));
            const bf16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc_o[nt] = Op::mma(pa, vb, acc_o[nt]);
          }
        } else {
#pragma unroll
          for (int nt = 0; nt < NT_H; ++nt) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc_o[nt] = Op::mma(pv[m][j], Kt[(m * 16 + g * 4 + j) * DS + half * (DC / 2) + nt * 16 + r16],
                                    acc_o[nt]);
            }
          }
        }
        // Publish tile i + 1's partial scores, stage tile i + 2 into the
        // buffer tile i - 1 used, then send the loads of tile i + 3.
#pragma unroll
        for (int m = 0; m < 2; ++m) sx[(i + 1) & 1][wv][m][lane] = sc_own[m];
        if (i + 2 < ntiles) {
          stage(Kbuf[nxt == 2 ? 0 : nxt + 1]);
          if (i + 3 < ntiles) issue((i + 3) * kTile);
        }
        __syncthreads();
        cur = nxt;
      }
    }
    // Recompute the split once if any head of the workgroup outgrew its reference.
    if (__any(over) && lane == 0) atomicOr(&redo_flag, 1);
    __syncthreads();
    const bool redo = redo_flag != 0;
    __syncthreads();
    if (!redo) break;
  }

  if (!wave_active) return;
  // ---- finalize: o = O / l for this wave's half, lse = (m + log2 l) * ln 2
  const bool bad = bad_flag != 0;
  const float l_run = wave_sum_xor16_32(l_lane);
  float inv_l[4];  // 1 / l of head g*4 + j (0 for a head with no valid token)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float li = __shfl(l_run, g * 4 + j);
    inv_l[j] = bad ? kNaN : (li > 0.f ? 1.f / li : 0.f);
  }
#pragma unroll
  for (int nt = 0; nt < NT_H; ++nt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = head0 + g * 4 + j;
      if (h < n_heads) {
        const float v = acc_o[nt][j] * inv_l[j];
        *out_o(h, half * (DC / 2) + nt * 16 + r16) = v;
      }
    }
  }
  if (half == 0 && g == 0 && head0 + r16 < n_heads) {
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
                     a.bt_stride, a.lens, a.max_len, a.indices, a.k, a.n_heads, sm_log2, a.num_splits, a.split_tokens, n_hg,
                     a.o_part, a.lse_part, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_decode(const DecodeArgs& a, hipStream_t s) {
  const int D = a.d_latent + a.d_rope;
  if (a.q_dtype == kBF16 && D == 576 && a.d_latent == 512) {
    if (a.kv_dtype == kBF16) return launch_decode_bf16(a, s);
    if (a.kv_dtype == kFP8) return launch_decode_f8(a, s);
    return -2;
  }
  if (a.q_dtype == kF32 && D == 80 && a.d_latent == 64) {
    if (a.kv_dtype == kF32) return launch_one<OpF32, kF32, 20, 4>(a, s);
    if (a.kv_dtype == kBF16) return launch_one<OpF32, kBF16, 20, 4>(a, s);
    if (a.kv_dtype == kFP8) return launch_one<OpF32, kFP8, 20, 4>(a, s);
    return -2;
  }
  return launch_decode_generic(a, s);  // any other shape the interface takes
}

}  // namespace spmla
