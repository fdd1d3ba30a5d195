// mla_paged_decode for a bf16 latent cache, bf16 query, 512 latent + 64 rope
// dims: split-KV MLA decode over the selected (or all) tokens, both
// contractions on MFMA, with the waves of a workgroup specialised by role so
// that vector work on one wave of a SIMD overlaps matrix work on the other.
// The schedule is the one of the FP8 kernel (mla_decode_f8.hip); what
// differs is the tile (1152-byte rows, no scales) and that the cache values
// are MFMA operands as they are.
//
// Workgroup = (request b, split s, group of 64 query heads); 8 waves.
//  - Waves 0-3, score waves: wave (hq, th) holds the query of heads
//    32hq..32hq+31 of the group in registers (144 VGPRs, loaded straight
//    from HBM in operand order) and computes, for every 32-token tile, the
//    scores of those heads against the tile's tokens 16th..16th+15 over all
//    576 dims on the 16x16x32 bf16 MFMA (tokens on M, heads on N), then
//    their softmax weights, written to LDS as bf16.
//  - Waves 4-7, value waves: wave (hq, dh) accumulates O[32 heads x 256 dims]
//    (heads 32hq.., dims 256dh..) += P[32 heads x 32 tokens] . V[32 tokens x
//    256 dims] on the 32x32x16 bf16 MFMA, one tile behind the score waves,
//    with V read from the same LDS tile by gfx950's 16-bit transposing LDS
//    read.  These waves also fetch the tiles: every lane's 16-byte piece of
//    a tile goes straight from HBM into LDS (global_load_lds_dwordx4).
// Tiles rotate through kNB LDS buffers and are requested kPF tiles ahead of
// the one being scored; one barrier per tile.
//
// LDS tile layout: 32 rows of 1152 bytes (72 16-byte chunks, no padding: four
// buffers and the tables just fit in the 160 KiB of LDS).  Chunk slot j of
// row r holds chunk j ^ f(r), f(r) = ((x & 1) << 2) | (x >> 1) with
// x = (r >> 1) & 7.  A score read (16 rows, one chunk each, per 16 lanes)
// then meets each of the 16 chunk positions of a 256-byte bank window once,
// and a transposing read (4 rows of 64 bytes per 32 lanes) meets the four
// 64-byte quarters of the window once: both are free of bank conflicts.  The
// permutation stays inside aligned groups of 8 chunks, so the rope chunks
// 64..71 stay in place as a group.
//
// The waits for the direct loads are explicit (see decode_ws.h): each value
// wave issues exactly kLoads loads per tile, so "tile i + 1 has landed" is
// "at most kLoads * (kPF - 1) loads outstanding".
//
// Softmax: weights are taken against a fixed reference per head, the
// largest logit of the split's first tile (both score waves of a head meet
// in LDS once, before the loop).  Later weights are exp2(z - m_ref) <=
// 2^kHeadroom unless a logit exceeds m_ref by more than kHeadroom; if that
// happens anywhere in the workgroup the split is recomputed once with the
// true maximum.  The reference cancels in o = O / l, so this is the same
// quantity as the running-max form, and the accumulators are never rescaled.
#include "common.h"
#include "launch.h"
#include "decode_ws.h"

#include <type_traits>

namespace spmla {
namespace {
using namespace ws;

constexpr int kThreads = 512;
constexpr int kTileTok = 32;
constexpr int kD = 576, kDC = 512;
constexpr int kRowBytes = 2 * kD;                  // 1152
constexpr int kRowChunks = kRowBytes / 16;         // 72
constexpr int kTileBytes = kTileTok * kRowBytes;   // 36864
constexpr int kLoads = kTileBytes / 1024 / 4;      // 9 wave loads of 1 KiB per value wave per tile
constexpr int kNB = 4;                             // tile buffers
constexpr int kPF = 2;                             // tiles requested ahead of the scored one
constexpr int kSeg = 1024;                         // positions resolved at once
constexpr int kHeadsWg = 64;
constexpr int kPStride = 40;                       // bf16 per weight row (32 tokens + 8 pad)
constexpr int kKSteps = kD / 32;                   // 18 score k-steps of the 16x16x32 MFMA
constexpr float kHeadroom = 16.f;
static_assert(kTileBytes == 4 * kLoads * 1024, "tile loads split evenly over the value waves");
static_assert(kNB >= kPF + 2, "a tile buffer is refilled only after both roles are done with it");
static_assert(kLoads * (kPF - 1) <= 63, "vmcnt range");

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v4bf16_t lds_v4bf16;

// A zero row: what a masked position loads, so every load is unconditional
// and a masked token scores exactly 0 before its -inf bias.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row16[kRowBytes];

__device__ __forceinline__ int cswz(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

__global__ __launch_bounds__(kThreads) void mla_decode_bf16ws_kernel(
    const __bf16* __restrict__ q, const uint8_t* __restrict__ kv, int32_t num_pages, int32_t page_shift,
    const int32_t* __restrict__ bt, int32_t bt_stride, const int32_t* __restrict__ lens, int64_t max_len,
    const int32_t* __restrict__ indices, int32_t k, int32_t n_heads, float sm_scale_log2, int32_t num_splits,
    int32_t split_tok, int32_t n_hg, float* __restrict__ o_part, float* __restrict__ lse_part, int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(16))) uint8_t Kbuf[kNB][kTileBytes];
  __shared__ __attribute__((aligned(16))) int32_t seg_row[kSeg];       // cache row, or -1 when masked
  __shared__ __attribute__((aligned(16))) __bf16 Pbuf[2][kHeadsWg * kPStride];
  __shared__ __attribute__((aligned(16))) float red[2][kHeadsWg];      // per token half: head maxima / sums
  __shared__ int redo_flag;
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wv < 4;
  const int role = wv & 3;
  const int hq = role >> 1;            // head tile: heads 32hq..32hq+31 of the group
  const int th = role & 1;             // score waves: token half of each tile
  const int dh = role & 1;             // value waves: dim half
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int page_size = 1 << page_shift;
  const float kNaN = __uint_as_float(0x7FC00000u);

  const WgCoord wc = wg_coord(blockIdx.x, gridDim.x, num_splits, n_hg, split_tok > 0);
  const int hg = wc.hg, s = wc.s, b = wc.b;
  const int head_base = hg * kHeadsWg;

  auto out_o = [&](int h, int dim) -> float* {
    return o_part + ((((int64_t)b * num_splits + s) * n_heads + h) * kDC + dim);
  };
  auto out_lse = [&](int h) -> float* { return lse_part + (((int64_t)b * num_splits + s) * n_heads + h); };

  // ---- value waves' share of each tile: loads 9w'..9w'+8 of the tile's 36
  // (w' = role).  Piece p of a load lands at slot p of the tile: row p / 72,
  // chunk slot p % 72, which holds chunk (p % 72) ^ f(row).
  int ld_off[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int slot = 64 * (kLoads * role + u) + lane;
    const int r = slot / kRowChunks;
    ld_off[u] = (r << 8) | ((slot % kRowChunks) ^ cswz(r));
  }
  auto piece_row = [&](int u) { return ld_off[u] >> 8; };

  // ---- first loads.  The split positions of a sparse call depend on k
  // alone, so the index loads for the first segment's table (and for the
  // value waves' pieces of tiles 0 and 1) go out before anything else.  A
  // dense call, or one with k = 0, reads the request's length there instead
  // and does not use it.
  const int32_t* btb = bt + (int64_t)b * bt_stride;
  const bool sparse = indices != nullptr;
  constexpr int kNT = kSeg / kThreads;   // table entries per thread
  constexpr int kNP = kNT + 2 * kLoads;  // and the value waves' pieces of tiles 0 and 1
  auto split_len = [&](int64_t n) -> int64_t {
    return split_tok > 0 ? split_tok : ((n + num_splits - 1) / num_splits + kTileTok - 1) / kTileTok * kTileTok;
  };
  auto pos_at = [&](int64_t p0, int i) -> int64_t {
    if (i < kNT) return p0 + tid + i * kThreads;
    return p0 + ((i - kNT) / kLoads) * kTileTok + piece_row((i - kNT) % kLoads);
  };
  int32_t iv[kNP];
  {
    const bool early = sparse && k > 0;
    const int64_t p0 = (int64_t)s * split_len(k);
    const int32_t* ib = early ? indices + (int64_t)b * k : lens + b;
#pragma unroll
    for (int i = 0; i < kNP; ++i) iv[i] = ib[early ? min(pos_at(p0, i), (int64_t)k - 1) : 0];
  }

  const int32_t L = lens[b];
  if (L < 0 || (int64_t)L > max_len || (int64_t)L > (int64_t)bt_stride * page_size) {
    vm_wait<0>();  // the early loads land before the workgroup ends
    if (tid == 0 && status) atomicOr(status + b, kBadLen);
    for (int i = tid; i < kHeadsWg * kDC; i += kThreads) {
      const int h = head_base + i / kDC;
      if (h < n_heads) *out_o(h, i % kDC) = kNaN;
    }
    if (tid < kHeadsWg && head_base + tid < n_heads) *out_lse(head_base + tid) = kNaN;
    return;
  }
  const int64_t n = sparse ? (int64_t)k : (int64_t)L;
  const int64_t per = split_len(n);
  const int64_t p_begin = (int64_t)s * per;
  const int64_t p_end = split_tok > 0 && s == num_splits - 1 ? n : min(n, p_begin + per);
  if (split_tok > 0 && p_begin >= p_end) {
    // A fixed split length leaves the splits past the request's last token
    // empty: they only mark their partial as empty (lse -inf).
    vm_wait<0>();  // the early loads land before the workgroup ends
    if (tid < kHeadsWg && head_base + tid < n_heads) *out_lse(head_base + tid) = -INFINITY;
    return;
  }
  const int32_t* idxb = sparse ? indices + (int64_t)b * k : nullptr;
  const bool any_token = p_begin < p_end;
  // Tokens at split positions and the pages of tokens, for the segments
  // after the first: every load reads a clamped, always valid address, and
  // its value passes through an empty asm before it is selected, so that
  // the compiler cannot move the load into the branch of the select.  Dense
  // calls have no index array: they read the block table's first entry and
  // do not use it.
  const int32_t* idx_src = idxb ? idxb : btb;
  auto tokens_at = [&](const auto& pos, int64_t seg_end, int64_t* out) {
    constexpr int N = std::extent<std::remove_reference_t<decltype(pos)>>::value;
    int32_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = idx_src[sparse ? min((int64_t)pos[i], n - 1) : 0];
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = pos[i] < seg_end ? (sparse ? (int64_t)v[i] : (int64_t)pos[i]) : -1;
  };
  auto pages_of = [&](const int64_t* t, int32_t* out, auto n_tag) {
    constexpr int N = decltype(n_tag)::value;
    int32_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = btb[(t[i] >= 0 && t[i] < L ? t[i] : 0) >> page_shift];
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = t[i] >= 0 && t[i] < L ? v[i] : -1;
  };
  if (tid == 0) bad_flag = 0;
  wg_barrier();  // bad_flag is cleared before any table entry may set it

  // The cache row of token t given its page, or -1 (masked); flags a bad
  // index or page.
  auto row_of = [&](int64_t t, int32_t page) -> int32_t {
    if (t < -1 || t >= L) {
      bad_flag = 1;
      if (status) atomicOr(status + b, kBadIndex);
    } else if (t >= 0) {
      if (page < 0 || page >= num_pages) {
        bad_flag = 1;
        if (status) atomicOr(status + b, kBadPage);
      } else {
        return (int32_t)(((int64_t)page << page_shift) + (t & (page_size - 1)));
      }
    }
    return -1;
  };
  // Resolve positions [seg, seg_end) of the split (index -> page -> row);
  // entries past seg_end are masked.
  auto build_table = [&](int64_t seg, int64_t seg_end) __attribute__((always_inline)) {
    int64_t pos[kNT], t[kNT];
#pragma unroll
    for (int u = 0; u < kNT; ++u) pos[u] = seg + tid + u * kThreads;
    tokens_at(pos, seg_end, t);
    int32_t page[kNT];
    pages_of(t, page, std::integral_constant<int, kNT>{});
#pragma unroll
    for (int u = 0; u < kNT; ++u) seg_row[tid + u * kThreads] = row_of(t[u], page[u]);
  };
  const uint8_t* zero_row = g_zero_row16;
  // Send this lane's loads of a tile whose pieces come from cache rows
  // row[u] (-1: masked, the zero row) into buffer `buf`.
  auto dma_rows = [&](const int32_t (&row)[kLoads], int buf) __attribute__((always_inline)) {
    const uint32_t dst = lds_addr(&Kbuf[0][0]) + buf * kTileBytes + 1024 * kLoads * role;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int c = ld_off[u] & 255;
      const uint8_t* src = row[u] >= 0 ? kv + (int64_t)row[u] * kRowBytes + 16 * c : zero_row + 16 * c;
      dma16(src, dst + 1024 * u);
    }
  };

  // ---- prologue: once the indices are in, the first segment's pages are
  // requested; the value waves resolve their pieces of tiles 0 and 1 and
  // request those tiles, and every thread writes its entries of the table.
  if (!any_token) vm_wait<0>();  // nothing to score: just let the early loads land
  if (any_token) {
    const int64_t seg_end = min(p_end, p_begin + kSeg);
    vm_wait<0>();  // the indices are in
    int32_t t[kNP], pv[kNP];
#pragma unroll
    for (int i = 0; i < kNP; ++i) {
      const int64_t p = pos_at(p_begin, i);
      t[i] = p < seg_end ? (sparse ? iv[i] : (int32_t)p) : -1;
      pv[i] = btb[(t[i] >= 0 && t[i] < L ? t[i] : 0) >> page_shift];
    }
#pragma unroll
    for (int i = 0; i < kNP; ++i) asm volatile("" : "+v"(pv[i]));
    if (!score_wave) {
      int32_t prow[2][kLoads];
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
          const int32_t tt = t[kNT + tl * kLoads + u], pp = pv[kNT + tl * kLoads + u];
          prow[tl][u] = tt >= 0 && tt < L && pp >= 0 && pp < num_pages ? (int32_t)(((int64_t)pp << page_shift) + (tt & (page_size - 1))) : -1;
        }
      }
      dma_rows(prow[0], 0);
      dma_rows(prow[1], 1);
    }
#pragma unroll
    for (int u = 0; u < kNT; ++u) seg_row[tid + u * kThreads] = row_of(t[u], pv[u]);
    wg_barrier();  // the first table is in LDS
  }

  int64_t built = any_token ? p_begin : -1;  // segment whose table is in LDS
  // Both roles run the same sequence of barriers.
  if (score_wave) {
    // The query, straight into registers in B-operand order: qf[nt][ks]
    // holds dims 32ks + 8g..+7 of head 32hq + 16nt + r16 of the group.  Its
    // loads overlap those of tiles 0 and 1 (requested in the prologue); they
    // are not issued earlier because the prologue's registers and these 144
    // do not fit together.  Heads past the last one load head 0: their
    // results are never stored.
    bf16x8 qf[2][kKSteps];
    {
      const __bf16* qb = q + (int64_t)b * n_heads * kD;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int h = head_base + hq * 32 + nt * 16 + r16;
        const __bf16* qrow = qb + (int64_t)(h < n_heads ? h : 0) * kD + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qf[nt][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
      }
    }
    // Scores of the tile in Kt for this wave's 16 tokens (rows 16th + r16 on
    // M) and its 32 heads (two N-tiles): S[nt] holds head 16nt + r16 for
    // tokens 16th + 4g + j.  Two accumulators per N-tile halve the chains.
    auto score_tile = [&](const uint8_t* __restrict__ Kt, f32x4 (&S)[2]) __attribute__((always_inline)) {
      f32x4 acc[2][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt][0] = acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = th * 16 + r16;
      const int sw = cswz(row);
      const uint8_t* rp = Kt + row * kRowBytes;
      static_for<kKSteps>([&](auto KS) {
        constexpr int ks = decltype(KS)::value;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(rp + 16 * ((4 * ks + g) ^ sw));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[nt][ks & 1] = OpBF16::mma(a, qf[nt][ks], acc[nt][ks & 1]);
      });
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) S[nt] = acc[nt][0] + acc[nt][1];
    };

    float m_ref[2] = {-INFINITY, -INFINITY};   // reference of head 16nt + r16 (log2 domain)
    float m_lane[2] = {-INFINITY, -INFINITY};  // this lane's largest logit
    float l_lane[2] = {0.f, 0.f};              // this lane's sum of weights
    bool fallback = false;                     // the first tile had no valid token: 0 stood in for m_ref
    // The -inf bias of masked tokens 16th + 4g + j of the tile at table
    // position tb.
    auto bias4 = [&](int tb) -> f32x4 {
      const int4 r4 = *reinterpret_cast<const int4*>(&seg_row[tb + th * 16 + 4 * g]);
      return f32x4{r4.x >= 0 ? 0.f : -INFINITY, r4.y >= 0 ? 0.f : -INFINITY, r4.z >= 0 ? 0.f : -INFINITY,
                   r4.w >= 0 ? 0.f : -INFINITY};
    };
    // Softmax weights of a scored tile, written to P as bf16.
    auto softmax_tile = [&](const f32x4 (&S)[2], int tb, __bf16* __restrict__ P, bool& over)
        __attribute__((always_inline)) {
      const int t0 = th * 16 + 4 * g;
      const f32x4 bi = bias4(tb);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float z[4], mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[j] = __builtin_fmaf(S[nt][j], sm_scale_log2, bi[j]);
          mx = fmaxf(mx, z[j]);
        }
        m_lane[nt] = fmaxf(m_lane[nt], mx);
        over |= mx > m_ref[nt] + kHeadroom;
        float pw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pw[j] = __builtin_amdgcn_exp2f(z[j] - m_ref[nt]);
          l_lane[nt] += pw[j];
        }
        const v4bf16_t w4 = {(__bf16)pw[0], (__bf16)pw[1], (__bf16)pw[2], (__bf16)pw[3]};
        *reinterpret_cast<v4bf16_t*>(P + (hq * 32 + nt * 16 + r16) * kPStride + t0) = w4;
      }
    };

    for (int pass = 0; pass < 2; ++pass) {
      l_lane[0] = l_lane[1] = 0.f;
      bool over = false;
      if (tid == 0) redo_flag = 0;
      for (int64_t seg = p_begin; seg < p_end; seg += kSeg) {
        const int64_t seg_end = min(p_end, seg + kSeg);
        const int T = (int)((seg_end - seg + kTileTok - 1) / kTileTok);
        const bool need_ref = pass == 0 && seg == p_begin;
        if (seg != built) {
          wg_barrier();  // the previous segment is done with the table
          build_table(seg, seg_end);
          built = seg;
          wg_barrier();
        }
        wg_barrier();  // tile 0 has landed
        f32x4 S[2];
        score_tile(Kbuf[0], S);
        if (need_ref) {
          const f32x4 bi = bias4(0);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = fmaxf(mx, __builtin_fmaf(S[nt][j], sm_scale_log2, bi[j]));
            mx = wave_max_xor16_32(mx);
            if (g == 0) red[th][hq * 32 + nt * 16 + r16] = mx;
          }
          wg_barrier();
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int hl = hq * 32 + nt * 16 + r16;
            m_ref[nt] = fmaxf(red[0][hl], red[1][hl]);
            // No valid token in the first tile (the same for every head): 0
            // stands in, and the split is recomputed with the true maximum
            // if any valid token turns up.
            if (m_ref[nt] == -INFINITY) {
              m_ref[nt] = 0.f;
              fallback = true;
            }
          }
        }
        softmax_tile(S, 0, Pbuf[0], over);
        wg_barrier();  // tile 1 has landed; P of tile 0 is written
        int buf = 1;  // buffer of tile i
        for (int i = 1; i <= T; ++i) {
          if (i < T) {
            score_tile(Kbuf[buf], S);
            softmax_tile(S, i * kTileTok, Pbuf[i & 1], over);
          }
          buf = buf == kNB - 1 ? 0 : buf + 1;
          wg_barrier();
        }
      }
      // Recompute the split once if a logit outgrew its head's reference,
      // or if the reference was a stand-in and valid tokens were seen.
      const bool seen = m_lane[0] > -INFINITY || m_lane[1] > -INFINITY;
      if (__any(over || (fallback && seen)) && lane == 0) atomicOr(&redo_flag, 1);
      wg_barrier();
      if (pass == 1 || redo_flag == 0) break;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mt = wave_max_xor16_32(m_lane[nt]);
        if (g == 0) red[th][hq * 32 + nt * 16 + r16] = mt;
      }
      wg_barrier();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int hl = hq * 32 + nt * 16 + r16;
        m_ref[nt] = fmaxf(red[0][hl], red[1][hl]);
        if (m_ref[nt] == -INFINITY) m_ref[nt] = 0.f;
      }
      fallback = false;
    }
    // ---- finish: l per head from both token halves, then lse.
    wg_barrier();  // red is free again
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float ls = wave_sum_xor16_32(l_lane[nt]);
      if (g == 0) red[th][hq * 32 + nt * 16 + r16] = ls;
    }
    wg_barrier();
    const bool bad = bad_flag != 0;
    if (th == 0 && g == 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int hl = hq * 32 + nt * 16 + r16;
        const int h = head_base + hl;
        if (h < n_heads) {
          const float l = red[0][hl] + red[1][hl];
          const float lse = l > 0.f ? (m_ref[nt] + log2f(l)) * 0.69314718055994530942f : -INFINITY;
          *out_lse(h) = bad ? kNaN : lse;
        }
      }
    }
  } else {
    // ---- value waves.  Send the loads of tile `tile` of the segment (T
    // tiles) into buffer `buf`; a tile past the segment's end loads the zero
    // row into a buffer no tile uses, so every call issues exactly kLoads
    // loads.
    auto issue_tile = [&](int tile, int T, int buf) __attribute__((always_inline)) {
      const bool real = tile < T;
      const int32_t* rows = seg_row + min(tile, T - 1) * kTileTok;
      int32_t row[kLoads];  // all table reads first, so that one LDS wait covers them
#pragma unroll
      for (int u = 0; u < kLoads; ++u) row[u] = real ? rows[piece_row(u)] : -1;
      dma_rows(row, buf);
    };
    // O += P . V for the tile in Vt with the weights in P.  A operand (P):
    // lane l holds head l % 32, tokens 16ks + 8(l / 32) + e.  B operand (V):
    // a transposing read hands lane i of each 16-lane group the value of
    // dim i of the 16-dim window its group points at, for the 4 tokens the
    // group points at (lane j of the group: dims 4(j & 3).. of token j / 4).
    // Lane i of group G thus gets dim 16(G & 1) + i of the N-tile for tokens
    // 16ks + 8(G >> 1) + 0..3 from one read and + 4..7 from a second, when
    // lane j of the group points at dims 16(G & 1) + 4(j & 3).. of those
    // tokens.
    // Byte offsets in a tile of this lane's transposing reads: token row
    // tr = 16ks + 8(G >> 1) + j / 4 (+4 for the second read), chunk
    // 32dh + 4nt + 2(G & 1) + (j & 3) / 2 of it, 8(j & 1) bytes in.  The
    // row's chunk permutation flips bits 0-1 of that chunk by f & 3 and bit
    // 2 (bit 0 of nt) by f >> 2, so the offset is a base for even nt and one
    // for odd nt, plus 64 nt.
    int v_off[2][2][2];
    {
      const int G = lane >> 4, j = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int tr = 16 * ks + 8 * (G >> 1) + (j >> 2) + 4 * hf;
          const int f = cswz(tr);
          const int base = tr * kRowBytes + 8 * (j & 1) + 16 * (32 * dh + ((2 * (G & 1) + ((j & 3) >> 1)) ^ (f & 3)));
          v_off[ks][hf][0] = base + 64 * (f >> 2);
          v_off[ks][hf][1] = base - 64 * (f >> 2);
        }
      }
    }
    auto pv_tile = [&](const uint8_t* __restrict__ Vt, const __bf16* __restrict__ P, f32x16 (&acc_o)[8])
        __attribute__((always_inline)) {
      // All LDS reads of the tile are issued before the first MFMA, so the
      // MFMAs wait for them once instead of one read latency each.
      bf16x8 pa[2];
      v4bf16_t vlo[2][8], vhi[2][8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pa[ks] = *reinterpret_cast<const bf16x8*>(P + (hq * 32 + (lane & 31)) * kPStride + 16 * ks + 8 * (lane >> 5));
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          vlo[ks][nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(Vt + v_off[ks][0][nt & 1] + 64 * nt));
          vhi[ks][nt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf16*)(Vt + v_off[ks][1][nt & 1] + 64 * nt));
        }
      }
      // Four groups of four independent MFMAs in this order (left to itself
      // the scheduler interleaves each read with its MFMA, one LDS latency
      // per MFMA).
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int nt = 4 * h4; nt < 4 * h4 + 4; ++nt) {
            const v4bf16_t lo = vlo[ks][nt], hi = vhi[ks][nt];
            const bf16x8 vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc_o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], vb, acc_o[nt], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 acc_o[8];
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc_o[nt] = f32x16{};
      for (int64_t seg = p_begin; seg < p_end; seg += kSeg) {
        const int64_t seg_end = min(p_end, seg + kSeg);
        const int T = (int)((seg_end - seg + kTileTok - 1) / kTileTok);
        const bool need_ref = pass == 0 && seg == p_begin;
        if (seg != built) {
          wg_barrier();
          build_table(seg, seg_end);
          built = seg;
          wg_barrier();
        }
        // Tiles 0 and 1 of the split's first segment were requested in the
        // prologue; the others are requested here.  Tile i of a segment
        // lives in buffer i % kNB.
        const int pre = need_ref ? 2 : 0;
#pragma unroll
        for (int i = 0; i < kPF; ++i)
          if (i >= pre) issue_tile(i, T, i % kNB);
        vm_wait<kLoads * (kPF - 1)>();  // tile 0 has landed
        wg_barrier();
        if (need_ref) wg_barrier();
        issue_tile(kPF, T, kPF % kNB);
        vm_wait<kLoads * (kPF - 1)>();  // tile 1 has landed
        wg_barrier();
        int buf_in = (kPF + 1) % kNB, buf_pv = 0;  // buffers of tiles i + kPF and i - 1
        for (int i = 1; i <= T; ++i) {
          issue_tile(i + kPF, T, buf_in);
          pv_tile(Kbuf[buf_pv], Pbuf[(i - 1) & 1], acc_o);
          __builtin_amdgcn_sched_barrier(0);  // the wait stays after this tile's MFMAs
          vm_wait<kLoads * (kPF - 1)>();  // tile i + 1 has landed
          buf_in = buf_in == kNB - 1 ? 0 : buf_in + 1;
          buf_pv = buf_pv == kNB - 1 ? 0 : buf_pv + 1;
          wg_barrier();
        }
        vm_wait<0>();  // the loads past the segment's end are done with
      }
      wg_barrier();
      if (pass == 1 || redo_flag == 0) break;
      wg_barrier();
    }
    // ---- finish: o = O / l.  D layout of the 32x32 MFMA: element e of
    // lane l is row (head) 8(e / 4) + 4(l / 32) + e % 4, column (dim) l % 32.
    wg_barrier();
    wg_barrier();
    const bool bad = bad_flag != 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int hl = hq * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const int h = head_base + hl;
      const float l = red[0][hl] + red[1][hl];
      const float inv = bad ? kNaN : (l > 0.f ? 1.f / l : 0.f);
      if (h < n_heads) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) *out_o(h, dh * 256 + nt * 32 + (lane & 31)) = acc_o[nt][e] * inv;
      }
    }
  }
}

}  // namespace

int launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  const int n_hg = (a.n_heads + kHeadsWg - 1) / kHeadsWg;
  const int64_t grid = (int64_t)a.batch * a.num_splits * n_hg;
  if (grid == 0) return 0;
  if (grid > 0x7FFFFFFF) return -2;
  const float sm_log2 = a.sm_scale * 1.44269504088896340736f;
  hipLaunchKernelGGL(mla_decode_bf16ws_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const uint8_t*>(a.kv), a.num_pages,
                     page_shift, a.bt, a.bt_stride, a.lens, a.max_len, a.indices, a.k, a.n_heads, sm_log2,
                     a.num_splits, a.split_tokens, n_hg, a.o_part, a.lse_part, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
