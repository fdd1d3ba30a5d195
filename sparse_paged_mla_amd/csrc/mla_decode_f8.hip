// mla_paged_decode for an FP8 e4m3 latent cache with a per-token scale, bf16
// query, 512 latent + 64 rope dims: split-KV MLA decode over the selected
// tokens, both contractions on MFMA, with the waves of a workgroup
// specialised by role so that vector work on one wave of a SIMD overlaps
// matrix work on the other.
//
// Workgroup = (request b, split s, group of HW query heads); 8 waves.  HW is
// 64, or 32 when a call has so few (request, split) pairs that 64-head
// groups would leave more than half of the CUs without a workgroup (twice
// the workgroups then share the same tiles, each with half the matrix work).
//  - Waves 0-3, score waves: wave (hq, th) holds the query of heads
//    hq*HW/2.. (HW/2 heads) of the group and computes, for every 32-token
//    tile, the scores of those heads against the tile's tokens
//    16th..16th+15 over all 576 dims, then their softmax weights.  Latent
//    dims: the scaled FP8 MFMA (16x16x128, tokens on M, heads on N) against
//    the query written as two scaled e4m3 terms per 128-dim block (the cache
//    codes are used as they are); rope dims: the bf16 MFMA with the codes
//    widened exactly in registers.  The weights go to LDS as bf16, already
//    multiplied by each token's FP8 scale.
//  - Waves 4-7, value waves: each accumulates O[32 heads x 512 * 32 / HW
//    dims] += P[32 heads x 32 tokens] . V[32 tokens x those dims] on the
//    32x32x16 bf16 MFMA, one tile behind the score waves (64 heads: two head
//    tiles x two dim halves; 32 heads: one head tile x four dim quarters).
//    V comes from the same LDS tile through gfx950's 8-bit transposing LDS
//    read and is widened exactly to bf16 in registers.  These waves also
//    fetch the tiles: every lane's 16-byte piece of a tile goes straight from
//    HBM into LDS (global_load_lds_dwordx4), so a tile costs no registers and
//    no vector instructions to stage.
// With waves w and w + 4 on the same SIMD, each SIMD runs one wave of each
// role.  Tiles rotate through kNB LDS buffers and are requested kPF tiles
// ahead of the one being scored; one barrier per tile.
//
// LDS tile layout: 608-byte rows (36 16-byte chunks of codes, 2 spare), and
// bit 0 of a row's chunk index flipped on rows r with bit 3 of r differing
// from bit 4: the score reads, the rope reads and the transposing value
// reads are then free of bank conflicts.  The direct loads fill whole 1 KiB
// blocks (one per wave instruction), so the spare chunks are filled with a
// repeat of the row's last chunk.
//
// The waits for the direct loads are explicit (the compiler does not track
// them): each value wave issues exactly kLoads loads per tile, so "tile i + 1
// has landed" is "at most kLoads * (kPF - 1) loads outstanding".  Barriers
// are s_barrier with the wave's LDS operations drained first, without the
// fence __syncthreads() carries (that fence would also wait for every direct
// load in flight).
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

#include <atomic>
#include <utility>

namespace spmla {
namespace {
using namespace ws;

constexpr int kThreads = 512;
constexpr int kTileTok = 32;
constexpr int kD = 576, kDC = 512;
constexpr int kRS = 608;                          // LDS row stride (bytes)
constexpr int kRowChunks = kRS / 16;              // 38 chunk slots per row
constexpr int kTileBytes = kTileTok * kRS;        // 19456
constexpr int kRowLoads = kTileBytes / 1024;      // 19 wave loads of 1 KiB per tile
constexpr int kLoads = 5;                         // per value wave per tile: 19 row loads + 1 scale load
constexpr int kPF = 2;                            // tiles requested ahead of the scored one (2 measured
                                                  // faster than 3 or 4: the loads still land in time)
constexpr int kSeg = 1024;                        // positions resolved at once
constexpr int kMaxDev = 64;                       // devices whose CU count is cached
constexpr int kPStride = 40;                      // bf16 per weight row (32 tokens + 8 pad)
constexpr float kHeadroom = 16.f;
static_assert(kTileBytes % 1024 == 0 && kRowLoads + 1 == 4 * kLoads, "tile loads split evenly");
static_assert(kLoads * (kPF - 1) <= 63, "vmcnt range");

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i;
typedef __attribute__((address_space(3))) void lds_void;

// A zero row and a unit scale: what a masked position loads, so every load
// is unconditional and a masked token scores exactly 0 before its -inf bias.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kD];
__device__ __attribute__((aligned(16))) float g_unit_scale[4] = {1.f, 1.f, 1.f, 1.f};

__device__ __forceinline__ int swz(int r) { return ((r >> 3) ^ (r >> 4)) & 1; }

// Four FP8 codes per dword, two dwords -> 8 bf16 values, exactly.
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  const bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

template <int HW>
__global__ __launch_bounds__(kThreads) void mla_decode_f8ws_kernel(
    const __bf16* __restrict__ q, const uint8_t* __restrict__ kv, const float* __restrict__ kv_scale,
    int32_t num_pages, int32_t page_shift, const int32_t* __restrict__ bt, int32_t bt_stride,
    const int32_t* __restrict__ lens, int64_t max_len, const int32_t* __restrict__ indices, int32_t k,
    int32_t n_heads, float sm_scale_log2, int32_t num_splits, int32_t split_tok, int32_t n_hg,
    float* __restrict__ o_part,
    float* __restrict__ lse_part, int32_t* __restrict__ status) {
  // HW heads per workgroup: 64, or 32 when a call has too few (request,
  // split) pairs to fill the GPU with 64-head groups.
  constexpr int kHeadsWg = HW;
  constexpr int NT = HW / 32;              // 16-head N-tiles of a score wave (it holds HW / 2 heads)
  constexpr int kDimParts = 128 / HW;      // value waves per 32-head tile: 2, or 4
  constexpr int kVDims = kDC / kDimParts;  // output dims of a value wave: 256, or 128
  constexpr int NTV = kVDims / 32;         // its 32-dim N-tiles
  constexpr int kHG16 = HW / 16;           // 16-head groups of the staged query
  constexpr int kQBufs = HW == 64 ? 4 : 2; // buffers holding the staged query; tile t of a segment
                                           // lives in buffer (t + kQBufs) % kNB
  constexpr int kNB = kQBufs + 2;          // tile buffers
  static_assert(HW == 64 || HW == 32, "head groups of 64 or 32");
  static_assert(kNB >= kPF + 2, "a tile buffer is refilled only after both roles are done with it");
  __shared__ __attribute__((aligned(16))) uint8_t Kbuf[kNB][kTileBytes];
  __shared__ __attribute__((aligned(16))) float Tsc[kNB][64];          // FP8 scales of a tile's rows (32 used)
  __shared__ __attribute__((aligned(16))) int32_t seg_row[kSeg];        // cache row, or -1 when masked
  __shared__ __attribute__((aligned(16))) float seg_bias[kSeg];         // 0, or -inf when masked
  __shared__ __attribute__((aligned(16))) __bf16 Pbuf[2][kHeadsWg * kPStride];
  __shared__ __attribute__((aligned(16))) float red[2][kHeadsWg];       // per token half: head maxima / sums
  __shared__ __attribute__((aligned(16))) bf16x8 Qrope[kHG16][2][64];   // [head tile of 16][ks][lane]: rope dims
  __shared__ __attribute__((aligned(16))) uint8_t Qsc[kHeadsWg][2][4];  // E8M0 scale per head, term and block
  __shared__ int redo_flag;
  __shared__ int bad_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wv < 4;
  const int role = wv & 3;
  const int hq = role >> 1;            // score waves: heads hq * HW / 2.. of the group
  const int th = role & 1;             // score waves: token half of each tile
  const int vht = role / kDimParts;    // value waves: heads 32vht..32vht+31 of the group
  const int dpart = role % kDimParts;  // value waves: output dims kVDims * dpart..
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

  // ---- value waves' share of each tile: row loads 4w'..4w'+3 and (w' <
  // 3) 16 + w' of the tile's 19 (w' = role); wave 3's fifth load is the
  // tile's scales.  Piece p of a load lands at slot p of the tile: row p /
  // 38, chunk slot p % 38, which holds chunk (p % 38) ^ swz(row) of the row
  // (the two spare slots repeat chunk 35).
  int ld_off[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int ld = u < 4 ? 4 * role + u : 16 + role;
    const int slot = 64 * ld + lane;
    const int r = min(slot / kRowChunks, kTileTok - 1);
    const int c = min((slot % kRowChunks) ^ swz(r), kD / 16 - 1);
    ld_off[u] = (r << 8) | c;
  }
  // Tile row of this lane's piece of load u (the scale load: row lane % 32).
  auto piece_row = [&](int u) { return (u < 4 || role < 3) ? ld_off[u] >> 8 : lane & 31; };

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

  // ---- the query of the group's heads is staged in LDS next (it depends
  // on nothing): tile buffers 0..kQBufs-1, free until those buffers are
  // first requested.  Layout: the latent dims as [half][head][32 chunks of
  // 16 bytes] (half hv = dims 256hv..256hv+255), then the rope dims as
  // [head][8 chunks]; chunk c of head h sits at slot c ^ (h % 16) (rope:
  // c ^ (h % 8)), so that the 16 heads a lane group reads at once fall on
  // distinct LDS banks.  A query wave stages half hv of 16 heads 16hw.. (8
  // wave loads; those with hv = 0 also their rope dims, 2 more), so the wave
  // that converts them (below) needs no other wave's loads.  Heads past the
  // last one stage head 0's query: their results are never stored.
  constexpr int kQLat = 0, kQRope = 2 * kHeadsWg * 512;
  static_assert(kQRope + kHeadsWg * 128 <= kQBufs * kTileBytes && kNB - kQBufs >= 2,
                "the staged query fits below the buffers of tiles 0 and 1");
  // Query waves: all 8 for 64 heads (wave w: half w / 4 of heads
  // 16(w % 4)..), waves 0-3 for 32 heads (half w / 2 of heads 16(w % 2)..).
  const bool q_wave = wv < 2 * kHG16;
  const int hv = wv / kHG16, hw = wv % kHG16;
  if (q_wave) {
    const uint32_t qs_lds = lds_addr(&Kbuf[0][0]);
    const __bf16* qb = q + (int64_t)b * n_heads * kD;
    auto qrow = [&](int hl) { const int h = head_base + hl; return qb + (int64_t)(h < n_heads ? h : 0) * kD; };
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = 64 * u + lane, hh = p / 32;
      dma16(qrow(16 * hw + hh) + 256 * hv + 8 * ((p % 32) ^ hh), qs_lds + kQLat + (hv * kHeadsWg + 16 * hw) * 512 + 1024 * u);
    }
    if (hv == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = 64 * u + lane, hh = p / 8;
        dma16(qrow(16 * hw + hh) + kDC + 8 * ((p % 8) ^ (hh & 7)), qs_lds + kQRope + 16 * hw * 128 + 1024 * u);
      }
    }
  }

  const int32_t L = lens[b];
  if (L < 0 || (int64_t)L > max_len || (int64_t)L > (int64_t)bt_stride * page_size) {
    vm_wait<0>();  // the staged query is not needed, but the loads must land before the workgroup ends
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
  // the compiler cannot move the load into the branch of the select (a load
  // under a branch is waited for inside it, one memory latency per load).
  // Dense calls have no index array: they read the block table's first
  // entry and do not use it.
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

  // Resolve positions [seg, seg_end) of the split (index -> page -> row);
  // entries past seg_end are masked.
  auto build_table = [&](int64_t seg, int64_t seg_end) __attribute__((always_inline)) {
    int64_t pos[kSeg / kThreads], t[kSeg / kThreads];
#pragma unroll
    for (int u = 0; u < kSeg / kThreads; ++u) pos[u] = seg + tid + u * kThreads;
    tokens_at(pos, seg_end, t);
    int32_t page[kSeg / kThreads];
    pages_of(t, page, std::integral_constant<int, kSeg / kThreads>{});
#pragma unroll
    for (int u = 0; u < kSeg / kThreads; ++u) {
      int32_t row = -1;
      if (t[u] < -1 || t[u] >= L) {
        bad_flag = 1;
        if (status) atomicOr(status + b, kBadIndex);
      } else if (t[u] >= 0) {
        if (page[u] < 0 || page[u] >= num_pages) {
          bad_flag = 1;
          if (status) atomicOr(status + b, kBadPage);
        } else {
          row = (int32_t)(((int64_t)page[u] << page_shift) + (t[u] & (page_size - 1)));
        }
      }
      seg_row[tid + u * kThreads] = row;
      seg_bias[tid + u * kThreads] = row >= 0 ? 0.f : -INFINITY;
    }
  };
  const uint8_t* zero_row = g_zero_row;
  const float* unit_scale = g_unit_scale;
  // Send this lane's loads of a tile whose pieces come from cache rows
  // row[u] (-1: masked, the zero row) into buffer `buf`.
  auto dma_rows = [&](const int32_t (&row)[kLoads], int buf) __attribute__((always_inline)) {
    const uint32_t dst = lds_addr(&Kbuf[0][0]) + buf * kTileBytes;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      if (u < 4 || role < 3) {
        const int ld = u < 4 ? 4 * role + u : 16 + role;
        const int c = ld_off[u] & 255;
        const uint8_t* src = row[u] >= 0 ? kv + ((int64_t)row[u] * (kD / 16) + c) * 16 : zero_row + 16 * c;
        dma16(src, dst + 1024 * ld);
      } else {
        const float* src = row[u] >= 0 ? kv_scale + row[u] : unit_scale;
        dma4(src, lds_addr(&Tsc[0][0]) + buf * 256);
      }
    }
  };

  // ---- prologue: once the indices are in, the first segment's pages are
  // requested, and while they load each wave rewrites its staged part of
  // the query in place as two scaled FP8 terms per 128-dim latent block
  // (lane (r16, g) converts blocks 2hv and 2hv + 1 of head 16(w % 4) + r16
  // with the lane layout the score waves use, the 64 bytes it read becoming
  // its 32 hi and 32 lo codes).  The value waves first resolve their pieces
  // of tiles 0 and 1 and request those tiles.  The score waves then load the
  // codes into registers.
  if (!any_token) vm_wait<0>();  // nothing to score: just let the early loads land
  if (any_token) {
    uint8_t* const qs = &Kbuf[0][0];
    const int64_t seg_end = min(p_end, p_begin + kSeg);
    vm_wait<0>();  // the indices are in, this wave's part of the query is staged
    int32_t t[kNP], pv[kNP];
#pragma unroll
    for (int i = 0; i < kNP; ++i) {
      const int64_t p = pos_at(p_begin, i);
      t[i] = p < seg_end ? (sparse ? iv[i] : (int32_t)p) : -1;
      pv[i] = btb[(t[i] >= 0 && t[i] < L ? t[i] : 0) >> page_shift];
    }
    auto pages_in = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kNP; ++i) asm volatile("" : "+v"(pv[i]));
    };
    auto convert = [&]() __attribute__((always_inline)) {
      const int hl = 16 * hw + r16;
      // block bb: chunks 16bb + 2g, +1 (dims 128(2hv + bb) + 16g..+15) and
      // 16bb + 8 + 2g, +1 (64 dims on); both blocks are read before either
      // is written back
      uint8_t* row = qs + kQLat + (hv * kHeadsWg + hl) * 512;
      uint4* q4[2][4];
      uint4 raw[2][4];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int c0 = 16 * bb + 2 * g;
        q4[bb][0] = reinterpret_cast<uint4*>(row + 16 * (c0 ^ r16));
        q4[bb][1] = reinterpret_cast<uint4*>(row + 16 * ((c0 + 1) ^ r16));
        q4[bb][2] = reinterpret_cast<uint4*>(row + 16 * ((c0 + 8) ^ r16));
        q4[bb][3] = reinterpret_cast<uint4*>(row + 16 * ((c0 + 9) ^ r16));
#pragma unroll
        for (int j = 0; j < 4; ++j) raw[bb][j] = *q4[bb][j];
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const uint4* r = raw[bb];
        const uint32_t w[16] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w,
                                r[2].x, r[2].y, r[2].z, r[2].w, r[3].x, r[3].y, r[3].z, r[3].w};
        v8i_t hi, lo;
        int shi, slo;
        split_q32(w, hi, lo, shi, slo);
        *q4[bb][0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *q4[bb][1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        *q4[bb][2] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *q4[bb][3] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
        // the four lanes of a row hold the same scales
        Qsc[hl][0][2 * hv + bb] = (uint8_t)shi;
        Qsc[hl][1][2 * hv + bb] = (uint8_t)slo;
      }
      if (hv == 0) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 r = *reinterpret_cast<const uint4*>(qs + kQRope + hl * 128 + 16 * ((4 * ks + g) ^ (hl & 7)));
          Qrope[hw][ks][lane] = __builtin_bit_cast(bf16x8, r);
        }
      }
    };
    if (score_wave) {
      convert();  // score waves are query waves for either head count
      pages_in();
    } else {
      pages_in();
      int32_t prow[2][kLoads];
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
          const int32_t tt = t[kNT + tl * kLoads + u], pp = pv[kNT + tl * kLoads + u];
          prow[tl][u] = tt >= 0 && tt < L && pp >= 0 && pp < num_pages ? (int32_t)(((int64_t)pp << page_shift) + (tt & (page_size - 1))) : -1;
        }
      }
      dma_rows(prow[0], kQBufs);
      dma_rows(prow[1], kQBufs + 1);
      if (q_wave) convert();
    }
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      int32_t row = -1;
      if (t[u] < -1 || t[u] >= L) {
        bad_flag = 1;
        if (status) atomicOr(status + b, kBadIndex);
      } else if (t[u] >= 0) {
        if (pv[u] < 0 || pv[u] >= num_pages) {
          bad_flag = 1;
          if (status) atomicOr(status + b, kBadPage);
        } else {
          row = (int32_t)(((int64_t)pv[u] << page_shift) + (t[u] & (page_size - 1)));
        }
      }
      seg_row[tid + u * kThreads] = row;
      seg_bias[tid + u * kThreads] = row >= 0 ? 0.f : -INFINITY;
    }
    wg_barrier();  // the query's FP8 terms and the first table are in LDS
  }

  int64_t built = any_token ? p_begin : -1;  // segment whose table is in LDS
  // Both roles run the same sequence of barriers.
  if (score_wave) {
    v8i_t qhi[NT][4], qlo[NT][4];
    uint32_t qs_hi[NT], qs_lo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qs_hi[nt] = qs_lo[nt] = 0;
    // Head of N-tile nt of this score wave (its lane r16), within the group.
    auto shead = [&](int nt) { return hq * (kHeadsWg / 2) + nt * 16 + r16; };
    if (any_token) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int hl = shead(nt);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const uint8_t* row = &Kbuf[0][0] + kQLat + ((blk >> 1) * kHeadsWg + hl) * 512;
          const int cb = 16 * (blk & 1) + 2 * g;  // hi codes in chunks cb, cb + 1; lo codes in cb + 8, cb + 9
          const int hs = hl & 15;
          const uint4 a0 = *reinterpret_cast<const uint4*>(row + 16 * (cb ^ hs));
          const uint4 a1 = *reinterpret_cast<const uint4*>(row + 16 * ((cb + 1) ^ hs));
          const uint4 c0 = *reinterpret_cast<const uint4*>(row + 16 * ((cb + 8) ^ hs));
          const uint4 c1 = *reinterpret_cast<const uint4*>(row + 16 * ((cb + 9) ^ hs));
          qhi[nt][blk] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          qlo[nt][blk] = v8i_t{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
        }
        qs_hi[nt] = *reinterpret_cast<const uint32_t*>(&Qsc[hl][0][0]);
        qs_lo[nt] = *reinterpret_cast<const uint32_t*>(&Qsc[hl][1][0]);
      }
      wg_barrier();  // the query's buffers are free for tiles
    }

    // Scores of the tile in Kt for this wave's 16 tokens (rows 16th + r16 on
    // M) and its 32 heads (two N-tiles): S[nt] holds head 16nt + r16 for
    // tokens 16th + 4g + j.
    auto score_tile = [&](const uint8_t* __restrict__ Kt, f32x4 (&S)[NT]) __attribute__((always_inline)) {
      f32x4 acc[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][0] = acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = th * 16 + r16;
      const int sw = swz(row);
      const uint8_t* rp = Kt + row * kRS;
      static_for<4>([&](auto B) {
        constexpr int blk = decltype(B)::value;
        const uint4 k0 = *reinterpret_cast<const uint4*>(rp + 16 * ((8 * blk + g) ^ sw));
        const uint4 k1 = *reinterpret_cast<const uint4*>(rp + 16 * ((8 * blk + 4 + g) ^ sw));
        const v8i_t a = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qhi[nt][blk], acc[nt][0], 0, 0, 0, 127,
                                                                        blk, (int)qs_hi[nt]);
          acc[nt][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qlo[nt][blk], acc[nt][1], 0, 0, 0, 127,
                                                                        blk, (int)qs_lo[nt]);
        }
      });
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint2 kr = *reinterpret_cast<const uint2*>(rp + 16 * ((32 + 2 * ks + (g >> 1)) ^ sw) + 8 * (g & 1));
        const bf16x8 kb = widen8(kr.x, kr.y);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][1] = OpBF16::mma(kb, Qrope[NT * hq + nt][ks][lane], acc[nt][1]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[nt] = acc[nt][0] + acc[nt][1];
    };

    float m_ref[NT], m_lane[NT], l_lane[NT];   // per N-tile: reference (log2 domain), this lane's
#pragma unroll                                 // largest logit, this lane's sum of weights
    for (int nt = 0; nt < NT; ++nt) m_ref[nt] = m_lane[nt] = -INFINITY;
    bool fallback = false;                     // the first tile had no valid token: 0 stood in for m_ref
    // Softmax weights of a scored tile, written to P as bf16 (times each
    // token's FP8 scale, which the value contraction needs).
    auto softmax_tile = [&](const f32x4 (&S)[NT], int buf, int tb, __bf16* __restrict__ P, bool& over)
        __attribute__((always_inline)) {
      const int t0 = th * 16 + 4 * g;
      const f32x4 ts = *reinterpret_cast<const f32x4*>(&Tsc[buf][t0]);
      const f32x4 bi = *reinterpret_cast<const f32x4*>(&seg_bias[tb + t0]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float z[4], mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[j] = __builtin_fmaf(S[nt][j], sm_scale_log2 * ts[j], bi[j]);
          mx = fmaxf(mx, z[j]);
        }
        m_lane[nt] = fmaxf(m_lane[nt], mx);
        over |= mx > m_ref[nt] + kHeadroom;
        float pv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pp = __builtin_amdgcn_exp2f(z[j] - m_ref[nt]);
          l_lane[nt] += pp;
          pv[j] = pp * ts[j];
        }
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        const bf16x4_t w4 = {(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3]};
        *reinterpret_cast<bf16x4_t*>(P + shead(nt) * kPStride + t0) = w4;
      }
    };

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) l_lane[nt] = 0.f;
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
        f32x4 S[NT];
        score_tile(Kbuf[kQBufs], S);
        if (need_ref) {
          const int t0 = th * 16 + 4 * g;
          const f32x4 ts = *reinterpret_cast<const f32x4*>(&Tsc[kQBufs][t0]);
          const f32x4 bi = *reinterpret_cast<const f32x4*>(&seg_bias[t0]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = fmaxf(mx, __builtin_fmaf(S[nt][j], sm_scale_log2 * ts[j], bi[j]));
            mx = wave_max_xor16_32(mx);
            if (g == 0) red[th][shead(nt)] = mx;
          }
          wg_barrier();
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int hl = shead(nt);
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
        softmax_tile(S, kQBufs, 0, Pbuf[0], over);
        wg_barrier();  // tile 1 has landed; P of tile 0 is written
        int buf = kQBufs + 1;  // buffer of tile i
        for (int i = 1; i <= T; ++i) {
          if (i < T) {
            score_tile(Kbuf[buf], S);
            softmax_tile(S, buf, i * kTileTok, Pbuf[i & 1], over);
          }
          buf = buf == kNB - 1 ? 0 : buf + 1;
          wg_barrier();
        }
      }
      // Recompute the split once if a logit outgrew its head's reference,
      // or if the reference was a stand-in and valid tokens were seen.
      bool seen = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) seen |= m_lane[nt] > -INFINITY;
      if (__any(over || (fallback && seen)) && lane == 0) atomicOr(&redo_flag, 1);
      wg_barrier();
      if (pass == 1 || redo_flag == 0) break;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float mt = wave_max_xor16_32(m_lane[nt]);
        if (g == 0) red[th][shead(nt)] = mt;
      }
      wg_barrier();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int hl = shead(nt);
        m_ref[nt] = fmaxf(red[0][hl], red[1][hl]);
        if (m_ref[nt] == -INFINITY) m_ref[nt] = 0.f;
      }
      fallback = false;
    }
    // ---- finish: l per head from both token halves, then lse.
    wg_barrier();  // red is free again
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float ls = wave_sum_xor16_32(l_lane[nt]);
      if (g == 0) red[th][shead(nt)] = ls;
    }
    wg_barrier();
    const bool bad = bad_flag != 0;
    if (th == 0 && g == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int hl = shead(nt);
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
    // the transposing read hands lane i of each 16-lane group G the dim
    // 16(G & 1) + i of the N-tile for tokens 16ks + 8(G >> 1) + e, e < 8,
    // when lane j of the group points at 8 dims (8(j & 1)..) of token row
    // 16ks + 8(G >> 1) + j / 2.
    auto pv_tile = [&](const uint8_t* __restrict__ Vt, const __bf16* __restrict__ P, f32x16 (&acc_o)[NTV])
        __attribute__((always_inline)) {
      const int G = lane >> 4, j = lane & 15;
      // All LDS reads of the tile are issued before the first MFMA (20
      // registers of codes), so the MFMAs wait for them once instead of one
      // read latency each.
      bf16x8 pa[2];
      v2i_t raw[2][NTV];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pa[ks] = *reinterpret_cast<const bf16x8*>(P + (vht * 32 + (lane & 31)) * kPStride + 16 * ks + 8 * (lane >> 5));
        const int tr = 16 * ks + 8 * (G >> 1) + (j >> 1);
        const int sw = swz(tr);
        const uint8_t* vrow = Vt + tr * kRS + 8 * (j & 1);
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
          const int chunk = (kVDims / 16) * dpart + 2 * nt + (G & 1);
          raw[ks][nt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vrow + 16 * (chunk ^ sw)));
        }
      }
      // Four groups of four independent MFMAs in this order (left to itself
      // the scheduler interleaves each read with its MFMA, one LDS latency
      // per MFMA).
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int h4 = 0; h4 < NTV / 4; ++h4) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int nt = 4 * h4; nt < 4 * h4 + 4; ++nt)
            acc_o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                pa[ks], widen8((uint32_t)raw[ks][nt][0], (uint32_t)raw[ks][nt][1]), acc_o[nt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // (Tiles 0 and 1 went to buffers 4 and 5 with the query.)
    if (any_token) wg_barrier();  // the score waves hold the query: its buffers are free for tiles

    f32x16 acc_o[NTV];
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) acc_o[nt] = f32x16{};
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
        // Tiles 0 and 1 of the split's first segment were requested with
        // the query; the others are requested here.
        const int pre = need_ref ? 2 : 0;
#pragma unroll
        for (int i = 0; i < kPF; ++i)
          if (i >= pre) issue_tile(i, T, (i + kQBufs) % kNB);
        vm_wait<kLoads * (kPF - 1)>();  // tile 0 has landed
        wg_barrier();
        if (need_ref) wg_barrier();
        issue_tile(kPF, T, (kPF + kQBufs) % kNB);
        vm_wait<kLoads * (kPF - 1)>();  // tile 1 has landed
        wg_barrier();
        int buf_in = (kPF + 1 + kQBufs) % kNB, buf_pv = kQBufs;  // buffers of tiles i + kPF and i - 1
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
      const int hl = vht * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const int h = head_base + hl;
      const float l = red[0][hl] + red[1][hl];
      const float inv = bad ? kNaN : (l > 0.f ? 1.f / l : 0.f);
      if (h < n_heads) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) *out_o(h, dpart * kVDims + nt * 32 + (lane & 31)) = acc_o[nt][e] * inv;
      }
    }
  }
}

}  // namespace

int launch_decode_f8(const DecodeArgs& a, hipStream_t stream) {
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  // 32-head groups when 64-head ones would leave more than half of the CUs
  // without a workgroup: twice the workgroups, each with half the matrix
  // work per tile over the same tiles.
  const int64_t pairs = (int64_t)a.batch * a.num_splits;
  if (pairs == 0) return 0;
  static std::atomic<int> n_cu[kMaxDev];  // CU count per device, 0 until first asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return -3;
  int cus = n_cu[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -3;
    n_cu[dev].store(cus, std::memory_order_relaxed);
  }
  const bool narrow = 2 * pairs * ((a.n_heads + 63) / 64) <= cus;
  const int hw = narrow ? 32 : 64;
  const int n_hg = (a.n_heads + hw - 1) / hw;
  const int64_t grid = pairs * n_hg;
  if (grid == 0) return 0;
  if (grid > 0x7FFFFFFF) return -2;
  const float sm_log2 = a.sm_scale * 1.44269504088896340736f;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, reinterpret_cast<const __bf16*>(a.q),
                       reinterpret_cast<const uint8_t*>(a.kv), a.kv_scale, a.num_pages, page_shift, a.bt, a.bt_stride,
                       a.lens, a.max_len, a.indices, a.k, a.n_heads, sm_log2, a.num_splits, a.split_tokens, n_hg, a.o_part, a.lse_part,
                       a.status);
  };
  if (narrow) go(mla_decode_f8ws_kernel<32>);
  else go(mla_decode_f8ws_kernel<64>);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
