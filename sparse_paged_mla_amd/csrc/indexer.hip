// dsa_indexer_scores kernel: streams the paged indexer-key pool once and
// scores every history token on MFMA.
//
// score(b, t) = sum_h w[b,h] * max(0, q_idx[b,h,:] . key(b,t)) (times the
// token's FP8 scale, which is positive and so commutes with the ReLU).
//
// Work split: one workgroup (4 waves) per (request, chunk of kChunk tokens).
// A wave scores 16 tokens per step: S[heads x 16 tokens] = Q[heads x d] .
// K^T[d x 16 tokens] with the heads on the MFMA's M side (the query stays in
// registers for the whole chunk) and the tokens on N, so each lane loads a
// contiguous slice of one key row straight from HBM.  Because a dot product
// may sum its terms in any order, lane group g owns the contiguous quarter
// [g*d/4, (g+1)*d/4) of the key row and k-step s takes KPL elements of it;
// the query fragments use the same permutation.  The ReLU-weighted head sum
// is a per-lane sum over the 4 rows it holds per M-tile plus two xor shuffles.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kIdxThreads = 256;
constexpr int kIdxChunk = 4096;  // tokens per workgroup

template <class Op, int KDT, int KSTEPS, int MT>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(
    const void* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_pool,
    const float* __restrict__ k_scale, int32_t num_pages, int32_t page_shift,
    const int32_t* __restrict__ bt, int32_t bt_stride, const int32_t* __restrict__ lens, int64_t max_len,
    int32_t n_heads, float* __restrict__ scores, int64_t score_stride, int32_t* __restrict__ status,
    int32_t chunks_per_req) {
  constexpr int KPL = Op::KPL;
  constexpr int D = KSTEPS * 4 * KPL;            // key dim
  constexpr int GROUP_ELEMS = D / 4;             // contiguous elements a lane group loads
  constexpr int ROW_BYTES = D * Storage<KDT>::bytes;
  constexpr int GROUP_BYTES = GROUP_ELEMS * Storage<KDT>::bytes;
  constexpr int RAW_DW = (GROUP_BYTES + 3) / 4;
  const int page_size = 1 << page_shift;

  const int b = blockIdx.x / chunks_per_req;
  const int chunk = blockIdx.x % chunks_per_req;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;

  const int32_t L = lens[b];
  if (L < 0 || (int64_t)L > max_len || (int64_t)L > (int64_t)bt_stride * page_size) {
    if (chunk == 0 && threadIdx.x == 0 && status) atomicOr(status + b, kBadLen);
    return;
  }
  const int64_t t_begin = (int64_t)chunk * kIdxChunk;
  if (t_begin >= L) return;
  const int64_t t_end = min((int64_t)L, t_begin + kIdxChunk);

  // Query fragments (A operand: rows = heads), permuted like the key loads.
  typename Op::frag qa[MT][KSTEPS];
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + r16;
    if (h < n_heads) {
      uint32_t raw[(GROUP_ELEMS * (std::is_same<Op, OpBF16>::value ? 2 : 4) + 3) / 4];
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(q_idx) +
                          (((int64_t)b * n_heads + h) * D + g * GROUP_ELEMS) *
                              (std::is_same<Op, OpBF16>::value ? 2 : 4);
      if constexpr (std::is_same<Op, OpBF16>::value) {
        load_raw<GROUP_ELEMS * 2>(qp, raw);
        raw_to_frags<Op, kBF16, KSTEPS>(raw, qa[mt]);
      } else {
        load_raw<GROUP_ELEMS * 4>(qp, raw);
        raw_to_frags<Op, kF32, KSTEPS>(raw, qa[mt]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qa[mt][s] = zero_frag<Op>();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = mt * 16 + g * 4 + i;
      wr[mt][i] = hh < n_heads ? w[(int64_t)b * n_heads + hh] : 0.f;
    }
  }

  const int32_t* btb = bt + (int64_t)b * bt_stride;
  float* sc_out = scores + (int64_t)b * score_stride;
  bool flagged = false;

  // Per-lane token of a step; resolve its row (or -1 if masked, -2 if bad page).
  auto row_of = [&](int64_t t0) -> int64_t {
    const int64_t t = t0 + wv * 16 + r16;
    if (t >= t_end) return -1;
    const int32_t page = btb[t >> page_shift];
    if (page < 0 || page >= num_pages) return -2;
    return ((int64_t)page << page_shift) + (t & (page_size - 1));
  };
  auto load_row = [&](int64_t row, uint32_t* raw) {
    if (row >= 0) {
      load_raw<GROUP_BYTES>(k_pool + row * ROW_BYTES + g * GROUP_BYTES, raw);
    } else {
#pragma unroll
      for (int i = 0; i < RAW_DW; ++i) raw[i] = 0u;
    }
  };

  int64_t row_cur = row_of(t_begin);
  uint32_t raw_cur[RAW_DW];
  load_row(row_cur, raw_cur);
  float scale_cur = (KDT == kFP8 && row_cur >= 0) ? k_scale[row_cur] : 1.f;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += 64) {
    // Prefetch the next step's row while this one is on the matrix cores.
    const int64_t t0n = t0 + 64;
    int64_t row_nxt = -1;
    uint32_t raw_nxt[RAW_DW];
    float scale_nxt = 1.f;
    if (t0n < t_end) {
      row_nxt = row_of(t0n);
      load_row(row_nxt, raw_nxt);
      if (KDT == kFP8 && row_nxt >= 0) scale_nxt = k_scale[row_nxt];
    } else {
#pragma unroll
      for (int i = 0; i < RAW_DW; ++i) raw_nxt[i] = 0u;
    }

    typename Op::frag kb[KSTEPS];
    raw_to_frags<Op, KDT, KSTEPS>(raw_cur, kb);
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = Op::mma(qa[mt][s], kb[s], acc[mt]);
    }
    float v = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v += wr[mt][i] * fmaxf(acc[mt][i], 0.f);
    }
    v = wave_sum_xor16_32(v);
    const int64_t t = t0 + wv * 16 + r16;
    if (g == 0 && t < t_end) {
      float outv = v * scale_cur;
      if (row_cur == -2) {
        outv = __uint_as_float(0x7FC00000u);
        flagged = true;
      }
      sc_out[t] = outv;
    }
    row_cur = row_nxt;
    scale_cur = scale_nxt;
#pragma unroll
    for (int i = 0; i < RAW_DW; ++i) raw_cur[i] = raw_nxt[i];
  }
  if (flagged && status) atomicOr(status + b, kBadPage);
}

template <class Op, int KDT, int KSTEPS, int MT>
static int launch_one(const IndexerArgs& a, hipStream_t stream) {
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  const int64_t chunks = (a.max_len + kIdxChunk - 1) / kIdxChunk;
  const int64_t grid = (int64_t)a.batch * (chunks > 0 ? chunks : 1);
  if (a.batch == 0 || a.max_len == 0) return 0;
  if (grid > 0x7FFFFFFF) return -2;
  hipLaunchKernelGGL((indexer_kernel<Op, KDT, KSTEPS, MT>), dim3((unsigned)grid), dim3(kIdxThreads), 0, stream,
                     a.q_idx, a.w, reinterpret_cast<const uint8_t*>(a.k_pool), a.k_scale, a.num_pages, page_shift,
                     a.bt, a.bt_stride, a.lens, a.max_len, a.n_heads, a.scores, a.score_stride, a.status,
                     (int32_t)(chunks > 0 ? chunks : 1));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <class Op, int KDT, int KSTEPS>
static int dispatch_heads(const IndexerArgs& a, hipStream_t s) {
  if (a.n_heads <= 16) return launch_one<Op, KDT, KSTEPS, 1>(a, s);
  if (a.n_heads <= 32) return launch_one<Op, KDT, KSTEPS, 2>(a, s);
  if (a.n_heads <= 64) return launch_one<Op, KDT, KSTEPS, 4>(a, s);
  if (a.n_heads <= 128) return launch_one<Op, KDT, KSTEPS, 8>(a, s);
  return -2;
}

template <class Op, int KDT>
static int dispatch_dim(const IndexerArgs& a, hipStream_t s) {
  constexpr int K = 4 * Op::KPL;
  switch (a.d) {
    case 16: if constexpr (16 % K == 0) return dispatch_heads<Op, KDT, 16 / K>(a, s); else return -2;
    case 32: return dispatch_heads<Op, KDT, 32 / K>(a, s);
    case 64: return dispatch_heads<Op, KDT, 64 / K>(a, s);
    case 128: return dispatch_heads<Op, KDT, 128 / K>(a, s);
    case 256: return dispatch_heads<Op, KDT, 256 / K>(a, s);
    default: return -2;
  }
}

int launch_indexer(const IndexerArgs& a, hipStream_t s) {
  if (a.q_dtype == kF32) {
    switch (a.k_dtype) {
      case kF32: return dispatch_dim<OpF32, kF32>(a, s);
      case kBF16: return dispatch_dim<OpF32, kBF16>(a, s);
      case kFP8: return dispatch_dim<OpF32, kFP8>(a, s);
    }
  } else if (a.q_dtype == kBF16) {
    switch (a.k_dtype) {
      case kBF16: return dispatch_dim<OpBF16, kBF16>(a, s);
      case kFP8: return dispatch_dim<OpBF16, kFP8>(a, s);
    }
  }
  return -2;
}

}  // namespace spmla
