// dsa_indexer_scores kernel: streams the paged indexer-key pool once and
// scores every history token on MFMA.
//
// score(b, t) = sum_h w[b,h] * max(0, q_idx[b,h,:] . key(b,t)) (times the
// token's FP8 scale, which is positive and so commutes with the ReLU).
//
// Work split: one workgroup (4 waves) per (request, chunk of kIdxChunk
// tokens); the chunk's page ids are resolved into LDS first, so the key loads
// never wait on a block-table load.  Each wave streams 64 tokens per step with
// fully coalesced 16-byte loads (one page of 64 FP8 keys is 8 KiB of
// consecutive bytes), always one step ahead (two register buffers), and
// transposes them into MFMA operand order through its own LDS rows.  The math
// is done in 16-token sub-blocks: S[heads x 16 tokens] = Q[heads x d] .
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
constexpr int kIdxChunk = 4096;         // tokens per workgroup
constexpr int kIdxStepBytes = 8192;     // key bytes a wave fetches per step

// Tokens a wave handles per step: 8 KiB of keys, at least one 16-token MFMA block.
template <int ROW_BYTES>
struct IdxStep {
  static constexpr int tok = ROW_BYTES * 64 <= kIdxStepBytes ? 64 : ROW_BYTES * 32 <= kIdxStepBytes ? 32 : 16;
};

// Flat workgroup id -> logical id such that consecutive logical ids share an
// XCD (the dispatcher deals workgroups round-robin over the 8 XCDs, each with
// its own L2), so the chunks of one request reuse its query in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

template <class Op, int KDT, int KSTEPS, int MT>
__global__ __launch_bounds__(kIdxThreads) void indexer_kernel(
    const void* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_pool,
    const float* __restrict__ k_scale, int32_t num_pages, int32_t page_shift,
    const int32_t* __restrict__ bt, int32_t bt_stride, const int32_t* __restrict__ lens, int64_t max_len,
    int32_t n_heads, float* __restrict__ scores, int64_t score_stride, int32_t* __restrict__ status,
    int32_t chunks_per_req) {
  constexpr int KPL = Op::KPL;
  constexpr int D = KSTEPS * 4 * KPL;            // key dim
  constexpr int GROUP_ELEMS = D / 4;             // contiguous elements a lane group owns
  constexpr int ROW_BYTES = D * Storage<KDT>::bytes;
  constexpr int GROUP_BYTES = GROUP_ELEMS * Storage<KDT>::bytes;
  constexpr int RAW_DW = (GROUP_BYTES + 3) / 4;
  constexpr bool kBf = std::is_same<Op, OpBF16>::value;
  constexpr int QE = kBf ? 2 : 4;                // query element bytes
  constexpr int STEP_TOK = IdxStep<ROW_BYTES>::tok;  // tokens per wave step
  constexpr int SUBS = STEP_TOK / 16;                // 16-token MFMA blocks per step
  constexpr int WG_STEP = 4 * STEP_TOK;              // tokens per workgroup step
  constexpr int STEP_BYTES = STEP_TOK * ROW_BYTES;
  static_assert(ROW_BYTES % 16 == 0 && GROUP_BYTES % 4 == 0, "key rows must be whole 16-byte pieces");
  constexpr int PIECES = STEP_BYTES / 16;        // 16-byte pieces per wave step
  constexpr int LOADS = (PIECES + 63) / 64;      // coalesced 16-byte loads per lane per step
  constexpr int ROW_PIECES = ROW_BYTES / 16;
  constexpr int LROW = ROW_BYTES + 16;           // padded LDS row (conflict-free slice reads)
  const int page_size = 1 << page_shift;

  __shared__ int32_t pg[kIdxChunk / 16 + 1];     // page ids of the chunk (-1: bad)
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][STEP_TOK * LROW];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int b = logical / chunks_per_req;
  const int chunk = logical % chunks_per_req;
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

  // Resolve the chunk's pages once (t_begin is a multiple of the page size).
  const int64_t pg0 = t_begin >> page_shift;
  const int n_pg = (int)(((t_end - 1) >> page_shift) - pg0 + 1);
  bool flagged = false;
  for (int i = threadIdx.x; i < n_pg; i += kIdxThreads) {
    int32_t p = bt[(int64_t)b * bt_stride + pg0 + i];
    if (p < 0 || p >= num_pages) {
      p = -1;
      flagged = true;
    }
    pg[i] = p;
  }
  if (flagged && status) atomicOr(status + b, kBadPage);

  // Query fragments (A operand: rows = heads), permuted like the key slices.
  typename Op::frag qa[MT][KSTEPS];
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + r16;
    if (h < n_heads) {
      uint32_t raw[(GROUP_ELEMS * QE + 3) / 4];
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(q_idx) + (((int64_t)b * n_heads + h) * D + g * GROUP_ELEMS) * QE;
      load_raw<GROUP_ELEMS * QE>(qp, raw);
      raw_to_frags<Op, kBf ? kBF16 : kF32, KSTEPS>(raw, qa[mt]);
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
  __syncthreads();  // pg[] ready

  float* sc_out = scores + (int64_t)b * score_stride;
  uint8_t* my_stage = stage[wv];

  // Row of token t of the chunk (>= 0), -1 past the end, -2 on a bad page.
  auto row_of = [&](int64_t t) __attribute__((always_inline)) -> int64_t {
    if (t >= t_end) return -1;
    const int32_t page = pg[(int)((t >> page_shift) - pg0)];
    if (page < 0) return -2;
    return ((int64_t)page << page_shift) + (t & (page_size - 1));
  };

  // A wave step covers tokens [t0 + STEP_TOK wv, +STEP_TOK).  Its key bytes are fetched as
  // 16-byte pieces in token-major order, lane l taking piece 64 i + l of load
  // i, so every load instruction reads 1 KiB of consecutive row bytes (a page
  // is contiguous), with non-temporal loads since every key is read once per
  // step.  The loads are unconditional (a piece past the end reads
  // row 0, which always exists, and is never used), so the compiler can count
  // them and keep the next step's loads in flight during this step's math.
  uint32_t raw_a[LOADS][4], raw_b[LOADS][4];
  float sc_a = 1.f, sc_b = 1.f;
  auto issue = [&](int64_t t0, uint32_t (*raw)[4], float& sc) __attribute__((always_inline)) {
    const int64_t tw = t0 + wv * STEP_TOK;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int piece = min(i * 64 + lane, PIECES - 1);
      const int64_t row = row_of(tw + piece / ROW_PIECES);
      const int64_t safe = row >= 0 ? row : 0;
      load_nt16(k_pool + safe * ROW_BYTES + (piece % ROW_PIECES) * 16, raw[i]);
    }
    if constexpr (KDT == kFP8) {
      const int64_t row = row_of(tw + min(lane, STEP_TOK - 1));
      sc = k_scale[row >= 0 ? row : 0];
    }
  };
  auto consume = [&](int64_t t0, const uint32_t (*raw)[4], float sc) __attribute__((always_inline)) {
    const int64_t tw = t0 + wv * STEP_TOK;
    // Transpose through the wave's own LDS rows (padded by 16 bytes).
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int piece = i * 64 + lane;
      if (piece < PIECES)
        *reinterpret_cast<uint4*>(my_stage + (piece / ROW_PIECES) * LROW + (piece % ROW_PIECES) * 16) =
            make_uint4(raw[i][0], raw[i][1], raw[i][2], raw[i][3]);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < SUBS; ++j) {
      const int tok = j * 16 + r16;  // token of this lane's MFMA column
      uint32_t sl[RAW_DW];
      const uint8_t* src = my_stage + tok * LROW + g * GROUP_BYTES;
#pragma unroll
      for (int x = 0; x < RAW_DW; x += 4) {
        if (x + 4 <= RAW_DW) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * x);
          sl[x] = v.x; sl[x + 1] = v.y; sl[x + 2] = v.z; sl[x + 3] = v.w;
        } else {
#pragma unroll
          for (int y = x; y < RAW_DW; ++y) sl[y] = *reinterpret_cast<const uint32_t*>(src + 4 * y);
        }
      }
      typename Op::frag kb[KSTEPS];
      raw_to_frags<Op, KDT, KSTEPS>(sl, kb);
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
      const float tsc = __shfl(sc, tok);
      const int64_t t = tw + tok;
      if (g == 0 && t < t_end) sc_out[t] = row_of(t) == -2 ? __uint_as_float(0x7FC00000u) : v * tsc;
    }
    __builtin_amdgcn_wave_barrier();
  };

  issue(t_begin, raw_a, sc_a);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * WG_STEP) {
    // Issued unconditionally so that the wait before consume() only covers
    // the older buffer.
    issue(t0 + WG_STEP, raw_b, sc_b);
    consume(t0, raw_a, sc_a);
    if (t0 + WG_STEP >= t_end) break;
    issue(t0 + 2 * WG_STEP, raw_a, sc_a);
    consume(t0 + WG_STEP, raw_b, sc_b);
  }
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
