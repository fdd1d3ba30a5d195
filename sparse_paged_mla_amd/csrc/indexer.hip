// dsa_indexer_scores kernel: streams the paged indexer-key pool once and
// scores every history token on MFMA.
//
// score(b, t) = sum_h w[b,h] * max(0, q_idx[b,h,:] . key(b,t)) (times the
// token's FP8 scale, which is positive and so commutes with the ReLU).
//
// Work split: the batch's history is cut into steps of STEP_TOK consecutive
// tokens of one request (8 KiB of keys), and every wave of a fixed,
// GPU-filling grid takes an equal contiguous run of the flattened step list,
// which may cross into the next request.  There is no tail of idle workgroups
// and no per-chunk start-up; each wave finds its first step with one scan
// over the request lengths.  A wave streams its steps with fully coalesced
// 16-byte non-temporal loads (a page of 64 FP8 keys is 8 KiB of consecutive
// bytes), always one step ahead (two register buffers), with the block-table
// entries of the step after that already in registers, and transposes each
// step into MFMA operand order through its own LDS rows.  The math is done in
// 16-token sub-blocks: S[heads x 16 tokens] = Q[heads x d] . K^T[d x 16
// tokens] with the heads on the MFMA's M side (the query stays in registers
// while the request does not change) and the tokens on N.  Because a dot
// product may sum its terms in any order, lane group g owns the contiguous
// quarter [g*d/4, (g+1)*d/4) of the key row and k-step s takes KPL elements
// of it; the query fragments use the same permutation.  In the two-query
// kernel FP8 keys of 128 dims skip the widening: the query is held as two
// scaled e4m3 terms (exact for every element within 2^14 of its row's
// largest, off by less than 2^-22 of it otherwise) and each 16x16 block is
// two scaled FP8 MFMAs over the stored key codes.  The ReLU-weighted head
// sum is a per-lane sum over the 4 rows it holds per M-tile plus two xor
// shuffles.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kIdxThreads = 256;
constexpr int kIdxStepBytes = 8192;     // key bytes a wave fetches per step
// Workgroup shape.  One query per request (NQ = 1): four waves, each with
// its own run of steps; two workgroups per compute unit, except for kernels
// holding 8 M-tiles of queries (more than 256 registers per lane: one wave
// per SIMD).  Two queries (NQ = 2): two waves, one per query, sharing each
// step's staged keys; four workgroups per compute unit.
template <int MT, int NQ = 1>
struct IdxWg {
  static constexpr int waves = NQ == 2 ? 2 : 4;
  static constexpr int per_cu = NQ == 2 ? 4 : MT >= 8 ? 1 : 2;
  // Waves per SIMD the compiler is held to: two for the pairs (their budget
  // must stay within 256 registers), no bound otherwise (as measured).
  static constexpr int min_simd_waves = NQ == 2 ? 2 : 1;
  static constexpr int lds = 160 * 1024 / per_cu;
};
constexpr int kIdxMaxHeldSteps = 40;    // steps of scores a wave holds in LDS before writing them
constexpr int kNumCu = 256;

// Tokens a wave handles per step: 8 KiB of keys, at least one 16-token MFMA block.
template <int ROW_BYTES>
struct IdxStep {
  static constexpr int tok = ROW_BYTES * 64 <= kIdxStepBytes ? 64 : ROW_BYTES * 32 <= kIdxStepBytes ? 32 : 16;
};

// Flat workgroup id -> logical id such that consecutive logical ids share an
// XCD (the dispatcher deals workgroups round-robin over the 8 XCDs, each with
// its own L2), so neighbouring runs of steps (mostly the same request) read
// its query through one L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Run of each wave: with two workgroups resident per CU, the two waves that
// share a SIMD do not progress alike (the older wave is issued first), so a
// wave of the workgroup placed first on its CU takes a larger share of the
// steps.  The dispatcher places workgroup ids round-robin over the XCDs and,
// within an XCD, one per CU before the second ones, so with the full grid
// the first half of each XCD's logical range (xcd_remap) is the first-placed
// half.  Shares are (100 + kIdxFirstExtra) : (100 - kIdxFirstExtra); any
// other grid splits evenly.  Wave i's run starts at step run_start(i).
// Measured on c3f (64 requests, 32K-128K tokens, FP8 keys): with even runs
// the first-placed workgroups end at about 96 us and the others at about
// 115; shares 120 : 80 took the kernel from 133 to 129.5 us (108 : 92 and
// 114 : 86 less, 126 : 74 slower again).
constexpr int64_t kIdxFirstExtra = 20;
__device__ __forceinline__ int64_t run_start(int64_t total, int64_t i, int64_t nw, int grid, bool two_per_cu) {
  if (!two_per_cu || grid != 2 * kNumCu || kIdxFirstExtra == 0) return total * i / nw;
  constexpr int64_t kFirst = 100 + kIdxFirstExtra, kSecond = 100 - kIdxFirstExtra;
  constexpr int64_t kPerXcd = 2 * kNumCu / 8, kHalf = kPerXcd / 2;
  const int64_t wg = i >> 2, wv = i & 3;
  const int64_t x = wg / kPerXcd, sl = wg % kPerXcd;
  const int64_t before = x * kHalf * (kFirst + kSecond) + min(sl, kHalf) * kFirst + max<int64_t>(0, sl - kHalf) * kSecond;
  const int64_t wcum = 4 * before + wv * (sl < kHalf ? kFirst : kSecond);
  return total * wcum / (4 * 8 * kHalf * (kFirst + kSecond));
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// MULTI: pages shorter than a step (a step's tokens span several pages).
// A compile-time choice: with both paths in one kernel the compiler's
// memory-wait accounting merges them and waits far more than either needs.
// NQ: queries scored per key read (a multi-query step): the request's NQ
// queries of n_heads heads each are NQ * n_heads consecutive rows and query i
// writes score row b * NQ + i (status entries likewise).  With NQ = 2 a
// workgroup is a pair of waves that walk one run of steps together: each
// loads half of a step's keys into the pair's stage (two buffers, one
// barrier per step) and scores the whole staged step against its own query
// (MT M-tiles of n_heads heads), so each key is read once for both queries
// while every wave keeps the one-query register budget.
template <class Op, int KDT, int KSTEPS, int MT, bool MULTI, int NQ>
__global__ __launch_bounds__(kIdxThreads) __attribute__((amdgpu_waves_per_eu(IdxWg<MT, NQ>::min_simd_waves)))
void indexer_kernel(
    const void* __restrict__ q_idx, const float* __restrict__ w, const uint8_t* __restrict__ k_pool,
    const float* __restrict__ k_scale, int32_t num_pages, int32_t page_shift,
    const int32_t* __restrict__ bt, int32_t bt_stride, const int32_t* __restrict__ lens, int32_t batch,
    int64_t max_len, int32_t n_heads, float* __restrict__ scores, int64_t score_stride,
    int32_t* __restrict__ status) {
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
  constexpr int STEP_BYTES = STEP_TOK * ROW_BYTES;
  static_assert(ROW_BYTES % 16 == 0 && GROUP_BYTES % 4 == 0, "key rows must be whole 16-byte pieces");
  constexpr int PIECES = STEP_BYTES / 16;        // 16-byte pieces per wave step
  constexpr int LOADS = (PIECES + 63) / 64;      // coalesced 16-byte loads per lane per step
  constexpr int ROW_PIECES = ROW_BYTES / 16;
  constexpr int LROW = ROW_BYTES + 16;           // padded LDS row (conflict-free slice reads)
  const int page_size = 1 << page_shift;
  const int64_t bt_cap = (int64_t)bt_stride * page_size;

  // Scores are held in LDS and written once a wave's run (or its part in one
  // request) ends, or when HELD steps are waiting: the stores then come after
  // nearly all of the grid's key reads instead of between them, where each
  // small write costs the reads far more than its bytes.
  static_assert(NQ == 1 || NQ == 2, "one or two queries per request");
  constexpr bool PAIR = NQ == 2;
  constexpr int WAVES = IdxWg<MT, NQ>::waves;
  constexpr int NSTAGE = PAIR ? 2 : 4;  // the pair's two buffers, or one per wave
  // Scaled FP8 MFMA on the stored key codes (FP8 keys of 128 dims, pairs):
  // measured on c3f (64 requests, 32K-128K tokens), the pair kernel 238 ->
  // about 219 us; the one-query kernel 131.5 -> 139 us, so it keeps bf16.
  constexpr bool F8S = PAIR && kBf && KDT == kFP8 && D == 128;
  constexpr int STAGE_BYTES = NSTAGE * STEP_TOK * LROW;
  constexpr int HELD_FIT = (IdxWg<MT, NQ>::lds - STAGE_BYTES) / (WAVES * STEP_TOK * 4);
  constexpr int HELD = HELD_FIT < 1 ? 1 : HELD_FIT > kIdxMaxHeldSteps ? kIdxMaxHeldSteps : HELD_FIT;
  constexpr int PW = PAIR ? PIECES / 2 : PIECES;  // pieces of a step this wave loads
  constexpr int WLOADS = (PW + 63) / 64;
  __shared__ __attribute__((aligned(16))) uint8_t stage[NSTAGE][STEP_TOK * LROW];
  __shared__ __attribute__((aligned(16))) float held[WAVES][HELD * STEP_TOK];
  const int32_t rows = NQ * n_heads;  // query rows of one request

  const int lane = threadIdx.x & 63;
  // Wave-uniform values are kept in scalar registers: the run bounds, the
  // cursors and the request lengths then never wait on vector memory.
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  // Run units: waves, or pairs of waves (the pair's waves share one run).
  const int64_t nw = PAIR ? (int64_t)gridDim.x : (int64_t)gridDim.x * 4;
  const int64_t gw = PAIR ? (int64_t)xcd_remap(blockIdx.x, gridDim.x)
                          : (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4 + wv;
  const int qw = PAIR ? wv : 0;          // the wave's query: every wave scores one
  const int pbase = PAIR ? wv * PW : 0;  // the wave's first piece of a step
  int cbuf = 0;                          // the pair's stage buffer for the next step consumed

  auto len_ok = [&](int32_t Lb) -> bool { return Lb >= 0 && (int64_t)Lb <= max_len && (int64_t)Lb <= bt_cap; };
  auto steps_of = [&](int32_t Lb) -> int64_t { return len_ok(Lb) ? ((int64_t)Lb + STEP_TOK - 1) / STEP_TOK : 0; };

  // ---- this wave's run of steps [u0, u1) of the flattened step list
  int64_t mine = 0;
  for (int i = lane; i < batch; i += 64) {
    const int32_t Lb = lens[i];
    mine += steps_of(Lb);
    if (gw == 0 && wv == 0 && !len_ok(Lb) && status)
      for (int qi = 0; qi < NQ; ++qi) atomicOr(status + (int64_t)i * NQ + qi, kBadLen);
  }
  int64_t total = wave_sum_i64(mine);
  total = ((int64_t)__builtin_amdgcn_readfirstlane((int32_t)(total >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)total);
  constexpr bool two_per_cu = !PAIR && IdxWg<MT, NQ>::per_cu == 2;
  const int64_t u0 = run_start(total, gw, nw, gridDim.x, two_per_cu);
  const int64_t u1 = run_start(total, gw + 1, nw, gridDim.x, two_per_cu);
  if (u0 >= u1) return;
  int32_t b0 = 0;
  int64_t s0 = 0;  // step index of u0 within request b0
  {
    int64_t base = 0;
    for (int c = 0; c < batch; c += 64) {
      const int i = c + lane;
      const int64_t un = i < batch ? steps_of(lens[i]) : 0;
      const int64_t inc = wave_incl_scan_i64(un, lane);
      const int64_t tot = __shfl(inc, 63);
      if (u0 < base + tot) {
        const int j = __ffsll((unsigned long long)__ballot(base + inc > u0)) - 1;
        b0 = __builtin_amdgcn_readfirstlane(c + j);
        s0 = u0 - (base + __shfl(inc - un, j));
        break;
      }
      base += tot;
    }
  }

  s0 = ((int64_t)__builtin_amdgcn_readfirstlane((int32_t)(s0 >> 32)) << 32) |
       (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)s0);

  // Query fragments (A operand: rows = heads), permuted like the key slices,
  // and head weights of request `rb`.
  // In the two-query kernel with FP8 keys of 128 dims the query is held
  // instead as two scaled e4m3 terms per row (qh, ql with E8M0 scales qsh,
  // qsl, the representation split_q32 states) and the keys go to the scaled
  // FP8 MFMA as they are stored: no widening.
  typename Op::frag qa[MT][KSTEPS];
  v8i_t qh[MT], ql[MT];
  int qsh[MT], qsl[MT];
  float wr[MT][4];
  auto load_query = [&](int32_t rb) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int hq = mt * 16 + r16;     // row within the wave's queries
      const int h = qw * n_heads + hq;  // row within the request's queries
      if constexpr (F8S) {
        uint32_t raw[16] = {};
        if (hq < n_heads)
          load_raw<64>(reinterpret_cast<const uint8_t*>(q_idx) + (((int64_t)rb * rows + h) * D + g * 32) * 2, raw);
        split_q32(raw, qh[mt], ql[mt], qsh[mt], qsl[mt]);  // the whole wave, every row
      } else if (hq < n_heads) {
        uint32_t raw[(GROUP_ELEMS * QE + 3) / 4];
        const uint8_t* qp =
            reinterpret_cast<const uint8_t*>(q_idx) + (((int64_t)rb * rows + h) * D + g * GROUP_ELEMS) * QE;
        load_raw<GROUP_ELEMS * QE>(qp, raw);
        raw_to_frags<Op, kBf ? kBF16 : kF32, KSTEPS>(raw, qa[mt]);
      } else {
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) qa[mt][st] = zero_frag<Op>();
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + g * 4 + i;
        wr[mt][i] = hh < n_heads ? w[(int64_t)rb * rows + qw * n_heads + hh] : 0.f;
      }
    }
  };

  // Token tok of a step whose first token is t0 lies on the step's page
  // tok >> page_shift when pages are shorter than a step (t0 is then a
  // multiple of the page size), else on its only page at offset
  // (t0 mod page size) + tok.
  constexpr bool multi_page = MULTI;

  // The run is walked one request at a time: steps [s, s_end) of request b
  // (length L).  Within a request everything the loop needs is in scalar
  // registers, so its only memory waits are for the keys themselves.
  int32_t b = b0;
  int32_t L = __builtin_amdgcn_readfirstlane(lens[b0]);
  int64_t s = s0;
  int64_t todo = u1 - u0;
  while (true) {
    const int64_t s_end = min(steps_of(L), s + todo);
    const int64_t n = s_end - s;
    load_query(b);
    int n_held = 0;     // steps whose scores wait in held[wv]
    int64_t t_held = 0; // first token of those steps (they are consecutive)
    const int32_t* btb = bt + (int64_t)b * bt_stride;
    float* sc_out = scores + (int64_t)b * NQ * score_stride;  // query i's row: sc_out + i * score_stride
    const int64_t last_page = ((int64_t)L - 1) >> page_shift;

    // Block-table entries of step si: lane j < 4 loads the entry of the
    // step's j-th page (a step spans at most 4 pages, as pages hold at least
    // 16 tokens); entries past the request's last page repeat its last page.
    auto prep = [&](int64_t si) __attribute__((always_inline)) -> int32_t {
      const int64_t first = (si * STEP_TOK) >> page_shift;
      return btb[min(first + min(lane, 3), last_page)];
    };
    // Issue the key loads of step si.  The loads are unconditional (a token
    // past the end, or a step past the run, reads row 0, which always
    // exists, and is never used), so the compiler can count them and keep
    // the next step's loads in flight during this step's math.  `sc` gets
    // the FP8 scale of token `lane` (1 for other key types) and `bad_tok` is
    // set if its page is invalid (applied at consume time, so that nothing
    // here waits for the scale load).
    auto issue = [&](int64_t si, int32_t pgv, uint32_t (*raw)[4], float& sc, int& bad_tok)
        __attribute__((always_inline)) {
      const int64_t t0 = si * STEP_TOK;
      const int t0_in_page = multi_page ? 0 : (int)(t0 & (page_size - 1));
      const int left = (int)max((int64_t)0, min((int64_t)L - t0, (int64_t)STEP_TOK));
      // Cache row of token `tok` of the step (row 0 when past the end or on
      // an invalid page, which `bad` then reports).  Branch-free, so the
      // loads stay in one basic block.
      auto row_of = [&](int tok, bool& bad) __attribute__((always_inline)) -> int64_t {
        const int32_t page = __shfl(pgv, multi_page ? tok >> page_shift : 0);
        const bool in = tok < left;
        const bool valid = (page >= 0) & (page < num_pages);
        bad = in & !valid;
        const bool ok = in & valid;
        return ((int64_t)(ok ? page : 0) << page_shift) + (ok ? (t0_in_page + tok) & (page_size - 1) : 0);
      };
      bool bad;
      if (!multi_page) {
        // The whole step is on one page: a scalar base address plus 32-bit
        // per-lane offsets (a token past the end reads the step's first row).
        const int32_t page = __builtin_amdgcn_readfirstlane(pgv);
        const bool page_ok = page >= 0 && page < num_pages;
        const int64_t row0 = page_ok ? ((int64_t)page << page_shift) + t0_in_page : 0;
        const uint8_t* base = k_pool + row0 * ROW_BYTES;
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
          const int piece = pbase + min(i * 64 + lane, PW - 1);
          const int tok = piece / ROW_PIECES;
          const int off = (tok < left ? tok * ROW_BYTES : 0) + (piece % ROW_PIECES) * 16;
          load_nt16(base + off, raw[i]);
        }
        const int tok = min(lane, STEP_TOK - 1);
        if constexpr (KDT == kFP8) sc = k_scale[row0 + (tok < left ? tok : 0)];
        else sc = 1.f;
        bad = tok < left && !page_ok;
      } else {
#pragma unroll
        for (int i = 0; i < WLOADS; ++i) {
          const int piece = pbase + min(i * 64 + lane, PW - 1);
          bool bad_i;
          const int64_t row = row_of(piece / ROW_PIECES, bad_i);
          load_nt16(k_pool + row * ROW_BYTES + (piece % ROW_PIECES) * 16, raw[i]);
        }
        const int64_t row = row_of(min(lane, STEP_TOK - 1), bad);
        if constexpr (KDT == kFP8) sc = k_scale[row];
        else sc = 1.f;
      }
      bad_tok = bad;
      if (__builtin_expect(__any(bad), 0) && bad && status)
        for (int qi = 0; qi < NQ; ++qi) atomicOr(status + (int64_t)b * NQ + qi, kBadPage);
    };
    // The whole wave writes the held scores with 16-byte stores.
    auto write_held = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_wave_barrier();
      const int cnt = n_held * STEP_TOK;
      float* out = sc_out + qw * score_stride;
      for (int i = lane * 4; i < cnt; i += 256) {
        const int64_t t = t_held + i;
        const float4 v4 = *reinterpret_cast<const float4*>(&held[wv][i]);
        if (t + 3 < L) {
          *reinterpret_cast<float4*>(out + t) = v4;
        } else {
          if (t < L) out[t] = v4.x;
          if (t + 1 < L) out[t + 1] = v4.y;
          if (t + 2 < L) out[t + 2] = v4.z;
        }
      }
      __builtin_amdgcn_wave_barrier();
      n_held = 0;
    };
    auto consume = [&](int64_t si, const uint32_t (*raw)[4], float sc, int bad_tok) __attribute__((always_inline)) {
      const int64_t t0 = si * STEP_TOK;
      // Transpose through LDS rows (padded by 16 bytes): the wave's own rows,
      // or the pair's stage buffer, which both waves fill (one barrier; with
      // two buffers a buffer is rewritten only after both waves have passed
      // the barrier of the step after the one that read it).
      uint8_t* my_stage = stage[PAIR ? cbuf : wv];
#pragma unroll
      for (int i = 0; i < WLOADS; ++i) {
        const int piece = pbase + i * 64 + lane;
        if (i * 64 + lane < PW)
          *reinterpret_cast<uint4*>(my_stage + (piece / ROW_PIECES) * LROW + (piece % ROW_PIECES) * 16) =
              make_uint4(raw[i][0], raw[i][1], raw[i][2], raw[i][3]);
      }
      if constexpr (PAIR) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        cbuf ^= 1;
      } else {
        __builtin_amdgcn_wave_barrier();
      }
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
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (F8S) {
          // The lane's 32 key codes are its 32 k-slots, as the query terms'.
          const v8i_t kc = {(int)sl[0], (int)sl[1], (int)sl[2], (int)sl[3],
                            (int)sl[4], (int)sl[5], (int)sl[6], (int)sl[7]};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qh[mt], kc, acc[mt], 0, 0, 0, qsh[mt], 0, 127);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ql[mt], kc, acc[mt], 0, 0, 0, qsl[mt], 0, 127);
        } else {
          typename Op::frag kb[KSTEPS];
          raw_to_frags<Op, KDT, KSTEPS>(sl, kb);
#pragma unroll
          for (int st = 0; st < KSTEPS; ++st) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = Op::mma(qa[mt][st], kb[st], acc[mt]);
          }
        }
        const float tsc = __shfl(sc, tok);
        const bool bad = __shfl(bad_tok, tok) != 0;
        float v = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // ReLU as an integer max on the bit pattern (one instruction: a
            // negative float has a negative integer pattern).
            const float r = __int_as_float(max(__float_as_int(acc[mt][i]), 0));
            v += wr[mt][i] * r;
          }
        }
        v = wave_sum_xor16_32(v);
        if (g == 0) held[wv][n_held * STEP_TOK + tok] = bad ? __uint_as_float(0x7FC00000u) : v * tsc;
      }
      if (n_held == 0) t_held = t0;
      if (++n_held == HELD) write_held();
    };

    // Software pipeline, per step: the block-table entries of the step two
    // ahead are requested first, then the key loads of the next step (whose
    // entries were requested one step earlier, before the keys consumed
    // now, so waiting for them never waits for those keys), then this step's
    // keys are consumed.  Memory requests complete in order, so this
    // ordering keeps two steps of keys in flight.  Steps past the request's
    // share of the run only touch row 0 and are never consumed.
    uint32_t raw_a[WLOADS][4], raw_b[WLOADS][4];
    float sc_a, sc_b;
    int bad_a, bad_b;
    int32_t pg_a = prep(s);
    int32_t pg_b = prep(s + 1);
    issue(s, pg_a, raw_a, sc_a, bad_a);
    int64_t k = 0;
    for (; k + 1 < n; k += 2) {
      pg_a = prep(s + k + 2);
      issue(s + k + 1, pg_b, raw_b, sc_b, bad_b);
      consume(s + k, raw_a, sc_a, bad_a);
      pg_b = prep(s + k + 3);
      issue(s + k + 2, pg_a, raw_a, sc_a, bad_a);
      consume(s + k + 1, raw_b, sc_b, bad_b);
    }
    if (k < n) consume(s + k, raw_a, sc_a, bad_a);
    if (n_held > 0) write_held();
    __builtin_amdgcn_s_waitcnt(0);  // the loads of a step past the run are done with

    todo -= n;
    if (todo <= 0) break;
    // The run goes on with the next request that has steps.
    do {
      ++b;
      L = __builtin_amdgcn_readfirstlane(lens[b]);
    } while (steps_of(L) == 0);
    s = 0;
  }
}

template <class Op, int KDT, int KSTEPS, int MT, int NQ>
static int launch_one(const IndexerArgs& a, hipStream_t stream) {
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  if (a.batch == 0) return 0;
  // Enough waves to fill the GPU, but not more than there are steps at most.
  // At least one workgroup runs even when max_len is 0: its first wave is
  // the one that flags requests whose length is out of range.
  constexpr int ROW_BYTES = KSTEPS * 4 * Op::KPL * Storage<KDT>::bytes;
  constexpr int STEP_TOK = IdxStep<ROW_BYTES>::tok;
  const int64_t max_steps = (int64_t)a.batch * ((a.max_len + STEP_TOK - 1) / STEP_TOK);
  constexpr int kUnits = NQ == 2 ? 1 : 4;  // run units per workgroup: one pair, or four waves
  const int64_t grid = std::max<int64_t>(
      1, std::min<int64_t>((int64_t)kNumCu * IdxWg<MT, NQ>::per_cu, (max_steps + kUnits - 1) / kUnits));
  const dim3 threads(IdxWg<MT, NQ>::waves * 64);
  if (a.page_size < STEP_TOK)
    hipLaunchKernelGGL((indexer_kernel<Op, KDT, KSTEPS, MT, true, NQ>), dim3((unsigned)grid), threads, 0,
                       stream, a.q_idx, a.w, reinterpret_cast<const uint8_t*>(a.k_pool), a.k_scale, a.num_pages,
                       page_shift, a.bt, a.bt_stride, a.lens, a.batch, a.max_len, a.n_heads, a.scores,
                       a.score_stride, a.status);
  else
    hipLaunchKernelGGL((indexer_kernel<Op, KDT, KSTEPS, MT, false, NQ>), dim3((unsigned)grid), threads, 0,
                       stream, a.q_idx, a.w, reinterpret_cast<const uint8_t*>(a.k_pool), a.k_scale, a.num_pages,
                       page_shift, a.bt, a.bt_stride, a.lens, a.batch, a.max_len, a.n_heads, a.scores,
                       a.score_stride, a.status);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <class Op, int KDT, int KSTEPS>
static int dispatch_heads(const IndexerArgs& a, hipStream_t s) {
  if (a.n_q == 2) {
    // Two queries per key read (bf16 queries): a pair of waves, one per
    // query, each with the query's M-tiles.
    if constexpr (std::is_same<Op, OpBF16>::value) {
      if (a.n_heads == 16) return launch_one<Op, KDT, KSTEPS, 1, 2>(a, s);
      if (a.n_heads == 32) return launch_one<Op, KDT, KSTEPS, 2, 2>(a, s);
      if (a.n_heads == 64) return launch_one<Op, KDT, KSTEPS, 4, 2>(a, s);
    }
    return -2;
  }
  if (a.n_q != 1) return -2;
  if (a.n_heads <= 16) return launch_one<Op, KDT, KSTEPS, 1, 1>(a, s);
  if (a.n_heads <= 32) return launch_one<Op, KDT, KSTEPS, 2, 1>(a, s);
  if (a.n_heads <= 64) return launch_one<Op, KDT, KSTEPS, 4, 1>(a, s);
  if (a.n_heads <= 128) return launch_one<Op, KDT, KSTEPS, 8, 1>(a, s);
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
