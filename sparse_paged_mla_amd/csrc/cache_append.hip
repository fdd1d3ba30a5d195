// kv_cache_append kernel: writes each request's new token row into its page
// slot (of one pool, or of two pools that share page ids in one launch),
// quantising to OCP e4m3 with a per-token scale when the pool is FP8.
//
// One wave per request.  The row is read in 8-element chunks (lane c takes
// chunks c, c + 64, ...) and kept in registers; the wave's absolute maximum
// gives the scale s = absmax / 448 (fp32, correctly rounded; 1 for an
// all-zero row), and each element is stored as the e4m3 code of the fp32
// quotient x / s (hardware conversion: nearest, ties to even).  bf16 pools
// take x rounded to nearest even, fp32 pools x itself.  The work is a few
// hundred bytes per request: the launch, not the bytes, sets its time.
#include "common.h"
#include "launch.h"

namespace spmla {

constexpr int kAppThreads = 256;
constexpr int kAppMaxChunksPerLane = 8;  // row_dim <= 8 * 8 * 64 = 4096

// One pool: its new rows, row length, storage and scales.
struct AppendPool {
  const void* rows;
  int32_t dim;
  void* pool;
  float* scale;
};

// Waves [0, batch) append to pool p0 and, when npools is 2, waves
// [batch, 2 * batch) to pool p1 (the latent rows and the indexer keys of the
// same tokens, which share page ids and so the block table).
template <int RDT, int PDT>
__global__ __launch_bounds__(kAppThreads) void cache_append_kernel(
    AppendPool p0, AppendPool p1, int32_t npools, int32_t batch, int32_t num_pages, int32_t page_shift,
    const int32_t* __restrict__ bt, int32_t bt_stride, const int32_t* __restrict__ positions,
    int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int v = blockIdx.x * (kAppThreads / 64) + (threadIdx.x >> 6);
  if (v >= npools * batch) return;
  const bool second = v >= batch;
  const int b = second ? v - batch : v;
  const void* __restrict__ rows = second ? p1.rows : p0.rows;
  const int32_t dim = second ? p1.dim : p0.dim;
  void* __restrict__ pool = second ? p1.pool : p0.pool;
  float* __restrict__ pool_scale = second ? p1.scale : p0.scale;
  const int32_t t = positions[b];
  if (t < 0) return;
  const int page_size = 1 << page_shift;
  if ((int64_t)t >= (int64_t)bt_stride * page_size) {
    if (lane == 0 && status) atomicOr(status + b, kBadLen);
    return;
  }
  const int32_t page = bt[(int64_t)b * bt_stride + (t >> page_shift)];
  if (page < 0 || page >= num_pages) {
    if (lane == 0 && status) atomicOr(status + b, kBadPage);
    return;
  }
  const int64_t row = ((int64_t)page << page_shift) + (t & (page_size - 1));
  const int chunks = dim >> 3;

  // The row, as fp32, in registers.
  float x[kAppMaxChunksPerLane][8];
#pragma unroll
  for (int i = 0; i < kAppMaxChunksPerLane; ++i) {
    const int c = lane + 64 * i;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
    if (c < chunks) {
      if constexpr (RDT == kBF16) {
        const uint4 v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(rows) + (int64_t)b * dim)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[i][2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
          x[i][2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        }
      } else {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(rows) + (int64_t)b * dim) + 2 * c;
        const float4 u = src[0], v = src[1];
        x[i][0] = u.x; x[i][1] = u.y; x[i][2] = u.z; x[i][3] = u.w;
        x[i][4] = v.x; x[i][5] = v.y; x[i][6] = v.z; x[i][7] = v.w;
      }
    }
  }

  if constexpr (PDT == kFP8) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kAppMaxChunksPerLane; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    if (lane == 0) pool_scale[row] = s;
    uint8_t* dst = static_cast<uint8_t*>(pool) + row * dim;
#pragma unroll
    for (int i = 0; i < kAppMaxChunksPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int p = 0;
          p = __builtin_amdgcn_cvt_pk_fp8_f32(x[i][4 * h] / s, x[i][4 * h + 1] / s, p, false);
          p = __builtin_amdgcn_cvt_pk_fp8_f32(x[i][4 * h + 2] / s, x[i][4 * h + 3] / s, p, true);
          w[h] = (uint32_t)p;
        }
        reinterpret_cast<uint2*>(dst)[c] = make_uint2(w[0], w[1]);
      }
    }
  } else if constexpr (PDT == kBF16) {
    uint16_t* dst = static_cast<uint16_t*>(pool) + row * dim;
#pragma unroll
    for (int i = 0; i < kAppMaxChunksPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 lo = (__bf16)x[i][2 * e], hi = (__bf16)x[i][2 * e + 1];
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        reinterpret_cast<uint4*>(dst)[c] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  } else {
    float* dst = static_cast<float*>(pool) + row * dim;
#pragma unroll
    for (int i = 0; i < kAppMaxChunksPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < chunks) {
        float4* d4 = reinterpret_cast<float4*>(dst) + 2 * c;
        d4[0] = make_float4(x[i][0], x[i][1], x[i][2], x[i][3]);
        d4[1] = make_float4(x[i][4], x[i][5], x[i][6], x[i][7]);
      }
    }
  }
}

int launch_cache_append(const AppendArgs& a, hipStream_t s) {
  if (a.batch == 0) return 0;
  const int npools = a.rows2 ? 2 : 1;
  for (int d : {a.dim, npools == 2 ? a.dim2 : a.dim})
    if (d % 8 != 0 || d < 8 || d > 8 * 64 * kAppMaxChunksPerLane) return -2;
  int page_shift = 0;
  while ((1 << page_shift) < a.page_size) ++page_shift;
  const AppendPool p0{a.rows, a.dim, a.pool, a.pool_scale};
  const AppendPool p1{a.rows2, a.dim2, a.pool2, a.pool_scale2};
  const unsigned grid = (unsigned)(((int64_t)npools * a.batch + kAppThreads / 64 - 1) / (kAppThreads / 64));
#define SPMLA_APPEND(R, P)                                                                                        \
  hipLaunchKernelGGL((cache_append_kernel<R, P>), dim3(grid), dim3(kAppThreads), 0, s, p0, p1, npools, a.batch, \
                     a.num_pages, page_shift, a.bt, a.bt_stride, a.positions, a.status)
  if (a.row_dtype == kBF16) {
    if (a.pool_dtype == kFP8) SPMLA_APPEND(kBF16, kFP8);
    else if (a.pool_dtype == kBF16) SPMLA_APPEND(kBF16, kBF16);
    else SPMLA_APPEND(kBF16, kF32);
  } else {
    if (a.pool_dtype == kFP8) SPMLA_APPEND(kF32, kFP8);
    else if (a.pool_dtype == kBF16) SPMLA_APPEND(kF32, kBF16);
    else SPMLA_APPEND(kF32, kF32);
  }
#undef SPMLA_APPEND
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace spmla
