// Device-side building blocks shared by the gfx950 kernels: MFMA operand
// traits, storage loaders (fp32 / bf16 / FP8 e4m3fn widened exactly), wave
// helpers.  CDNA4 only: 64-lane wavefronts, v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, hardware OCP e4m3 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace spmla {

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };
enum : int { kBadPage = 1, kBadLen = 2, kBadIndex = 4, kBadTag = 8 };

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __bf16 v4bf16_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Storage element size in bytes.
template <int DT> struct Storage;
template <> struct Storage<kF32> { static constexpr int bytes = 4; };
template <> struct Storage<kBF16> { static constexpr int bytes = 2; };
template <> struct Storage<kFP8> { static constexpr int bytes = 1; };

// MFMA operand traits.  A 16x16 MFMA with K = 4 * KPL: lane l supplies row
// (or column) l % 16 and the KPL consecutive k-slots 4-group l / 16 owns; the
// 16x16 fp32 result leaves rows 4 * (l / 16) + i, i < 4, of column l % 16 in
// lane l.  (Layout confirmed on gfx950 hardware for both instructions.)
struct OpBF16 {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  typedef __bf16 elem;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
struct OpF32 {
  static constexpr int KPL = 1;
  typedef float frag;
  typedef float elem;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// ---- raw loads of BYTES contiguous bytes into dwords (widest aligned vector loads)
template <int BYTES>
__device__ __forceinline__ void load_raw(const uint8_t* __restrict__ p, uint32_t* out) {
  if constexpr (BYTES % 16 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      uint4 v = *reinterpret_cast<const uint4*>(p + 16 * i);
      out[4 * i + 0] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else if constexpr (BYTES % 8 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 8; ++i) {
      uint2 v = *reinterpret_cast<const uint2*>(p + 8 * i);
      out[2 * i + 0] = v.x; out[2 * i + 1] = v.y;
    }
  } else if constexpr (BYTES % 4 == 0) {
#pragma unroll
    for (int i = 0; i < BYTES / 4; ++i) out[i] = *reinterpret_cast<const uint32_t*>(p + 4 * i);
  } else if constexpr (BYTES == 2) {
    out[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    static_assert(BYTES == 1, "unsupported raw width");
    out[0] = *p;
  }
}

typedef uint32_t u32x4_ev __attribute__((ext_vector_type(4)));

// 16-byte streaming load that does not allocate in the caches (data read once).
__device__ __forceinline__ void load_nt16(const uint8_t* __restrict__ p, uint32_t* out) {
  const u32x4_ev v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_ev*>(p));
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Element j of a raw dword array holding storage type DT, widened to fp32.
template <int DT>
__device__ __forceinline__ float raw_elem_f32(const uint32_t* raw, int j) {
  if constexpr (DT == kF32) {
    return __uint_as_float(raw[j]);
  } else if constexpr (DT == kBF16) {
    return bf16_bits_to_f32((raw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
  } else {
    const int word = (int)raw[j >> 2];
    f32x2 v = ((j >> 1) & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true) : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
    return (j & 1) ? v[1] : v[0];
  }
}

// Convert raw storage holding N = NFRAG * KPL elements into MFMA fragments.
template <class Op, int DT, int NFRAG>
__device__ __forceinline__ void raw_to_frags(const uint32_t* raw, typename Op::frag* f) {
  if constexpr (std::is_same<Op, OpBF16>::value) {
    static_assert(DT == kBF16 || DT == kFP8, "bf16 MFMA operands come from bf16 or FP8 storage");
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int s = 0; s < NFRAG; ++s) {
        uint4 v = make_uint4(raw[4 * s], raw[4 * s + 1], raw[4 * s + 2], raw[4 * s + 3]);
        f[s] = __builtin_bit_cast(bf16x8, v);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NFRAG; ++s) {
        // FP8 e4m3fn -> bf16 is exact (3 mantissa bits fit in 7); scale 1.
        bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[2 * s], 1.0f, false);
        bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[2 * s], 1.0f, true);
        bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[2 * s + 1], 1.0f, false);
        bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[2 * s + 1], 1.0f, true);
        bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        f[s] = r;
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < NFRAG; ++s) f[s] = raw_elem_f32<DT>(raw, s);
  }
}

// Zero fragment.
template <class Op>
__device__ __forceinline__ typename Op::frag zero_frag() {
  typename Op::frag z;
  if constexpr (std::is_same<Op, OpBF16>::value) {
    z = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  } else {
    z = 0.f;
  }
  return z;
}

__device__ __forceinline__ float wave_max_xor16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Writes this lane's 32 bf16 values (w[i] holds values 2i, low half, and
// 2i + 1) as v = 2^(E-7) * (hi + lo/16), hi and lo e4m3 codes, where
// E = floor(log2 M) and M is the largest |v| over the four lanes of the row
// (lanes l, l^16, l^32, l^48: the 128 k-slots of one MFMA row), so one scale
// per row and term serves the block.  hi is v scaled below 256 and rounded
// to 4 significant bits; the remainder of an element within 2^14 of M is a
// multiple of its last bf16 bit below half an e4m3 step, so 16 times it is
// an e4m3 value and the sum is exact; a smaller element keeps an error below
// 2^-22 of M.  A non-finite element turns the hi codes of its lane into NaN,
// so the scores it feeds come out NaN.  Magnitudes are compared as bf16
// bits: without the sign, finite values order as integers and Inf and NaN
// lie above them.  Call with the whole wave active.
__device__ __forceinline__ void split_q32(const uint32_t (&w)[16], v8i_t& hi, v8i_t& lo, int& shi, int& slo) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  uint32_t mb = max((uint32_t)m[0], (uint32_t)m[1]);
  const bool bad = mb >= 0x7F80u;
  mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
  mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32));
  const int E = max((int)(mb >> 7) - 127, -115);
  const float mul = __uint_as_float((uint32_t)(134 - E) << 23);  // 2^(7 - E)
  shi = E + 120;
  slo = E + 116;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const float x0 = __uint_as_float(w[2 * d] << 16) * mul, x1 = __uint_as_float(w[2 * d] & 0xFFFF0000u) * mul;
    const float x2 = __uint_as_float(w[2 * d + 1] << 16) * mul, x3 = __uint_as_float(w[2 * d + 1] & 0xFFFF0000u) * mul;
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
    const f32x2 r01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false), r23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
    int l = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - r01[0]) * 16.f, (x1 - r01[1]) * 16.f, 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32((x2 - r23[0]) * 16.f, (x3 - r23[1]) * 16.f, l, true);
    hi[d] = bad ? 0x7F7F7F7F : h;
    lo[d] = l;
  }
}

}  // namespace spmla
