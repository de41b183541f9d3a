// common.hpp -- element formats, E4M3 codec and wave helpers for gfx950.
//
// Element formats of the paged cache ("PagedAttention in mistral.rs",
// section "KV Cache Quantization"): the cache holds either the activation
// type (fp16 / bf16) or FP8 E4M3.  E4M3 here is the OCP "FN" variant: bias 7,
// largest finite magnitude 448, no infinities, NaN = S.1111.111.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Fmt { FMT_F16 = 0, FMT_BF16 = 1, FMT_E4M3 = 2 };

// ---------------------------------------------------------------------------
// 16-bit activation formats <-> fp32.

template <int F>
__device__ __forceinline__ float lo16_to_f32(uint32_t w);
template <int F>
__device__ __forceinline__ float hi16_to_f32(uint32_t w);

template <>
__device__ __forceinline__ float lo16_to_f32<FMT_BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <>
__device__ __forceinline__ float hi16_to_f32<FMT_BF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
template <>
__device__ __forceinline__ float lo16_to_f32<FMT_F16>(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
template <>
__device__ __forceinline__ float hi16_to_f32<FMT_F16>(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// fp32 -> 16-bit, round to nearest even (NaN stays NaN).
template <int F>
__device__ __forceinline__ uint32_t f32_to_16(float x);

template <>
__device__ __forceinline__ uint32_t f32_to_16<FMT_BF16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
template <>
__device__ __forceinline__ uint32_t f32_to_16<FMT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <int F>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return f32_to_16<F>(a) | (f32_to_16<F>(b) << 16);
}

// ---------------------------------------------------------------------------
// E4M3 encode: code of t = fp32(x) / fp32(scale).
//
// Round to nearest, ties to even; |t| >= 448 saturates to 0x7E; NaN -> 0x7F;
// the sign bit of t is kept (so -0 and tiny negatives give 0x80).
__device__ __forceinline__ uint32_t e4m3_encode_t(float t) {
  const uint32_t bits = __float_as_uint(t);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7fffffffu;
  uint32_t code;
  if (a > 0x7f800000u) {
    code = 0x7fu;                     // NaN
  } else if (a >= 0x43e00000u) {      // |t| >= 448 (inf included)
    code = 0x7eu;
  } else if (a >= 0x3c800000u) {      // |t| >= 2^-6: normal range
    // Keep 3 mantissa bits with round-to-nearest-even on the 20 dropped bits,
    // then rebias the exponent from 127 to 7.  A mantissa carry moves into
    // the exponent field, which is the correct next code.
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    // Subnormal range: value = m * 2^-9 with m = rne(|t| * 512) in 0..8
    // (8 is the smallest normal, code 0x08).  Scaling by 512 is exact.
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    code = static_cast<uint32_t>(m);
  }
  return code | sign;
}

__device__ __forceinline__ uint32_t e4m3_encode(float x, float scale) {
  return e4m3_encode_t(__fdiv_rn(x, scale));
}

// E4M3 -> fp32 for the two codes in the low (HI = false) or high half of w.  Every E4M3
// value is exactly representable in fp32, bf16 and fp16.
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// ---------------------------------------------------------------------------
// Wave helpers (64 lanes).

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Max / sum over the 16 lanes of a row (lanes 16r .. 16r+15), by xor-shuffles
// that stay inside the row.
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
