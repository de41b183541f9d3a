// common.hpp -- element formats, page layout, E4M3 codec and wave helpers
// shared by the gfx950 kernels.
//
// Element formats of the paged cache ("PagedAttention in mistral.rs",
// section "KV Cache Quantization"): the cache holds either the activation
// type (fp16 / bf16) or FP8 E4M3.  E4M3 here is the OCP "FN" variant: bias 7,
// largest finite magnitude 448, no infinities, NaN = S.1111.111.  A third
// option ("libmir-metal 0.2.0, src/native/trace/kv.rs", fn build) packs INT8
// codes with one fp32 scale per (token, KV head), kept beside the pages.
//
// Page layout (one (block, KV head) page of BS = 32 tokens, head-major as in
// "libmir-metal 0.2.0, src/native/trace/kv.rs", fn build):
//   K page [D/8][BS][8]  : element (t, d) at ((d/8)*BS + t)*8 + d%8
//   V page [BS/8][D][8]  : element (t, d) at ((t/8)*D + d)*8 + t%8
// With these layouts both matrix-core operands of the attention kernels (K
// for S = Q K^T with the head dimension as the reduction axis, V for
// O = P V with tokens as the reduction axis) are single 16-byte (8-byte for
// byte caches) loads per lane: 8 dims of one key, 8 keys of one dim.  The V
// page keeps its keys in groups of 8 (rather than one [D][BS] transposed
// page) so that a single appended row lands in D 16-byte runs within 2 KiB
// (D = 128) instead of D elements 64 bytes apart over the whole page: the
// decode's fused append measured 56.0 -> 54.1 us on the Mistral batch with
// the grouped V rows, and grouping K's rows the same way changed nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Fmt { FMT_F16 = 0, FMT_BF16 = 1, FMT_E4M3 = 2, FMT_I8 = 3 };

// One byte per cached element.
constexpr bool byte_fmt(int f) { return f == FMT_E4M3 || f == FMT_I8; }

constexpr int kPage = 32;  // tokens per block (page)

// Offsets (in elements) inside one (block, head) page.
__device__ __forceinline__ int k_page_off(int t, int d) { return ((d >> 3) * kPage + t) * 8 + (d & 7); }
__device__ __forceinline__ int v_page_off(int t, int d, int D) {
  return (((t >> 3) * D + d) << 3) + (t & 7);
}

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

// fp32 -> 16-bit with the hardware converter (round to nearest even); for
// finite values only (softmax probabilities).
template <int F>
__device__ __forceinline__ uint16_t cvt16(float x);
template <>
__device__ __forceinline__ uint16_t cvt16<FMT_BF16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
template <>
__device__ __forceinline__ uint16_t cvt16<FMT_F16>(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// ---------------------------------------------------------------------------
// Buffer resources: a descriptor over [base, base + bytes) for buffer loads.
// Loads at offsets past `bytes` return zero instead of touching memory.
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}
// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) leaving the other counters alone.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Cache policy of a buffer load: kCacheNT marks a non-temporal (streaming)
// access, for data that no other instruction of the launch reads again.
constexpr int kCacheDefault = 0;
constexpr int kCacheNT = 2;

template <int POLICY = kCacheDefault>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY);
}
template <int POLICY = kCacheDefault>
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POLICY);
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

// E4M3 -> fp32 for the two codes in the low (HI = false) or high half of w.
// Every E4M3 value is exactly representable in fp32, bf16 and fp16.
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// E4M3 -> two packed 16-bit values of format F (exact; unit scale).
template <int F, bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_16(uint32_t w);
template <>
__device__ __forceinline__ uint32_t e4m3x2_to_16<FMT_BF16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t e4m3x2_to_16<FMT_BF16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
template <>
__device__ __forceinline__ uint32_t e4m3x2_to_16<FMT_F16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t e4m3x2_to_16<FMT_F16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Eight E4M3 codes (two words) -> eight 16-bit values (four words).
template <int F>
__device__ __forceinline__ u32x4 e4m3x8_to_16(u32x2 c) {
  return u32x4{e4m3x2_to_16<F, false>(c[0]), e4m3x2_to_16<F, true>(c[0]),
               e4m3x2_to_16<F, false>(c[1]), e4m3x2_to_16<F, true>(c[1])};
}

// Eight int8 codes (two words, code i in byte i) -> eight 16-bit values of
// format F.  |code| <= 128 has at most 8 significant bits, so fp32 and then
// bf16 / fp16 hold it exactly.
template <int F>
__device__ __forceinline__ u32x4 i8x8_to_16(u32x2 c) {
  typedef float f32x8_t __attribute__((ext_vector_type(8)));
  f32x8_t f;
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[4 * w + i] = static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(c[w] >> (8 * i))));
  if constexpr (F == FMT_BF16) {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(u32x4, __builtin_convertvector(f, v8));
  } else {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(u32x4, __builtin_convertvector(f, v8));
  }
}

// INT8 code of t = x / scale: round half to even, clamped to +-127; a zero
// scale (an all-zero row) gives 0.
__device__ __forceinline__ uint32_t i8_encode(float x, float scale) {
  if (scale == 0.f) return 0u;
  const float q = __builtin_rintf(__fdiv_rn(x, scale));
  const float c = fminf(fmaxf(q, -127.f), 127.f);
  return static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(c)));
}

// ---------------------------------------------------------------------------
// Wave helpers (64 lanes).

// DPP lane permutations inside a row of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// max(v, v of the DPP-selected lane) as one v_max_f32_dpp.  Written as
// inline assembly because the compiler otherwise splits it into a DPP move,
// a NaN-quieting max and the max.  The leading s_nop covers the two wait
// states a DPP read needs after a VALU write of its source; the inputs here
// are finite or -inf, never NaN.
#define PA_DPP_MAX(v, CTRL)                                                                  \
  do {                                                                                       \
    float r_;                                                                                \
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf" \
                 : "=&v"(r_)                                                                 \
                 : "v"(v));                                                                  \
    v = r_;                                                                                  \
  } while (0)

// Max / sum over the 16 lanes of a row (lanes 16r .. 16r+15), all in DPP:
// swap neighbours, swap pairs, mirror halves of 8, mirror the row of 16.
__device__ __forceinline__ float row16_max(float v) {
  PA_DPP_MAX(v, "quad_perm:[1,0,3,2]");
  PA_DPP_MAX(v, "quad_perm:[2,3,0,1]");
  PA_DPP_MAX(v, "row_half_mirror");
  PA_DPP_MAX(v, "row_mirror");
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Max / sum over all 64 lanes, result uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA 16x16x32 with 16-bit inputs, fp32 accumulate.
template <int AF>
struct Mfma;
template <>
struct Mfma<FMT_BF16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma<FMT_F16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

}  // namespace pa
