// reshape_and_cache.hip -- the cache slot writer.
//
// Stores each new token's K and V rows into the cache slot named by its slot
// number ("Optimization plans", mistral.rs discussion 46, "Update" post,
// names this operation reshape_and_cache): block slot / 32, row slot % 32, for
// every KV head.  A negative slot skips the token.  With an E4M3 cache each
// element is quantised on the way in ("PagedAttention in mistral.rs",
// section "KV Cache Quantization"); with an INT8 cache each (token, head) row
// gets its own fp32 scale, max |x| / 127, stored beside the page, and its
// codes round x / scale half to even ("libmir-metal 0.2.0,
// src/native/trace/kv.rs", fn build: per-token/head INT8 pages).
//
// A workgroup takes 32 consecutive input tokens of one KV head.  It reads
// their K and V rows with fully coalesced 16-byte loads into LDS, then writes
// them out: K token-fastest, one 16-byte (8-byte) chunk of the [D/8][32][8]
// page per store, so consecutive lanes write consecutive rows; V, when 8
// tokens fill a whole 8-token group of rows of the [4][D][8] page (a
// prefill chunk), one 16-byte (8-byte) chunk per store, 8 tokens of one
// dimension gathered from LDS, else element by element.  Decode-time
// writes (one token per sequence) take the same kernel.
#include "common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

constexpr int kGroup = 32;   // tokens per workgroup
constexpr int kThreads = 256;

template <int AF, int CF>
__global__ __launch_bounds__(kThreads) void cache_write(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ slot_mapping, int T, int Hkv, int D, float k_scale,
    float v_scale, float* __restrict__ key_scales, float* __restrict__ value_scales) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int CPR = D / 8;              // 8-element chunks per row
  const int ROW = D + 8;              // padded LDS row (elements)
  uint16_t* k_s = lds;                // [kGroup][ROW]
  uint16_t* v_s = lds + kGroup * ROW; // [kGroup][ROW]
  __shared__ int slot_s[kGroup];
  __shared__ float ksc_s[kGroup], vsc_s[kGroup];  // INT8: row scales

  const int n0 = blockIdx.x * kGroup;
  const int h = blockIdx.y;
  const int nt = min(kGroup, T - n0);
  const int tid = threadIdx.x;

  if (tid < kGroup) slot_s[tid] = tid < nt ? slot_mapping[n0 + tid] : -1;
  // Coalesced reads: chunk-fastest over the group's rows.
  for (int i = tid; i < nt * CPR; i += kThreads) {
    const int n = i / CPR;
    const int c = i - n * CPR;
    const size_t src = ((size_t)(n0 + n) * Hkv + h) * D + 8 * c;
    *reinterpret_cast<u32x4*>(&k_s[n * ROW + 8 * c]) = *reinterpret_cast<const u32x4*>(key + src);
    *reinterpret_cast<u32x4*>(&v_s[n * ROW + 8 * c]) = *reinterpret_cast<const u32x4*>(value + src);
  }
  __syncthreads();

  if constexpr (CF == FMT_I8) {
    // Row scales: eight threads per row take every eighth chunk, then a
    // butterfly over the eight lanes (adjacent lanes of one wave).
    const int n = tid >> 3;
    const int part = tid & 7;
    float ka = 0.f, va = 0.f;
    if (n < nt) {
      for (int c = part; c < CPR; c += 8) {
        const u32x4 kw = *reinterpret_cast<const u32x4*>(&k_s[n * ROW + 8 * c]);
        const u32x4 vw = *reinterpret_cast<const u32x4*>(&v_s[n * ROW + 8 * c]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ka = fmaxf(ka, fmaxf(fabsf(lo16_to_f32<AF>(kw[w])), fabsf(hi16_to_f32<AF>(kw[w]))));
          va = fmaxf(va, fmaxf(fabsf(lo16_to_f32<AF>(vw[w])), fabsf(hi16_to_f32<AF>(vw[w]))));
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      ka = fmaxf(ka, __shfl_xor(ka, m, 64));
      va = fmaxf(va, __shfl_xor(va, m, 64));
    }
    if (part == 0) {
      const float ks = __fdiv_rn(ka, 127.f);
      const float vs = __fdiv_rn(va, 127.f);
      ksc_s[n] = ks;
      vsc_s[n] = vs;
      const int slot = slot_s[n];
      if (slot >= 0) {
        const int blk = slot / kPage;
        const size_t at = ((size_t)blk * Hkv + h) * kPage + (slot - blk * kPage);
        key_scales[at] = ks;
        value_scales[at] = vs;
      }
    }
    __syncthreads();
  }

  constexpr int EB = byte_fmt(CF) ? 1 : 2;
  const size_t page_elems = (size_t)kPage * D;
  // K: token-fastest 8-element chunks, each one 16-byte (8-byte) store.
  for (int i = tid; i < kGroup * CPR; i += kThreads) {
    const int n = i % kGroup;
    const int c = i / kGroup;
    const int slot = slot_s[n];
    if (slot < 0) continue;
    const int blk = slot / kPage;
    const int off = slot - blk * kPage;
    const size_t dst = (((size_t)blk * Hkv + h) * page_elems + k_page_off(off, 8 * c)) * EB;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(&k_s[n * ROW + 8 * c]);
    if constexpr (byte_fmt(CF)) {
      u32x2 kq;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t kb = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t x = kw[2 * w + k];
          if constexpr (CF == FMT_E4M3) {
            kb |= e4m3_encode(lo16_to_f32<AF>(x), k_scale) << (16 * k);
            kb |= e4m3_encode(hi16_to_f32<AF>(x), k_scale) << (16 * k + 8);
          } else {
            kb |= i8_encode(lo16_to_f32<AF>(x), ksc_s[n]) << (16 * k);
            kb |= i8_encode(hi16_to_f32<AF>(x), ksc_s[n]) << (16 * k + 8);
          }
        }
        kq[w] = kb;
      }
      *reinterpret_cast<u32x2*>(key_cache + dst) = kq;
    } else {
      *reinterpret_cast<u32x4*>(key_cache + dst) = kw;
    }
  }
  // V: the page holds 8-token groups, one 16-byte (8-byte) chunk per
  // (group, dimension).  Where a group's 8 tokens fill 8 consecutive rows
  // starting at a multiple of 8 (a prefill chunk), a thread gathers the 8
  // elements of one dimension from LDS and stores the chunk at once;
  // consecutive threads take consecutive dimensions, so the stores are
  // contiguous runs.  Other groups (decode rows, a chunk that starts
  // mid-group) are stored element by element.
  for (int i = tid; i < (kGroup / 8) * D; i += kThreads) {
    const int tq = i / D;
    const int d = i - tq * D;
    const int n8 = 8 * tq;
    const int s0 = slot_s[n8];
    bool whole = s0 >= 0 && (s0 & 7) == 0;
#pragma unroll
    for (int j = 1; j < 8; ++j) whole = whole && slot_s[n8 + j] == s0 + j;
    if (whole) {
      const int blk = s0 / kPage;
      const size_t dst = ((size_t)blk * Hkv + h) * page_elems + v_page_off(s0 - blk * kPage, d, D);
      uint16_t x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = v_s[(n8 + j) * ROW + d];
      if constexpr (byte_fmt(CF)) {
        u32x2 q = u32x2{0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t e;
          if constexpr (CF == FMT_E4M3) {
            e = e4m3_encode(lo16_to_f32<AF>(x[j]), v_scale);
          } else {
            e = i8_encode(lo16_to_f32<AF>(x[j]), vsc_s[n8 + j]);
          }
          q[j >> 2] |= (e & 0xffu) << (8 * (j & 3));
        }
        *reinterpret_cast<u32x2*>(value_cache + dst) = q;
      } else {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (uint32_t)x[2 * k] | ((uint32_t)x[2 * k + 1] << 16);
        *reinterpret_cast<u32x4*>(value_cache + dst * 2) = w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = n8 + j;
        const int slot = slot_s[n];
        if (slot < 0) continue;
        const int blk = slot / kPage;
        const int off = slot - blk * kPage;
        const size_t dst = ((size_t)blk * Hkv + h) * page_elems + v_page_off(off, d, D);
        const uint16_t x = v_s[n * ROW + d];
        if constexpr (CF == FMT_E4M3) {
          value_cache[dst] = static_cast<uint8_t>(e4m3_encode(lo16_to_f32<AF>(x), v_scale));
        } else if constexpr (CF == FMT_I8) {
          value_cache[dst] = static_cast<uint8_t>(i8_encode(lo16_to_f32<AF>(x), vsc_s[n]));
        } else {
          reinterpret_cast<uint16_t*>(value_cache)[dst] = x;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  dim3 grid((a.T + kGroup - 1) / kGroup, a.Hkv);
  const size_t lds = 2 * (size_t)kGroup * (a.D + 8) * sizeof(uint16_t);
  const uint16_t* k = (const uint16_t*)a.key;
  const uint16_t* v = (const uint16_t*)a.value;
  uint8_t* kc = (uint8_t*)a.key_cache;
  uint8_t* vc = (uint8_t*)a.value_cache;
#define PA_LAUNCH(AF, CF)                                                                   \
  hipLaunchKernelGGL((cache_write<AF, CF>), grid, dim3(kThreads), lds, s, k, v, kc, vc,      \
                     a.slot_mapping, a.T, a.Hkv, a.D, a.k_scale, a.v_scale, a.key_scales,     \
                     a.value_scales)
  if (a.act == FMT_BF16 && a.cache == FMT_BF16) PA_LAUNCH(FMT_BF16, FMT_BF16);
  else if (a.act == FMT_F16 && a.cache == FMT_F16) PA_LAUNCH(FMT_F16, FMT_F16);
  else if (a.act == FMT_BF16 && a.cache == FMT_E4M3) PA_LAUNCH(FMT_BF16, FMT_E4M3);
  else if (a.act == FMT_F16 && a.cache == FMT_E4M3) PA_LAUNCH(FMT_F16, FMT_E4M3);
  else if (a.act == FMT_BF16 && a.cache == FMT_I8) PA_LAUNCH(FMT_BF16, FMT_I8);
  else if (a.act == FMT_F16 && a.cache == FMT_I8) PA_LAUNCH(FMT_F16, FMT_I8);
  else return hipErrorInvalidValue;
#undef PA_LAUNCH
  return hipGetLastError();
}

}  // namespace pa
