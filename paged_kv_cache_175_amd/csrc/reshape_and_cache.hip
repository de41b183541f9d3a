// reshape_and_cache.hip -- the cache slot writer.
//
// Stores each new token's K and V rows into the cache slot named by its slot
// number ("Optimization plans", mistral.rs discussion 46, "Update" post,
// names this operation reshape_and_cache): block slot / 32, row slot % 32, for
// every KV head.  A negative slot skips the token.  With an E4M3 cache each
// element is quantised on the way in ("PagedAttention in mistral.rs",
// section "KV Cache Quantization").
//
// One thread moves one 8-element chunk of one (token, head): a 16-byte read
// of K and of V from the packed [T][Hkv][D] inputs (threads token-major, so
// reads are fully coalesced), one 16-byte (8-byte for E4M3) store of the K
// chunk into the page's [D/8][32][8] layout, and eight 2-byte (1-byte) stores
// of V into the transposed [D][32] page.
#include "common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

template <int AF, int CF>
__global__ __launch_bounds__(256) void cache_write(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ slot_mapping, int T, int Hkv, int D, float k_scale,
    float v_scale) {
  constexpr int EB = (CF == FMT_E4M3) ? 1 : 2;
  const int chunks_per_row = D / 8;
  const long long per_token = (long long)Hkv * chunks_per_row;
  const long long total = (long long)T * per_token;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int n = (int)(i / per_token);
    const int rem = (int)(i - (long long)n * per_token);
    const int h = rem / chunks_per_row;
    const int c = rem - h * chunks_per_row;
    const int slot = slot_mapping[n];
    if (slot < 0) continue;
    const int blk = slot / kPage;
    const int off = slot - blk * kPage;
    const size_t src = ((size_t)n * Hkv + h) * D + 8 * c;
    const size_t page = ((size_t)blk * Hkv + h) * (size_t)kPage * D;
    const size_t kdst = (page + k_page_off(off, 8 * c)) * EB;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(key + src);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(value + src);
    if constexpr (CF == FMT_E4M3) {
      u32x2 kq;
      uint32_t vb[8];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        uint32_t kb = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t kx = kw[2 * w + k], vx = vw[2 * w + k];
          kb |= e4m3_encode(lo16_to_f32<AF>(kx), k_scale) << (16 * k);
          kb |= e4m3_encode(hi16_to_f32<AF>(kx), k_scale) << (16 * k + 8);
          vb[4 * w + 2 * k] = e4m3_encode(lo16_to_f32<AF>(vx), v_scale);
          vb[4 * w + 2 * k + 1] = e4m3_encode(hi16_to_f32<AF>(vx), v_scale);
        }
        kq[w] = kb;
      }
      *reinterpret_cast<u32x2*>(key_cache + kdst) = kq;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        value_cache[page + v_page_off(off, 8 * c + e)] = static_cast<uint8_t>(vb[e]);
    } else {
      *reinterpret_cast<u32x4*>(key_cache + kdst) = kw;
      uint16_t* vdst = reinterpret_cast<uint16_t*>(value_cache);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vdst[page + v_page_off(off, 8 * c + 2 * w)] = static_cast<uint16_t>(vw[w] & 0xffffu);
        vdst[page + v_page_off(off, 8 * c + 2 * w + 1)] = static_cast<uint16_t>(vw[w] >> 16);
      }
    }
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const long long total = (long long)a.T * a.Hkv * (a.D / 8);
  const int threads = 256;
  long long blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  dim3 grid((unsigned)blocks);
  const uint16_t* k = (const uint16_t*)a.key;
  const uint16_t* v = (const uint16_t*)a.value;
  uint8_t* kc = (uint8_t*)a.key_cache;
  uint8_t* vc = (uint8_t*)a.value_cache;
#define PA_LAUNCH(AF, CF)                                                                  \
  hipLaunchKernelGGL((cache_write<AF, CF>), grid, dim3(threads), 0, s, k, v, kc, vc,        \
                     a.slot_mapping, a.T, a.Hkv, a.D, a.k_scale, a.v_scale)
  if (a.act == FMT_BF16 && a.cache == FMT_BF16) PA_LAUNCH(FMT_BF16, FMT_BF16);
  else if (a.act == FMT_F16 && a.cache == FMT_F16) PA_LAUNCH(FMT_F16, FMT_F16);
  else if (a.act == FMT_BF16 && a.cache == FMT_E4M3) PA_LAUNCH(FMT_BF16, FMT_E4M3);
  else if (a.act == FMT_F16 && a.cache == FMT_E4M3) PA_LAUNCH(FMT_F16, FMT_E4M3);
  else return hipErrorInvalidValue;
#undef PA_LAUNCH
  return hipGetLastError();
}

}  // namespace pa
