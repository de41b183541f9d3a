// copy_blocks.hip -- whole-block copies for copy-on-write of shared blocks.
//
// Prefix caching shares cache blocks between sequences ("PagedAttention in
// mistral.rs": prefix caching reuses cached KV; "libmir-metal 0.2.0,
// src/native/trace/kv.rs", fn build: copy-on-write page maps).  When a
// sequence is about to write into a block it shares, it gets a fresh block
// holding a copy of the shared one.  One launch copies N (src, dst) pairs:
// the block's K pages and V pages of every KV head (contiguous in the
// head-major pools) and, for an INT8 cache, its per-row scales.
//
// Grid: x = chunk of the block, y = pair, z = which array (K, V, K scales,
// V scales).  Every lane moves 16-byte chunks; a block of Hkv pages is one
// contiguous run of Hkv * 32 * D * elem bytes, a multiple of 16.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    uint8_t* __restrict__ key_scales, uint8_t* __restrict__ value_scales,
    const int32_t* __restrict__ block_mapping, long long block_bytes, long long scale_bytes) {
  const int pair = blockIdx.y;
  const int which = blockIdx.z;
  const long long src = block_mapping[2 * pair];
  const long long dst = block_mapping[2 * pair + 1];
  uint8_t* base = which == 0 ? key_cache : which == 1 ? value_cache
                : which == 2 ? key_scales : value_scales;
  const long long nbytes = which < 2 ? block_bytes : scale_bytes;
  const u32x4* s = reinterpret_cast<const u32x4*>(base + src * nbytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + dst * nbytes);
  const long long n16 = nbytes / 16;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (long long)gridDim.x * kThreads)
    d[i] = s[i];
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  const long long elem = byte_fmt(a.cache) ? 1 : 2;
  const long long block_bytes = (long long)a.Hkv * kPage * a.D * elem;
  const long long scale_bytes = (long long)a.Hkv * kPage * 4;
  const long long chunks = (block_bytes / 16 + kThreads - 1) / kThreads;
  dim3 grid((unsigned)std::min(chunks, 64LL), a.N, a.cache == FMT_I8 ? 4 : 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, s, (uint8_t*)a.key_cache,
                     (uint8_t*)a.value_cache, (uint8_t*)a.key_scales, (uint8_t*)a.value_scales,
                     a.block_mapping, block_bytes, scale_bytes);
  return hipGetLastError();
}

}  // namespace pa
