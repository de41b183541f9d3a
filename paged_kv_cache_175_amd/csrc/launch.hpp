// launch.hpp -- internal interface between the C ABI (pa_api.cpp) and the
// kernel translation units.  Not part of the public API.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int32_t* slot_mapping;
  int T, Hkv, D, BS;
  int act, cache;  // Fmt codes
  float k_scale, v_scale;
  float* key_scales;    // INT8 cache: [NB][Hkv][BS] fp32, written per row
  float* value_scales;
};

struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int B, Hkv, G, D, MBPS, window;
  // Tokens a sequence may attend to at most: max_context_len, capped at the
  // window.  The kernels clamp each length to it, so a length above the
  // host's bound cannot take a wave past the pages the plan sized it for.
  int len_cap;
  int S;  // grid mode: splits per (sequence, KV head); balanced: partials per item
  int pair;  // grid mode, one split: short sequences help long ones
  int W;  // waves per workgroup (4 or 8)
  int N;  // balanced mode: workgroups (0 = grid mode)
  int stream_k;  // balanced mode: 16-bit K pages non-temporal
  int act, cache;  // Fmt codes
  float softmax_scale, k_scale, v_scale;
  float* ws_m;  // [B*Hq*slots]
  float* ws_l;  // [B*Hq*slots]
  float* ws_o;  // [B*Hq*slots*D]
  int* ws_count;  // split arrival counters (B*Hkv used), zero between launches
  const void* new_key;    // append mode: [B][Hkv][D] act, or null
  const void* new_value;
  float* key_scales;    // INT8 cache: [NB][Hkv][BS] fp32 (written by an append)
  float* value_scales;
};

struct PrefillArgs {
  void* out;
  const void* query;
  const int32_t* cu_q_lens;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int B, Hq, Hkv, D, MBPS, max_chunk;
  int act, cache;
  float softmax_scale, k_scale, v_scale;
  const float* key_scales;    // INT8 cache: [NB][Hkv][BS] fp32
  const float* value_scales;
  // Sliding-window layer: window > 0, the cache is a ring of `window` rows
  // and key_act / value_act [total_q][Hkv][D] hold the chunk's own K/V.
  const void* key_act;
  const void* value_act;
  int window;
};

struct CopyBlocksArgs {
  void* key_cache;
  void* value_cache;
  float* key_scales;     // INT8 cache only
  float* value_scales;
  const int32_t* block_mapping;  // [N][2] (src, dst)
  int N, Hkv, D;
  int cache;  // Fmt code
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);

bool decode_supported(int D, int G, int act, int cache);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

bool prefill_supported(int D, int G, int act, int cache);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

}  // namespace pa
