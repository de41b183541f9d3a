// pa_api.cpp -- the C ABI declared in include/pa.h: argument checks, the
// split-context plan and workspace layout, and dispatch to the kernels.
//
// Nothing here allocates device memory or synchronises; every launch goes to
// the caller's stream.  All host-visible arguments are checked before the
// first launch, so an error status means nothing ran.

#include "../../include/pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "launch.hpp"
#include "plan.hpp"

namespace plan = pa::plan;

namespace {

thread_local char g_last_error[256] = "";

pa_status fail(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status fail(pa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

pa_status ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

pa_status hip_fail(hipError_t e, const char* where) {
  return fail(PA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int fmt_of(pa_dtype d) { return static_cast<int>(d); }

bool act_ok(pa_dtype a) { return a == PA_F16 || a == PA_BF16; }

bool cache_ok(pa_dtype act, pa_dtype cache) { return cache == act || cache == PA_F8E4M3; }

size_t elem_bytes(pa_dtype d) { return d == PA_F8E4M3 ? 1 : 2; }

constexpr int kBlock = plan::kBlock;
constexpr int kMaxGridDim = 65535;  // decode grid (splits, Hkv, B); writer and copy grids
constexpr size_t kAlign = plan::kAlign;

// Compute units of the current device, queried once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev < 0 || dev >= 64) return -1;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

using plan::Plan;
using plan::make_plan;
using plan::workspace_for;
using plan::ws_layout;
using plan::WsLayout;
using plan::counter_bytes;
using plan::kMinCounters;

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID: return "PA_ERR_INVALID";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

pa_status cache_write_common(const void* key, const void* value, void* key_cache,
                             void* value_cache, float* key_scales, float* value_scales,
                             const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                             int32_t BS, int32_t NB, pa_dtype act_dtype, pa_dtype cache_dtype,
                             float k_scale, float v_scale, void* stream) {
  if (T < 0) return fail(PA_ERR_INVALID, "T must be >= 0 (got %d)", T);
  if (Hkv < 1 || D < 1 || NB < 1 || BS < 1)
    return fail(PA_ERR_INVALID, "Hkv, D, BS and NB must be positive");
  if (!act_ok(act_dtype)) return fail(PA_ERR_UNSUPPORTED, "act dtype must be PA_F16 or PA_BF16");
  if (BS != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 32 (got %d)", BS);
  if (D % 8 != 0 || D > 512)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8, at most 512");
  if (Hkv > kMaxGridDim) return fail(PA_ERR_UNSUPPORTED, "Hkv must be <= %d", kMaxGridDim);
  if ((long long)NB * BS >= (1LL << 31)) return fail(PA_ERR_INVALID, "NB*BS must be < 2^31");
  if (cache_dtype == PA_F8E4M3 &&
      !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(PA_ERR_INVALID, "E4M3 scales must be finite and > 0");
  if (T == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID, "null pointer argument");
  if (cache_dtype == PA_I8 && (!key_scales || !value_scales))
    return fail(PA_ERR_INVALID, "null scale pool");
  if (!aligned(key, 16) || !aligned(value, 16))
    return fail(PA_ERR_INVALID, "key/value must be 16-byte aligned");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16))
    return fail(PA_ERR_INVALID, "caches must be 16-byte aligned");
  if (!aligned(key_scales, 4) || !aligned(value_scales, 4))
    return fail(PA_ERR_INVALID, "scale pools must be 4-byte aligned");
  pa::CacheWriteArgs a{key,  value, key_cache, value_cache, slot_mapping, T,
                       Hkv,  D,     BS,        fmt_of(act_dtype), fmt_of(cache_dtype),
                       k_scale, v_scale, key_scales, value_scales};
  hipError_t e = pa::launch_cache_write(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reshape_and_cache launch");
  return ok();
}

}  // namespace

extern "C" {

pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int32_t* slot_mapping, int32_t T,
                               int32_t Hkv, int32_t D, int32_t BS, int32_t NB,
                               pa_dtype act_dtype, pa_dtype cache_dtype, float k_scale,
                               float v_scale, void* stream) {
  if (!cache_ok(act_dtype, cache_dtype))
    return fail(PA_ERR_UNSUPPORTED, "cache dtype must equal the act dtype or be PA_F8E4M3");
  return cache_write_common(key, value, key_cache, value_cache, nullptr, nullptr, slot_mapping,
                            T, Hkv, D, BS, NB, act_dtype, cache_dtype, k_scale, v_scale,
                            stream);
}

pa_status pa_reshape_and_cache_i8(const void* key, const void* value, int8_t* key_cache,
                                  int8_t* value_cache, float* key_scales, float* value_scales,
                                  const int32_t* slot_mapping, int32_t T, int32_t Hkv,
                                  int32_t D, int32_t BS, int32_t NB, pa_dtype act_dtype,
                                  void* stream) {
  return cache_write_common(key, value, key_cache, value_cache, key_scales, value_scales,
                            slot_mapping, T, Hkv, D, BS, NB, act_dtype, PA_I8, 1.f, 1.f,
                            stream);
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, float* key_scales,
                         float* value_scales, const int32_t* block_mapping, int32_t N,
                         int32_t Hkv, int32_t D, int32_t BS, int32_t NB, pa_dtype cache_dtype,
                         void* stream) {
  if (N < 0) return fail(PA_ERR_INVALID, "N must be >= 0 (got %d)", N);
  if (Hkv < 1 || D < 1 || NB < 1 || BS < 1)
    return fail(PA_ERR_INVALID, "Hkv, D, BS and NB must be positive");
  if (cache_dtype != PA_F16 && cache_dtype != PA_BF16 && cache_dtype != PA_F8E4M3 &&
      cache_dtype != PA_I8)
    return fail(PA_ERR_UNSUPPORTED, "unknown cache dtype");
  if (BS != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 32 (got %d)", BS);
  if (D % 8 != 0 || D > 512)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 8, at most 512");
  if (Hkv > kMaxGridDim) return fail(PA_ERR_UNSUPPORTED, "Hkv must be <= %d", kMaxGridDim);
  if (N > 65535) return fail(PA_ERR_UNSUPPORTED, "at most 65535 pairs per call");
  if (N == 0) return ok();
  if (!key_cache || !value_cache || !block_mapping)
    return fail(PA_ERR_INVALID, "null pointer argument");
  if (cache_dtype == PA_I8 && (!key_scales || !value_scales))
    return fail(PA_ERR_INVALID, "null scale pool");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(key_scales, 16) ||
      !aligned(value_scales, 16))
    return fail(PA_ERR_INVALID, "pools and scale pools must be 16-byte aligned");
  pa::CopyBlocksArgs a{key_cache, value_cache, key_scales, value_scales, block_mapping,
                       N, Hkv, D, fmt_of(cache_dtype)};
  hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return ok();
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_context_len, int32_t window,
                                 int32_t partition_tokens) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || max_context_len < 0 || window < 0 ||
      partition_tokens < 0)
    return (size_t)-1;
  // The plan depends on the cache format, which this query does not take:
  // the larger of the two workspaces.
  Plan p16, p8;
  const int G = Hq % Hkv == 0 ? Hq / Hkv : 1;
  if (!make_plan(B, Hkv, G, D, max_context_len, window, partition_tokens, false, &p16) ||
      !make_plan(B, Hkv, G, D, max_context_len, window, partition_tokens, true, &p8))
    return (size_t)-1;
  return std::max(workspace_for(B, Hq, Hkv, D, p16), workspace_for(B, Hq, Hkv, D, p8));
}

size_t pa_decode_workspace_bytes_for(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                     int32_t max_context_len, int32_t window,
                                     int32_t partition_tokens, pa_dtype cache_dtype) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || max_context_len < 0 || window < 0 ||
      partition_tokens < 0)
    return (size_t)-1;
  Plan p;
  const int G = Hq % Hkv == 0 ? Hq / Hkv : 1;
  if (!make_plan(B, Hkv, G, D, max_context_len, window, partition_tokens,
                 cache_dtype == PA_F8E4M3 || cache_dtype == PA_I8, &p))
    return (size_t)-1;
  return workspace_for(B, Hq, Hkv, D, p);
}

}  // extern "C"

namespace {

// pa_decode and pa_decode_append share everything but the appended row.
pa_status decode_common(void* out, const void* query, const void* new_key,
                        const void* new_value, const void* key_cache, const void* value_cache,
                        float* key_scales, float* value_scales,
                        const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, int32_t MBPS,
                        int32_t max_context_len, float softmax_scale, pa_dtype act_dtype,
                        pa_dtype cache_dtype, float k_scale, float v_scale, int32_t window,
                        int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || MBPS < 1 || max_context_len < 0)
    return fail(PA_ERR_INVALID, "B, Hq, Hkv, D, MBPS, max_context_len out of range");
  if (B > kMaxGridDim || Hkv > kMaxGridDim)
    return fail(PA_ERR_UNSUPPORTED, "B and Hkv must be <= %d (grid dimensions)", kMaxGridDim);
  if (Hq % Hkv != 0) return fail(PA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!act_ok(act_dtype)) return fail(PA_ERR_UNSUPPORTED, "act dtype must be PA_F16 or PA_BF16");
  if (BS != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 32 (got %d)", BS);
  const int G = Hq / Hkv;
  if (!pa::decode_supported(D, G, fmt_of(act_dtype), fmt_of(cache_dtype)))
    return fail(PA_ERR_UNSUPPORTED, "decode supports head_dim 64/96/128 and Hq/Hkv in {1,2,4,8,16}");
  if (!std::isfinite(softmax_scale)) return fail(PA_ERR_INVALID, "softmax_scale must be finite");
  if (cache_dtype == PA_F8E4M3 &&
      !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(PA_ERR_INVALID, "E4M3 scales must be finite and > 0");
  if (window < 0) return fail(PA_ERR_INVALID, "window must be >= 0");
  if (window > 0 && (window % BS != 0 || window > (long long)MBPS * BS))
    return fail(PA_ERR_INVALID, "window must be a multiple of block_size and <= MBPS*block_size");
  if (window == 0 && max_context_len > (long long)MBPS * BS)
    return fail(PA_ERR_INVALID, "max_context_len exceeds MBPS*block_size");
  if (partition_tokens < 0 || partition_tokens % BS != 0)
    return fail(PA_ERR_INVALID, "partition_tokens must be a non-negative multiple of block_size");
  if (B == 0) return ok();
  if (!out || !query || !key_cache || !value_cache || !context_lens)
    return fail(PA_ERR_INVALID, "null pointer argument");
  if (!block_tables && (long long)B * MBPS > 0x7fffffffLL)
    return fail(PA_ERR_INVALID, "identity map: B * MBPS must fit in int32");
  if (cache_dtype == PA_I8 && (!key_scales || !value_scales))
    return fail(PA_ERR_INVALID, "null scale pool");
  if (!aligned(out, 16) || !aligned(query, 16))
    return fail(PA_ERR_INVALID, "out/query must be 16-byte aligned");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16))
    return fail(PA_ERR_INVALID, "caches must be 16-byte aligned");
  if (!aligned(key_scales, 16) || !aligned(value_scales, 16))
    return fail(PA_ERR_INVALID, "scale pools must be 16-byte aligned");
  if ((long long)B * Hq > 0x7fffffffLL / D) return fail(PA_ERR_UNSUPPORTED, "B*Hq*D too large");
  Plan p;
  if (!make_plan(B, Hkv, G, D, max_context_len, window, partition_tokens,
                 cache_dtype == PA_F8E4M3 || cache_dtype == PA_I8, &p))
    return fail(PA_ERR_INVALID, "bad partition size");
  const size_t need = workspace_for(B, Hq, Hkv, D, p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (need > 0 && !aligned(workspace, kAlign))
    return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  pa::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.B = B;
  a.Hkv = Hkv;
  a.G = G;
  a.D = D;
  a.MBPS = MBPS;
  a.window = window;
  a.len_cap = (int)plan::len_cap(max_context_len, window);
  a.S = p.S;
  a.W = p.W;
  a.pair = p.pair ? 1 : 0;
  if (p.balanced) {
    const long long cus = device_cus();
    if (cus <= 0) return fail(PA_ERR_HIP, "cannot query the device's compute units");
    a.N = (int)plan::balanced_workgroups(B, Hkv, max_context_len, window, cus, p.W);
    a.stream_k = 1;
  }
  a.act = fmt_of(act_dtype);
  a.cache = fmt_of(cache_dtype);
  a.softmax_scale = softmax_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  if (need > 0) {
    const WsLayout l = ws_layout(B, Hq, Hkv, D, p.slots);
    char* w = static_cast<char*>(workspace);
    a.ws_count = reinterpret_cast<int*>(w);
    a.ws_m = reinterpret_cast<float*>(w + l.m);
    a.ws_l = reinterpret_cast<float*>(w + l.l);
    a.ws_o = reinterpret_cast<float*>(w + l.o);
  }
  a.new_key = new_key;
  a.new_value = new_value;
  a.key_scales = key_scales;
  a.value_scales = value_scales;
  hipError_t e = pa::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // namespace

extern "C" {

pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                    int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                    float softmax_scale, pa_dtype act_dtype, pa_dtype cache_dtype,
                    float k_scale, float v_scale, int32_t window,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!cache_ok(act_dtype, cache_dtype))
    return fail(PA_ERR_UNSUPPORTED, "cache dtype must equal the act dtype or be PA_F8E4M3");
  return decode_common(out, query, nullptr, nullptr, key_cache, value_cache, nullptr, nullptr,
                       block_tables,
                       context_lens, B, Hq, Hkv, D, BS, MBPS, max_context_len, softmax_scale,
                       act_dtype, cache_dtype, k_scale, v_scale, window, partition_tokens,
                       workspace, workspace_bytes, stream);
}

pa_status pa_decode_append(void* out, const void* query, const void* key, const void* value,
                           void* key_cache, void* value_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                           float softmax_scale, pa_dtype act_dtype, pa_dtype cache_dtype,
                           float k_scale, float v_scale, int32_t window,
                           int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (B > 0 && (key == nullptr || value == nullptr))
    return fail(PA_ERR_INVALID, "null pointer argument");
  if (!aligned(key, 2) || !aligned(value, 2))
    return fail(PA_ERR_INVALID, "key/value must be 2-byte aligned");
  if (!cache_ok(act_dtype, cache_dtype))
    return fail(PA_ERR_UNSUPPORTED, "cache dtype must equal the act dtype or be PA_F8E4M3");
  return decode_common(out, query, key, value, key_cache, value_cache, nullptr, nullptr,
                       block_tables,
                       context_lens, B, Hq, Hkv, D, BS, MBPS, max_context_len, softmax_scale,
                       act_dtype, cache_dtype, k_scale, v_scale, window, partition_tokens,
                       workspace, workspace_bytes, stream);
}

pa_status pa_decode_i8(void* out, const void* query, const int8_t* key_cache,
                       const int8_t* value_cache, const float* key_scales,
                       const float* value_scales, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                       float softmax_scale, pa_dtype act_dtype, int32_t window,
                       int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                       void* stream) {
  // Read only: the kernel writes the scale pools only when appending.
  return decode_common(out, query, nullptr, nullptr, key_cache, value_cache,
                       const_cast<float*>(key_scales), const_cast<float*>(value_scales),
                       block_tables, context_lens, B, Hq, Hkv, D, BS, MBPS, max_context_len,
                       softmax_scale, act_dtype, PA_I8, 1.f, 1.f, window, partition_tokens,
                       workspace, workspace_bytes, stream);
}

pa_status pa_decode_append_i8(void* out, const void* query, const void* key, const void* value,
                              int8_t* key_cache, int8_t* value_cache, float* key_scales,
                              float* value_scales, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                              float softmax_scale, pa_dtype act_dtype, int32_t window,
                              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (B > 0 && (key == nullptr || value == nullptr))
    return fail(PA_ERR_INVALID, "null pointer argument");
  if (!aligned(key, 2) || !aligned(value, 2))
    return fail(PA_ERR_INVALID, "key/value must be 2-byte aligned");
  return decode_common(out, query, key, value, key_cache, value_cache, key_scales, value_scales,
                       block_tables, context_lens, B, Hq, Hkv, D, BS, MBPS, max_context_len,
                       softmax_scale, act_dtype, PA_I8, 1.f, 1.f, window, partition_tokens,
                       workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The decode scratch of pa_decode_noalloc: a fixed array in device memory,
// one copy per GPU the library runs on, held until the process ends.  Host
// code never uses its name as an address (on the host it is only a stand-in
// for the symbol): the device address comes from hipGetSymbolAddress, once
// per device, and only that pointer is handed to kernels.

static __device__ __align__(256) unsigned char scratch[PA_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Zero n 32-bit words (the counter region) on the stream: a kernel, not a
// memset node, so the set-up may also sit inside a captured graph.
__global__ void zero_words(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The current device's scratch address, set up on the first call on that
// device: the symbol's address there, and its counter region zeroed (a
// decode leaves its counters zero, so this is needed once).
pa_status scratch_for_current_device(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    const int words = (int)(counter_bytes(0, 0) / sizeof(int));
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<int*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch counter zero-fill launch");
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t BS, int32_t MBPS, int32_t max_context_len,
                            float softmax_scale, pa_dtype act_dtype, pa_dtype cache_dtype,
                            float k_scale, float v_scale, int32_t window,
                            int32_t partition_tokens, void* stream) {
  if (!cache_ok(act_dtype, cache_dtype))
    return fail(PA_ERR_UNSUPPORTED, "cache dtype must equal the act dtype or be PA_F8E4M3");
  // The scratch need of this call's plan; invalid arguments are reported by
  // the checks of decode_common below.
  const size_t need = pa_decode_workspace_bytes_for(B, Hq, Hkv, D, max_context_len, window,
                                                    partition_tokens, cache_dtype);
  if (need != (size_t)-1 && need > 0) {
    if (need > (size_t)PA_DECODE_SCRATCH_BYTES)
      return fail(PA_ERR_WORKSPACE,
                  "this decode needs %zu bytes of scratch; the no-allocation entry point has "
                  "%zu (use pa_decode with a workspace)",
                  need, (size_t)PA_DECODE_SCRATCH_BYTES);
    if ((long long)B * Hkv > (long long)kMinCounters)
      return fail(PA_ERR_WORKSPACE,
                  "a split decode over %lld (sequence, KV head) pairs; the no-allocation entry "
                  "point keeps counters for %zu (use pa_decode with a workspace)",
                  (long long)B * Hkv, kMinCounters);
  }
  void* ws = nullptr;
  const pa_status st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st != PA_OK) return st;
  return decode_common(out, query, nullptr, nullptr, key_cache, value_cache, nullptr, nullptr,
                       block_tables, context_lens, B, Hq, Hkv, D, BS, MBPS, max_context_len,
                       softmax_scale, act_dtype, cache_dtype, k_scale, v_scale, window,
                       partition_tokens, ws, (size_t)PA_DECODE_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {

pa_status prefill_common(void* out, const void* query, const int32_t* cu_q_lens,
                         const void* key_cache, const void* value_cache,
                         const float* key_scales, const float* value_scales,
                         const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, int32_t MBPS,
                         int32_t max_chunk_len, float softmax_scale, pa_dtype act_dtype,
                         pa_dtype cache_dtype, float k_scale, float v_scale, void* stream,
                         const void* key_act = nullptr, const void* value_act = nullptr,
                         int32_t window = 0) {
  if (B < 0 || Hq < 1 || Hkv < 1 || D < 1 || MBPS < 1 || max_chunk_len < 0)
    return fail(PA_ERR_INVALID, "B, Hq, Hkv, D, MBPS, max_chunk_len out of range");
  if (Hq % Hkv != 0) return fail(PA_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!act_ok(act_dtype)) return fail(PA_ERR_UNSUPPORTED, "act dtype must be PA_F16 or PA_BF16");
  if (BS != kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 32 (got %d)", BS);
  if (!pa::prefill_supported(D, Hq / Hkv, fmt_of(act_dtype), fmt_of(cache_dtype)))
    return fail(PA_ERR_UNSUPPORTED, "prefill supports head_dim 64/96/128 and Hq/Hkv <= 16");
  // The prefill kernel scales each lane's maximum raw score, which is the
  // maximum scaled score only for a positive scale, and masks raw scores
  // with -inf before scaling them (-inf * 0 would be NaN).
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
    return fail(PA_ERR_INVALID, "prefill softmax_scale must be finite and > 0");
  if (cache_dtype == PA_F8E4M3 &&
      !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(PA_ERR_INVALID, "E4M3 scales must be finite and > 0");
  if (B == 0 || max_chunk_len == 0) return ok();
  if (!out || !query || !cu_q_lens || !key_cache || !value_cache || !context_lens)
    return fail(PA_ERR_INVALID, "null pointer argument");
  if (!block_tables && (long long)B * MBPS > 0x7fffffffLL)
    return fail(PA_ERR_INVALID, "identity map: B * MBPS must fit in int32");
  if (cache_dtype == PA_I8 && (!key_scales || !value_scales))
    return fail(PA_ERR_INVALID, "null scale pool");
  if (!aligned(out, 16) || !aligned(query, 16))
    return fail(PA_ERR_INVALID, "out/query must be 16-byte aligned");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16))
    return fail(PA_ERR_INVALID, "caches must be 16-byte aligned");
  if (!aligned(key_scales, 4) || !aligned(value_scales, 4))
    return fail(PA_ERR_INVALID, "scale pools must be 4-byte aligned");
  if (window > 0) {
    if (!key_act || !value_act) return fail(PA_ERR_INVALID, "null chunk key/value");
    if (!aligned(key_act, 16) || !aligned(value_act, 16))
      return fail(PA_ERR_INVALID, "chunk key/value must be 16-byte aligned");
  }
  // Query rows (position, head) of one sequence and the flat grid must fit in int32.
  if ((long long)max_chunk_len * Hq * B > 0x7fffff00LL)
    return fail(PA_ERR_UNSUPPORTED, "max_chunk_len * Hq * B too large");
  pa::PrefillArgs a{};
  a.out = out;
  a.query = query;
  a.cu_q_lens = cu_q_lens;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.MBPS = MBPS;
  a.max_chunk = max_chunk_len;
  a.act = fmt_of(act_dtype);
  a.cache = fmt_of(cache_dtype);
  a.softmax_scale = softmax_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.key_scales = key_scales;
  a.value_scales = value_scales;
  a.key_act = key_act;
  a.value_act = value_act;
  a.window = window;
  hipError_t e = pa::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

}  // namespace

extern "C" {

pa_status pa_prefill_chunk(void* out, const void* query, const int32_t* cu_q_lens,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                           int32_t MBPS, int32_t max_chunk_len, float softmax_scale,
                           pa_dtype act_dtype, pa_dtype cache_dtype, float k_scale,
                           float v_scale, void* stream) {
  if (!cache_ok(act_dtype, cache_dtype))
    return fail(PA_ERR_UNSUPPORTED, "cache dtype must equal the act dtype or be PA_F8E4M3");
  return prefill_common(out, query, cu_q_lens, key_cache, value_cache, nullptr, nullptr,
                        block_tables, context_lens, B, Hq, Hkv, D, BS, MBPS, max_chunk_len,
                        softmax_scale, act_dtype, cache_dtype, k_scale, v_scale, stream);
}

pa_status pa_prefill_chunk_i8(void* out, const void* query, const int32_t* cu_q_lens,
                              const int8_t* key_cache, const int8_t* value_cache,
                              const float* key_scales, const float* value_scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                              int32_t MBPS, int32_t max_chunk_len, float softmax_scale,
                              pa_dtype act_dtype, void* stream) {
  return prefill_common(out, query, cu_q_lens, key_cache, value_cache, key_scales,
                        value_scales, block_tables, context_lens, B, Hq, Hkv, D, BS, MBPS,
                        max_chunk_len, softmax_scale, act_dtype, PA_I8, 1.f, 1.f, stream);
}

pa_status pa_prefill_chunk_window(void* out, const void* query, const void* key,
                                  const void* value, const int32_t* cu_q_lens,
                                  const void* key_cache, const void* value_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS,
                                  int32_t MBPS, int32_t max_chunk_len, float softmax_scale,
                                  pa_dtype act_dtype, int32_t window, void* stream) {
  return pa_prefill_chunk_window_quant(out, query, key, value, cu_q_lens, key_cache,
                                       value_cache, nullptr, nullptr, block_tables, context_lens,
                                       B, Hq, Hkv, D, BS, MBPS, max_chunk_len, softmax_scale,
                                       act_dtype, act_dtype, 1.f, 1.f, window, stream);
}

pa_status pa_prefill_chunk_window_quant(void* out, const void* query, const void* key,
                                        const void* value, const int32_t* cu_q_lens,
                                        const void* key_cache, const void* value_cache,
                                        const float* key_scales, const float* value_scales,
                                        const int32_t* block_tables, const int32_t* context_lens,
                                        int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t BS, int32_t MBPS, int32_t max_chunk_len,
                                        float softmax_scale, pa_dtype act_dtype,
                                        pa_dtype cache_dtype, float k_scale, float v_scale,
                                        int32_t window, void* stream) {
  if (window <= 0 || window % kBlock != 0)
    return fail(PA_ERR_INVALID, "window must be a positive multiple of 32 (got %d)", window);
  if (MBPS < 1 || window / kBlock > MBPS)
    return fail(PA_ERR_INVALID, "the ring of %d rows needs %d table entries (MBPS %d)", window,
                window / kBlock, MBPS);
  if (cache_dtype != act_dtype && cache_dtype != PA_F8E4M3 && cache_dtype != PA_I8)
    return fail(PA_ERR_UNSUPPORTED,
                "ring dtype must equal the act dtype or be PA_F8E4M3 or PA_I8");
  if (cache_dtype != PA_F8E4M3) k_scale = v_scale = 1.f;
  if (cache_dtype != PA_I8) key_scales = value_scales = nullptr;
  return prefill_common(out, query, cu_q_lens, key_cache, value_cache, key_scales,
                        value_scales, block_tables, context_lens, B, Hq, Hkv, D, BS, MBPS,
                        max_chunk_len, softmax_scale, act_dtype, cache_dtype, k_scale, v_scale,
                        stream, key, value, window);
}

}  // extern "C"
