// paged_decode.hip -- split-context paged decode attention for gfx950.
//
// One new query token per sequence attends over that sequence's cached K/V,
// which live in fixed-size pages reached through a block table
// ("PagedAttention in mistral.rs", opening section).  With an E4M3 cache the
// codes are widened on read and the scales are applied once
// (same page, section "KV Cache Quantization").  With window > 0 the table
// addresses a W-row ring ("Rolling buffer cache", llama.cpp discussion 3581,
// opening post) and min(L, W) rows are read.
//
// Work split.  A workgroup of W waves (W = 4 or 8) owns one split of the
// pages of (sequence b, KV head g); its waves take the split's pages
// round-robin, so they stream neighbouring pages side by side, and each wave
// prefetches its next page into a second register buffer while it computes
// the current one.  Per wave and page everything is computed transposed, so
// the probabilities never leave registers:
//
//   * S^T = K Q^T (v_mfma_f32_16x16x32): the page's 32 keys are two 16-row
//     A tiles; 16-bit caches: tile kt row x is key 16 kt + x, so each K
//     load instruction reads whole 128-byte lines; E4M3 and INT8: tile kt
//     row x is key 2x + kt (one 16-byte load per lane holds both tiles'
//     8-byte chunks, whole lines again).  The G query heads of the
//     group are the B columns (columns G..15 are zero); D/32 k-steps.  The K
//     page layout [D/8][32][8] makes each A operand one 16-byte load (one
//     16-byte load holds both tiles' chunks for E4M3).  Lane (q, col) then
//     holds, for head col, the eight consecutive keys 8q .. 8q + 7.
//   * Softmax in log2 units (scale * log2 e folded in) with a lazily moved
//     reference max: only when some score exceeds it by more than 2^8 (a
//     ballot) is the max taken across the four lanes of a head and O
//     rescaled, so a page normally needs no cross-lane reduction at all.
//   * O^T += V^T P^T: the eight probabilities of a lane are exactly its B
//     operand; the A operands are single loads from the transposed V page
//     [D][32] (dimension 16n + col, tokens 8q .. 8q + 7).  One more MFMA
//     against an all-ones A tile accumulates the running sum l.
//
// INT8 cache (per-token/head codes, "libmir-metal 0.2.0,
// src/native/trace/kv.rs", fn build): the codes widen exactly like E4M3, and
// each lane also loads the fp32 scales of its eight keys; the K scales
// multiply the scores, the V scales multiply P for the V MFMAs (the all-ones
// tile takes the unscaled P, so l stays the plain sum).
//
// Append mode (pa_decode_append) also stores the decoded token's K/V into its
// cache row in the same launch; the wave reading that row takes it from LDS.
//
// The W partial results of a workgroup are combined through LDS.  When a
// sequence is one split (S == 1, the usual case once B * Hkv workgroups fill
// the GPU) that is the output; otherwise each split writes (m, l, o) to the
// workspace and counts itself in, and the last split of the (sequence, KV
// head) to arrive combines the S partials in the same launch: M = max m_s,
// w_s = 2^(m_s - M), out = sum w_s o_s / sum w_s l_s.

#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;  // log2 units a row max may grow before rescaling

// Eight cache elements: 16 bytes for 16-bit formats, 8 bytes for E4M3.
template <int CF>
struct Raw8 {
  u32x4 w;
};
template <>
struct Raw8<FMT_E4M3> {
  u32x2 w;
};
template <>
struct Raw8<FMT_I8> {
  u32x2 w;
};

template <int CF, int POLICY = kCacheDefault>
__device__ __forceinline__ Raw8<CF> load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  Raw8<CF> x;
  if constexpr (byte_fmt(CF)) {
    x.w = buf_load8<POLICY>(r, voff, soff);
  } else {
    x.w = buf_load16<POLICY>(r, voff, soff);
  }
  return x;
}

// Eight cache elements as an MFMA operand in the activation format.  E4M3
// values are exact in bf16 and fp16, so the widening is exact.
template <int CF, int AF>
__device__ __forceinline__ typename Mfma<AF>::vec as_operand(const Raw8<CF>& r) {
  if constexpr (CF == FMT_E4M3) {
    return __builtin_bit_cast(typename Mfma<AF>::vec, e4m3x8_to_16<AF>(r.w));
  } else if constexpr (CF == FMT_I8) {
    return __builtin_bit_cast(typename Mfma<AF>::vec, i8x8_to_16<AF>(r.w));
  } else {
    return __builtin_bit_cast(typename Mfma<AF>::vec, r.w);
  }
}

// Registers of one page.  16-bit caches: K operand of key tile kt and k-step
// j is one 16-byte load (key 16 kt + col).  E4M3: one 16-byte load per k-step
// holds the 8-byte chunks of keys 2 col and 2 col + 1, which are row col of
// key tiles 0 and 1.
template <int D, int CF>
struct PageRegs {
  Raw8<CF> k[2][D / 32];   // [key tile][k-step]
  Raw8<CF> v[D / 16];      // [output tile]
};
template <int D>
struct PageRegs<D, FMT_E4M3> {
  u32x4 k[D / 32];         // [k-step]: tile 0 in words 0-1, tile 1 in words 2-3
  Raw8<FMT_E4M3> v[D / 16];
};
// INT8: as E4M3, plus the scales of the lane's eight keys 8q .. 8q + 7.
template <int D>
struct PageRegs<D, FMT_I8> {
  u32x4 k[D / 32];
  Raw8<FMT_I8> v[D / 16];
  f32x4 ks[2];
  f32x4 vs[2];
};

typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, v), mask, 64));
}

// Split partials cross workgroups, and the workgroups of one (sequence, KV
// head) may run on different XCDs, whose L2 caches are not coherent with
// each other.  So the partials are stored and loaded with agent-scope
// atomics (relaxed): on gfx950 these are stores written through to, and
// loads served from, the device's point of coherence, with no L2 write-back
// or invalidate (a release / acquire fence would write back or drop the
// whole L2).  A workgroup's stores are complete (s_waitcnt vmcnt(0)) before
// it counts itself in; the last of the S to arrive merges.
__device__ __forceinline__ void ws_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ws_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the S split partials of one (sequence, query head) with one wave,
// lanes over the head dimension.  Partials are taken 16 at a time with
// every load of a group issued before any use, so a group costs one memory
// round trip; the running max is rescaled between groups.  Empty splits
// carry m = -inf and weigh nothing.
constexpr int kMergeGroup = 16;

template <int D, int AF>
__device__ __forceinline__ void merge_head(uint16_t* __restrict__ dst, int S, float v_scale,
                                           const float* __restrict__ ws_m,
                                           const float* __restrict__ ws_l,
                                           const float* __restrict__ ws_o, size_t row,
                                           int lane) {
  constexpr int DPT = (D + 63) / 64;  // dims per lane
  int dk[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) dk[k] = min(lane + 64 * k, D - 1);

  float M = -INFINITY, den = 0.f, num[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) num[k] = 0.f;
  for (int p0 = 0; p0 < S; p0 += kMergeGroup) {
    const int n = min(kMergeGroup, S - p0);
    float mp[kMergeGroup], lp[kMergeGroup], op[kMergeGroup][DPT];
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i) {
      const size_t r = row + p0 + min(i, n - 1);
      mp[i] = ws_load(ws_m + r);
      lp[i] = ws_load(ws_l + r);
#pragma unroll
      for (int k = 0; k < DPT; ++k) op[i][k] = ws_load(ws_o + r * D + dk[k]);
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i)
      if (i < n) Mg = fmaxf(Mg, mp[i]);
    if (Mg == -INFINITY) continue;  // nothing but empty splits so far
    const float f = M == -INFINITY ? 0.f : fast_exp2(M - Mg);
    den *= f;
#pragma unroll
    for (int k = 0; k < DPT; ++k) num[k] *= f;
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i) {
      const float w = (i < n && mp[i] != -INFINITY) ? fast_exp2(mp[i] - Mg) : 0.f;
      den = fmaf(w, lp[i], den);
#pragma unroll
      for (int k = 0; k < DPT; ++k) num[k] = fmaf(w, op[i][k], num[k]);
    }
    M = Mg;
  }
  const float inv = v_scale / den;
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int d = lane + 64 * k;
    if (d < D) dst[d] = static_cast<uint16_t>(f32_to_16<AF>(num[k] * inv));
  }
}

template <int D, int G, int CF, int AF, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void decode_split(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int Hkv, int MBPS, int window, int S, float qk_scale_log2, float v_scale,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    int* __restrict__ ws_count, const uint16_t* __restrict__ new_key, const uint16_t* __restrict__ new_value,
    float k_enc_scale, float v_enc_scale, float* __restrict__ key_scales,
    float* __restrict__ value_scales) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int EB = byte_fmt(CF) ? 1 : 2;
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  typedef typename Mfma<AF>::vec vec;

  __shared__ float m_lds[W][G];
  __shared__ float l_lds[W][G];
  __shared__ __attribute__((aligned(16))) float o_lds[W][G][D];
  __shared__ __attribute__((aligned(16))) uint16_t newk_lds[D];
  __shared__ __attribute__((aligned(16))) uint16_t newv_lds[D];

  // The wave index is uniform across the wave; saying so keeps everything
  // derived from it (page counts, prefetch indices) in scalar registers.
  // A vector temporary there can be allocated to a register that an
  // in-flight page load targets, which forces a wait for every outstanding
  // load before the next page's loads are issued.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int q4 = lane >> 4;

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = Hkv * G;

  int L = context_lens[b];
  if (window > 0) L = min(L, window);
  if (L <= 0) {
    // Empty context: zeros, written once by split 0.
    if (s == 0) {
      for (int i = threadIdx.x; i < G * D; i += 64 * W) out[((size_t)b * Hq + g * G) * D + i] = 0;
    }
    return;
  }

  // Pages [pa, pb) of the sequence belong to this split; wave w takes pages
  // pa + w, pa + w + W, ... so the waves of the workgroup stream neighbouring
  // pages side by side.
  const int P = (L + kPage - 1) / kPage;
  const int pa = (int)((long long)s * P / S);
  const int pb = (int)((long long)(s + 1) * P / S);
  const int npg = pb - pa > wave ? (pb - pa - wave + W - 1) / W : 0;  // <= 64 (host plan)

  // Append mode: the decoded token's K/V (new_key / new_value [B][Hkv][D])
  // belong in cache row r_new (the last position, or its ring row).  The
  // split that owns that row's page stores it (E4M3-encoded when the cache
  // is FP8; INT8 codes and the row's two scales when it is INT8) and stages
  // the stored cache elements in LDS; the one wave that
  // reads the page patches the row into its page registers, so nothing in
  // this launch depends on the store becoming visible.  The row's loads
  // are issued here, its stores only after the first page's loads, so the
  // append adds no memory round trip before the page stream starts.
  static_assert(D <= 64 * W, "one head-dimension element per thread");
  int row_new = -1, k_new = -1, w_new = -1;
  bool append = false;
  size_t new_page = 0, new_srow = 0;
  uint16_t kx = 0, vx = 0;
  float new_ks = 0.f, new_vs = 0.f;       // INT8: the new row's scales
  constexpr int DPL = CF == FMT_I8 ? (D + 63) / 64 : 1;
  uint16_t krow[DPL], vrow[DPL];          // INT8: this lane's share of the row
  const int d_new = threadIdx.x;
  if (new_key != nullptr) {
    const int ctx = context_lens[b];
    const int r_new = window > 0 ? (ctx - 1) % window : ctx - 1;
    const int pg_new = r_new / kPage;
    if (pg_new >= pa && pg_new < pb) {
      append = true;
      row_new = r_new - pg_new * kPage;
      w_new = (pg_new - pa) % W;
      k_new = (pg_new - pa) / W;
      const int phys = block_tables ? block_tables[(size_t)b * MBPS + pg_new] : b * MBPS + pg_new;
      new_page = ((size_t)phys * Hkv + g) * (size_t)kPage * D;
      new_srow = ((size_t)phys * Hkv + g) * kPage + row_new;
      const size_t src = ((size_t)b * Hkv + g) * D;
      if (d_new < D) {
        kx = new_key[src + d_new];
        vx = new_value[src + d_new];
      }
      if constexpr (CF == FMT_I8) {
        // Every wave reduces the whole row for its scales itself (below),
        // so no wave waits for another; the loads go out now.
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const int d = lane + 64 * i;
          krow[i] = d < D ? new_key[src + d] : 0;
          vrow[i] = d < D ? new_value[src + d] : 0;
        }
      }
    }
  }
  // Store the row (non-temporal: nothing in this launch reads it back from
  // memory; measured 1.3 us faster on the Mistral batch) and stage it in
  // LDS, then make the LDS copy visible to every wave; the global stores
  // need not have completed (__syncthreads would wait for them).  Every
  // wave runs this exactly once.
  auto stage_new_row = [&]() {
    if constexpr (CF == FMT_I8) {
      if (append) {
        // Row scales, amax / 127 as the writer computes them.
        float ka = 0.f, va = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          ka = fmaxf(ka, fabsf(lo16_to_f32<AF>(krow[i])));
          va = fmaxf(va, fabsf(lo16_to_f32<AF>(vrow[i])));
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          ka = fmaxf(ka, shfl_xor_f(ka, m));
          va = fmaxf(va, shfl_xor_f(va, m));
        }
        new_ks = __fdiv_rn(ka, 127.f);
        new_vs = __fdiv_rn(va, 127.f);
      }
    }
    if (append && d_new < D) {
      if constexpr (byte_fmt(CF)) {
        uint32_t kq, vq;
        if constexpr (CF == FMT_I8) {
          kq = i8_encode(lo16_to_f32<AF>(kx), new_ks);
          vq = i8_encode(lo16_to_f32<AF>(vx), new_vs);
          if (d_new == 0) {
            key_scales[new_srow] = new_ks;
            value_scales[new_srow] = new_vs;
          }
        } else {
          kq = e4m3_encode(lo16_to_f32<AF>(kx), k_enc_scale);
          vq = e4m3_encode(lo16_to_f32<AF>(vx), v_enc_scale);
        }
        __builtin_nontemporal_store(static_cast<uint8_t>(kq),
                                    key_cache + new_page + k_page_off(row_new, d_new));
        __builtin_nontemporal_store(static_cast<uint8_t>(vq),
                                    value_cache + new_page + v_page_off(row_new, d_new));
        newk_lds[d_new] = static_cast<uint16_t>(kq);
        newv_lds[d_new] = static_cast<uint16_t>(vq);
      } else {
        __builtin_nontemporal_store(
            kx, reinterpret_cast<uint16_t*>(key_cache) + new_page + k_page_off(row_new, d_new));
        __builtin_nontemporal_store(
            vx, reinterpret_cast<uint16_t*>(value_cache) + new_page + v_page_off(row_new, d_new));
        newk_lds[d_new] = kx;
        newv_lds[d_new] = vx;
      }
    }
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // o_acc[NT] is the all-ones tile: every row holds the running sum l.
  float m_run = -INFINITY;
  f32x4 o_acc[NT + 1];
#pragma unroll
  for (int n = 0; n <= NT; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (npg > 0) {
    // Q^T as the B operand: column = head `col` of the group (zero when
    // col >= G), k-group q4 of k-step j = head-dimension chunk (q4 + 4j).
    vec qb[KSTEPS];
    {
      const uint16_t* qrow = query + ((size_t)b * Hq + g * G + (col < G ? col : 0)) * D;
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * (q4 + 4 * j));
        if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
        qb[j] = __builtin_bit_cast(vec, w);
      }
    }
    const vec ones = __builtin_convertvector(f32x8{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f}, vec);

    const size_t page_elems = (size_t)kPage * D;
    // Physical blocks of this wave's pages, lane k holding its k-th page, so
    // the page loop never waits on a block-table load.  Without a table the
    // map is the identity (block b * MBPS + j) and nothing is loaded.
    const int lpg = pa + wave + W * (lane < npg ? lane : 0);
    const int bt_lane = block_tables ? block_tables[(size_t)b * MBPS + lpg] : b * MBPS + lpg;

    // Per-lane byte offsets inside a page (loop invariant).  K operand of
    // k-step j, key tile kt: chunk (q4 + 4j), key 16 kt + col (16-bit) or
    // keys 2 col and 2 col + 1 (bytes); V operand of output tile n: dim
    // 16n + col, tokens 8 q4 .. 8 q4 + 7.
    constexpr bool kContig = !byte_fmt(CF);
    const int k_lane = ((q4 * kPage + (kContig ? col : 2 * col)) * 8) * EB;
    const int v_lane = (col * kPage + 8 * q4) * EB;
    constexpr int K_J = 4 * kPage * 8 * EB;    // byte step between k-steps
    constexpr int K_KT = 16 * 8 * EB;          // byte step between key tiles (16-bit)
    constexpr int V_N = 16 * kPage * EB;       // byte step between output tiles
    constexpr uint32_t PAGE_BYTES = (uint32_t)kPage * D * EB;

    // Cache policy: every page load reads whole 128-byte lines that nothing
    // else in the launch reads again, so V pages and byte-format K pages
    // stream (non-temporal; this took the FP8 decode from 125 to 114 us).
    // 16-bit K tiles take contiguous keys so that their loads read whole
    // lines too (interleaved tiles, key 2x + kt, shared every line between
    // the two tiles' loads); they stream when a workgroup reads a whole
    // sequence (S == 1: 63.2 -> 61.2 us on the Mistral batch) and keep the
    // default policy when sequences are split (streaming was 3% slower on
    // the 4-split sliding-window batch).
    const bool stream_k = S == 1;
    // Page k of this wave; a prefetch past the last page (k >= npg) gets
    // empty buffer ranges, so its loads return zeros without touching
    // memory and no load sits behind a branch.
    auto load_page = [&](int k, PageRegs<D, CF>& Pg) {
      const bool live = k < npg;
      const int phys = __builtin_amdgcn_readlane(bt_lane, live ? k : 0);
      const size_t base = ((size_t)phys * Hkv + g) * page_elems * EB;
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(key_cache + base, live ? PAGE_BYTES : 0u);
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(value_cache + base, live ? PAGE_BYTES : 0u);
      if constexpr (CF == FMT_I8) {
        // fp32 scales of keys 8 q4 .. 8 q4 + 7 of this (block, head) page.
        const size_t srow = ((size_t)phys * Hkv + g) * kPage;
        const uint32_t sbytes = live ? kPage * 4 : 0u;
        const __amdgpu_buffer_rsrc_t ksr = make_rsrc(key_scales + srow, sbytes);
        const __amdgpu_buffer_rsrc_t vsr = make_rsrc(value_scales + srow, sbytes);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          Pg.ks[h] = __builtin_bit_cast(f32x4, buf_load16(ksr, 32 * q4 + 16 * h, 0));
          Pg.vs[h] = __builtin_bit_cast(f32x4, buf_load16(vsr, 32 * q4 + 16 * h, 0));
        }
      }
      if constexpr (byte_fmt(CF)) {
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) Pg.k[j] = buf_load16<kCacheNT>(kr, k_lane, j * K_J);
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j)
            Pg.k[kt][j] = stream_k ? load8<CF, kCacheNT>(kr, k_lane, j * K_J + kt * K_KT)
                                   : load8<CF>(kr, k_lane, j * K_J + kt * K_KT);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) Pg.v[n] = load8<CF, kCacheNT>(vr, v_lane, n * V_N);
    };

    // K operand of key tile kt, k-step j.
    auto k_operand = [&](const PageRegs<D, CF>& Pg, int kt, int j) -> vec {
      if constexpr (byte_fmt(CF)) {
        Raw8<CF> r;
        r.w = kt == 0 ? u32x2{Pg.k[j][0], Pg.k[j][1]} : u32x2{Pg.k[j][2], Pg.k[j][3]};
        return as_operand<CF, AF>(r);
      } else {
        return as_operand<CF, AF>(Pg.k[kt][j]);
      }
    };

    // Set element e (0..7, any lane-varying value) of a lane's eight
    // consecutive cache elements.  Register arrays are only ever indexed by
    // constants (a runtime index would move them to scratch memory).
    auto set_elem = [&](auto& raw, int e, uint32_t x) {
      constexpr int EPW = byte_fmt(CF) ? 4 : 2;   // elements per word
      constexpr int BITS = 32 / EPW;
      constexpr uint32_t EMASK = (1u << BITS) - 1u;
      const int sh = BITS * (e % EPW);
      const uint32_t keep = ~(EMASK << sh);
      const uint32_t put = (x & EMASK) << sh;
#pragma unroll
      for (int w = 0; w < 8 / EPW; ++w)
        if (w == e / EPW) raw[w] = (raw[w] & keep) | put;
    };

    auto compute_page = [&](PageRegs<D, CF>& Pg, int k) {
      const int base = (pa + wave + W * k) * kPage;
      // The page holding the appended row (a wave-uniform test): put the row
      // into the page registers.  Key row_new is row row_new % 16 of key
      // tile row_new / 16 (16-bit) or row row_new / 2 of tile row_new % 2
      // (bytes); in V it is element row_new % 8 of lane group row_new / 8.
      if (wave == w_new && k == k_new) {
        const int kt_new = kContig ? row_new >> 4 : row_new & 1;
        if (col == (kContig ? row_new & 15 : row_new >> 1)) {
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j) {
            const u32x4 nk = *reinterpret_cast<const u32x4*>(&newk_lds[8 * (q4 + 4 * j)]);
            if constexpr (byte_fmt(CF)) {
              // The codes were staged one per 16-bit slot: pack eight into
              // two words.
              u32x2 c;
#pragma unroll
              for (int w = 0; w < 2; ++w)
                c[w] = (nk[2 * w] & 0xffu) | ((nk[2 * w] >> 8) & 0xff00u) |
                       ((nk[2 * w + 1] & 0xffu) << 16) | ((nk[2 * w + 1] << 8) & 0xff000000u);
              if (kt_new == 0) {
                Pg.k[j][0] = c[0];
                Pg.k[j][1] = c[1];
              } else {
                Pg.k[j][2] = c[0];
                Pg.k[j][3] = c[1];
              }
            } else {
#pragma unroll
              for (int kt = 0; kt < 2; ++kt)
                if (kt == kt_new) Pg.k[kt][j].w = nk;
            }
          }
        }
        if (q4 == (row_new >> 3)) {
#pragma unroll
          for (int n = 0; n < NT; ++n) set_elem(Pg.v[n].w, row_new & 7, newv_lds[16 * n + col]);
          if constexpr (CF == FMT_I8) {
            // The row's scales, as the patched codes were encoded with.
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (e == (row_new & 7)) {
                Pg.ks[e >> 2][e & 3] = new_ks;
                Pg.vs[e >> 2][e & 3] = new_vs;
              }
            }
          }
        }
      }
      // Rows past the context end may hold anything (NaN included): their
      // scores are masked below, and their V elements are zeroed here, since
      // a zero probability times NaN is still NaN.  (A wave-uniform test.)
      const bool partial = base + kPage > L;
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (base + 8 * q4 + e >= L) {
#pragma unroll
            for (int n = 0; n < NT; ++n) set_elem(Pg.v[n].w, e, 0u);
            if constexpr (CF == FMT_I8) Pg.vs[e >> 2][e & 3] = 0.f;  // stale scale
          }
        }
      }

      // S^T = K Q^T; element (kt, r) of lane (q4, col) is key 8 q4 + 2r + kt.
      f32x4 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) st[kt] = Mfma<AF>::mma(k_operand(Pg, kt, j), qb[j], st[kt]);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[kt] *= qk_scale_log2;
      if constexpr (CF == FMT_I8) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) st[kt][r] *= Pg.ks[r >> 1][2 * (r & 1) + kt];
      }
      // Element (kt, r) of a lane is key 16 kt + 4 q4 + r (16-bit) or
      // 8 q4 + 2 r + kt (bytes).
      auto key_of = [&](int kt, int r) {
        return kContig ? 16 * kt + 4 * q4 + r : 8 * q4 + 2 * r + kt;
      };
      if (partial) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (base + key_of(kt, r) >= L) st[kt][r] = -INFINITY;
      }
      const float lmax = fmaxf(fmaxf(fmaxf(st[0][0], st[0][1]), fmaxf(st[0][2], st[0][3])),
                               fmaxf(fmaxf(st[1][0], st[1][1]), fmaxf(st[1][2], st[1][3])));
      // The reference max only moves when some score exceeds it by more than
      // kRescaleSlack (log2 units); it is then raised to the max over the
      // four lanes that hold each head, so all of a head's lanes agree.
      if (__builtin_amdgcn_ballot_w64(lmax > m_run + kRescaleSlack) != 0) {
        float cm = fmaxf(lmax, shfl_xor_f(lmax, 16));
        cm = fmaxf(cm, shfl_xor_f(cm, 32));
        const float m_new = fmaxf(m_run, cm);
        const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
        for (int n = 0; n <= NT; ++n) o_acc[n] *= alpha;
        m_run = m_new;
      }
      // P as the B operand of O^T = V^T P^T: lane (q4, col) must hold the
      // probabilities of keys 8 q4 .. 8 q4 + 7, the tokens of its V operand.
      f32x8 pv;
      vec pb_l;
      if constexpr (kContig) {
        // The lane holds keys 4 q4 + r (words x0, x1) and 16 + 4 q4 + r (y0,
        // y1).  With X_g / Y_g the words of lane group q4 = g, the target
        // groups hold (X0 X1), (X2 X3), (Y0 Y1), (Y2 Y3): a swap of the two
        // lane halves between X and Y, then of odd and even lane groups.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) pv[4 * kt + r] = fast_exp2(st[kt][r] - m_run);
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_convertvector(pv, vec));
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const auto h = __builtin_amdgcn_permlane32_swap(w[i], w[2 + i], false, false);
          const auto q = __builtin_amdgcn_permlane16_swap(h[0], h[1], false, false);
          o[i] = q[0];       // keys 8 q4 + 2i, + 1
          o[2 + i] = q[1];   // keys 8 q4 + 4 + 2i, + 1
        }
        pb_l = __builtin_bit_cast(vec, o);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) pv[2 * r + kt] = fast_exp2(st[kt][r] - m_run);
        pb_l = __builtin_convertvector(pv, vec);
      }
      // l += 1^T P^T.
      o_acc[NT] = Mfma<AF>::mma(ones, pb_l, o_acc[NT]);
      // O^T += V^T P^T; with INT8 each key's V scale goes into its P.
      vec pb = pb_l;
      if constexpr (CF == FMT_I8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] *= Pg.vs[e >> 2][e & 3];
        pb = __builtin_convertvector(pv, vec);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) o_acc[n] = Mfma<AF>::mma(as_operand<CF, AF>(Pg.v[n]), pb, o_acc[n]);
    };

    // Two register buffers: page k is computed while page k + 1 loads.
    PageRegs<D, CF> A, Bf;
    load_page(0, A);
    stage_new_row();
    for (int k = 0;;) {
      load_page(k + 1, Bf);
      compute_page(A, k);
      if (++k >= npg) break;
      load_page(k + 1, A);
      compute_page(Bf, k);
      if (++k >= npg) break;
    }
  } else {
    stage_new_row();
  }

  // Combine the W waves through LDS.  Lane (q4, col) holds O[head col]
  // [dim 16n + 4 q4 + r] and l in every row of the ones tile; waves without
  // pages contribute (-inf, 0, 0).
  if (col < G) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o_lds[wave][col][16 * n + 4 * q4 + r] = o_acc[n][r];
    if (q4 == 0) {
      m_lds[wave][col] = m_run;
      l_lds[wave][col] = o_acc[NT][0];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += 64 * W) {
    const int h = i / D;
    const int d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, m_lds[w][h]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = m_lds[w][h];
        const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        num = fmaf(f, o_lds[w][h][d], num);
        den = fmaf(f, l_lds[w][h], den);
      }
    }
    if (S == 1) {
      out[((size_t)b * Hq + g * G + h) * D + d] = static_cast<uint16_t>(f32_to_16<AF>(num * (v_scale / den)));
    } else {
      const size_t row = ((size_t)b * Hq + g * G + h) * S + s;
      ws_store(ws_o + row * D + d, num);
      if (d == 0) {
        ws_store(ws_m + row, M);
        ws_store(ws_l + row, den);
      }
    }
  }
  if (S == 1) return;

  // Count this split in; the last of the S merges them.  The counter is
  // back at zero when the launch ends.
  __shared__ int last_split;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    int* cnt = ws_count + (size_t)b * Hkv + g;
    const int arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_split = arrived == S - 1;
    if (arrived == S - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last_split) return;
  for (int h = wave; h < G; h += W)
    merge_head<D, AF>(out + ((size_t)b * Hq + g * G + h) * D, S, v_scale, ws_m, ws_l, ws_o,
                      ((size_t)b * Hq + g * G + h) * S, lane);
}

template <int D, int G, int CF, int AF>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const float qk = a.softmax_scale * (CF == FMT_E4M3 ? a.k_scale : 1.f) * LOG2E;
  const float vs = CF == FMT_E4M3 ? a.v_scale : 1.f;
  dim3 grid(a.S, a.Hkv, a.B);
  if (a.W == 8) {
    hipLaunchKernelGGL((decode_split<D, G, CF, AF, 8>), grid, dim3(512), 0, stream,
                       (uint16_t*)a.out, (const uint16_t*)a.query, (uint8_t*)a.key_cache,
                       (uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.Hkv,
                       a.MBPS, a.window, a.S, qk, vs, a.ws_m, a.ws_l, a.ws_o, a.ws_count,
                       (const uint16_t*)a.new_key, (const uint16_t*)a.new_value, a.k_scale,
                       a.v_scale, a.key_scales, a.value_scales);
  } else if (a.W == 4) {
    hipLaunchKernelGGL((decode_split<D, G, CF, AF, 4>), grid, dim3(256), 0, stream,
                       (uint16_t*)a.out, (const uint16_t*)a.query, (uint8_t*)a.key_cache,
                       (uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.Hkv,
                       a.MBPS, a.window, a.S, qk, vs, a.ws_m, a.ws_l, a.ws_o, a.ws_count,
                       (const uint16_t*)a.new_key, (const uint16_t*)a.new_value, a.k_scale,
                       a.v_scale, a.key_scales, a.value_scales);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_fmt(const DecodeArgs& a, hipStream_t s) {
  if (a.act == FMT_BF16) {
    if (a.cache == FMT_BF16) return launch_typed<D, G, FMT_BF16, FMT_BF16>(a, s);
    if (a.cache == FMT_E4M3) return launch_typed<D, G, FMT_E4M3, FMT_BF16>(a, s);
    if (a.cache == FMT_I8) return launch_typed<D, G, FMT_I8, FMT_BF16>(a, s);
  } else if (a.act == FMT_F16) {
    if (a.cache == FMT_F16) return launch_typed<D, G, FMT_F16, FMT_F16>(a, s);
    if (a.cache == FMT_E4M3) return launch_typed<D, G, FMT_E4M3, FMT_F16>(a, s);
    if (a.cache == FMT_I8) return launch_typed<D, G, FMT_I8, FMT_F16>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_group(const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_fmt<D, 1>(a, s);
    case 2: return launch_fmt<D, 2>(a, s);
    case 4: return launch_fmt<D, 4>(a, s);
    case 8: return launch_fmt<D, 8>(a, s);
    case 16: return launch_fmt<D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int D, int G, int act, int cache) {
  if (D != 64 && D != 96 && D != 128) return false;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return false;
  if (act != FMT_BF16 && act != FMT_F16) return false;
  return cache == act || cache == FMT_E4M3 || cache == FMT_I8;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_group<64>(a, s);
    case 96: return launch_group<96>(a, s);
    case 128: return launch_group<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
