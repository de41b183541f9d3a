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
// Work split, two modes chosen by the host plan.  Grid mode (decode_split):
// a workgroup of W waves (W = 4 or 8) owns one split of the pages of
// (sequence b, KV head g) and, in pair mode, also the tail of the sequence
// its own is paired with; its waves claim the job's pages one at a time
// from an LDS counter, so they stream neighbouring pages side by side and
// finish together.  Balanced mode (decode_balanced, E4M3 and INT8 caches
// where pair mode does not apply): the pages of the whole batch are
// cut into equal ranges, one per workgroup, whatever the mix of context
// lengths, and the waves claim a range's pages one at a time.  Either way
// each wave prefetches its next page into a second register buffer while it
// computes the current one.  Per wave and page everything is computed
// transposed, so the probabilities never leave registers:
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
//     operand; the A operands are single loads from the V page
//     [4][D][8] (dimension 16n + col, tokens 8q .. 8q + 7).  One more MFMA
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
// the GPU), or lies wholly in one balanced range, that is the output;
// otherwise each split (range) writes (m, l, o) to the workspace and counts
// itself in, and the last of the (sequence, KV head) to arrive combines the
// S partials in the same launch: M = max m_s, w_s = 2^(m_s - M),
// out = sum w_s o_s / sum w_s l_s.

#include "common.hpp"
#include "launch.hpp"
#include "plan.hpp"

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

// ---------------------------------------------------------------------------
// Per-page work shared by both kernels.

// K operand of key tile kt, k-step j.
template <int D, int CF, int AF>
__device__ __forceinline__ typename Mfma<AF>::vec k_operand(const PageRegs<D, CF>& Pg, int kt, int j) {
  if constexpr (byte_fmt(CF)) {
    Raw8<CF> r;
    r.w = kt == 0 ? u32x2{Pg.k[j][0], Pg.k[j][1]} : u32x2{Pg.k[j][2], Pg.k[j][3]};
    return as_operand<CF, AF>(r);
  } else {
    return as_operand<CF, AF>(Pg.k[kt][j]);
  }
}

// Set element e (0..7, any lane-varying value) of a lane's eight consecutive
// cache elements.  Register arrays are only ever indexed by constants (a
// runtime index would move them to scratch memory).
template <int CF, typename V>
__device__ __forceinline__ void set_elem(V& raw, int e, uint32_t x) {
  constexpr int EPW = byte_fmt(CF) ? 4 : 2;   // elements per word
  constexpr int BITS = 32 / EPW;
  constexpr uint32_t EMASK = (1u << BITS) - 1u;
  const int sh = BITS * (e % EPW);
  const uint32_t keep = ~(EMASK << sh);
  const uint32_t put = (x & EMASK) << sh;
#pragma unroll
  for (int w = 0; w < 8 / EPW; ++w)
    if (w == e / EPW) raw[w] = (raw[w] & keep) | put;
}

// Load one (block, KV head) page, page_id = block * Hkv + head, into
// registers.  Cache policy: every page load reads whole 128-byte lines that
// nothing else in the launch reads again, so V pages and byte-format K pages
// stream (non-temporal; this took the FP8 decode from 125 to 114 us).  16-bit
// K tiles take contiguous keys so that their loads read whole lines too
// (interleaved tiles, key 2x + kt, shared every line between the two tiles'
// loads); they stream when the caller says so (stream_k), which pays where
// a workgroup reads whole sequences (63.2 -> 61.2 us on the Mistral batch)
// and not on short splits (3% slower on the 4-split sliding-window batch).
// A page that is not live (a prefetch past a wave's last page) gets empty
// buffer ranges, so its loads return zeros without touching memory and no
// load sits behind a branch.
template <int D, int CF>
__device__ __forceinline__ void load_page(PageRegs<D, CF>& Pg, const uint8_t* key_cache,
                                          const uint8_t* value_cache, const float* key_scales,
                                          const float* value_scales, uint32_t page_id, bool live,
                                          int lane, bool stream_k) {
  constexpr int EB = byte_fmt(CF) ? 1 : 2;
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  constexpr bool kContig = !byte_fmt(CF);
  const int col = lane & 15;
  const int q4 = lane >> 4;
  // Per-lane byte offsets inside a page.  K operand of k-step j, key tile
  // kt: chunk (q4 + 4j), key 16 kt + col (16-bit) or keys 2 col and
  // 2 col + 1 (bytes); V operand of output tile n: dim 16n + col, tokens
  // 8 q4 .. 8 q4 + 7.
  const int k_lane = ((q4 * kPage + (kContig ? col : 2 * col)) * 8) * EB;
  const int v_lane = (q4 * D + col) * 8 * EB;
  constexpr int K_J = 4 * kPage * 8 * EB;    // byte step between k-steps
  constexpr int K_KT = 16 * 8 * EB;          // byte step between key tiles (16-bit)
  constexpr int V_N = 16 * 8 * EB;           // byte step between output tiles
  constexpr uint32_t PAGE_BYTES = (uint32_t)kPage * D * EB;
  const size_t base = (size_t)page_id * PAGE_BYTES;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(key_cache + base, live ? PAGE_BYTES : 0u);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(value_cache + base, live ? PAGE_BYTES : 0u);
  if constexpr (CF == FMT_I8) {
    // fp32 scales of keys 8 q4 .. 8 q4 + 7 of this (block, head) page.
    const size_t srow = (size_t)page_id * kPage;
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
}

// Attend one page: positions base .. base + 31 of a sequence with L cached
// tokens.  With `patch` (a wave-uniform flag) the page holds the appended
// row row_new, whose stored cache elements newk / newv (and, INT8, scales
// new_ks / new_vs) replace what the loads returned.
template <int D, int G, int CF, int AF>
__device__ __forceinline__ void compute_page(PageRegs<D, CF>& Pg, float& m_run,
                                             f32x4 (&o_acc)[D / 16 + 1],
                                             const typename Mfma<AF>::vec (&qb)[D / 32],
                                             typename Mfma<AF>::vec ones, int base, int L,
                                             bool patch, int row_new, const uint16_t* newk,
                                             const uint16_t* newv, float new_ks, float new_vs,
                                             uint8_t* kpage, uint8_t* vpage, float qk_scale_log2,
                                             int lane) {
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  constexpr bool kContig = !byte_fmt(CF);
  typedef typename Mfma<AF>::vec vec;
  const int col = lane & 15;
  const int q4 = lane >> 4;
  // Key row_new is row row_new % 16 of key tile row_new / 16 (16-bit) or
  // row row_new / 2 of tile row_new % 2 (bytes); in V it is element
  // row_new % 8 of lane group row_new / 8.
  if (patch) {
    // Lane-derived addresses are recomputed here from an opaque copy of the
    // lane index rather than kept live across the caller's page loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int col = ln & 15;
    const int q4 = ln >> 4;
    const int kt_new = kContig ? row_new >> 4 : row_new & 1;
    if (col == (kContig ? row_new & 15 : row_new >> 1)) {
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) {
        const u32x4 nk = *reinterpret_cast<const u32x4*>(&newk[8 * (q4 + 4 * j)]);
        if constexpr (byte_fmt(CF)) {
          // The codes were staged one per 16-bit slot: pack eight into two
          // words.
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
    if (kpage != nullptr) {
      // With kpage / vpage the patched row also goes to the cache here, as
      // whole 128-byte lines: the rest of each line is written back as it
      // was loaded.  A K line is one 8-element chunk of 8 consecutive keys
      // (16-bit) or of 16 (bytes); 16 consecutive dims of a V row group are
      // one line of bytes, two of 16-bit elements.  Full-line writes need no
      // read-modify-write below the cache, which the row's scattered
      // elements did.
      if constexpr (byte_fmt(CF)) {
        if ((col >> 3) == (row_new >> 4)) {
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j)
            __builtin_nontemporal_store(
                Pg.k[j], reinterpret_cast<u32x4*>(kpage + (size_t)(((q4 + 4 * j) * kPage + 2 * col) * 8)));
        }
      } else {
        if ((col >> 3) == ((row_new & 15) >> 3)) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            if (kt == kt_new) {
#pragma unroll
              for (int j = 0; j < KSTEPS; ++j)
                __builtin_nontemporal_store(
                    Pg.k[kt][j].w,
                    reinterpret_cast<u32x4*>(
                        kpage + (size_t)(((q4 + 4 * j) * kPage + 16 * kt + col) * 16)));
            }
          }
        }
      }
    }
    if (q4 == (row_new >> 3)) {
#pragma unroll
      for (int n = 0; n < NT; ++n) set_elem<CF>(Pg.v[n].w, row_new & 7, newv[16 * n + col]);
      if (vpage != nullptr) {
        constexpr int EB = byte_fmt(CF) ? 1 : 2;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          auto* dst = reinterpret_cast<decltype(Pg.v[n].w)*>(
              vpage + (size_t)((q4 * D + 16 * n + col) * 8 * EB));
          __builtin_nontemporal_store(Pg.v[n].w, dst);
        }
      }
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
  // scores are masked below, and their V elements are zeroed here, since a
  // zero probability times NaN is still NaN.  (A wave-uniform test.)
  const bool partial = base + kPage > L;
  if (partial) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (base + 8 * q4 + e >= L) {
#pragma unroll
        for (int n = 0; n < NT; ++n) set_elem<CF>(Pg.v[n].w, e, 0u);
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
    for (int j = 0; j < KSTEPS; ++j)
      st[kt] = Mfma<AF>::mma(k_operand<D, CF, AF>(Pg, kt, j), qb[j], st[kt]);
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
  auto key_of = [&](int kt, int r) { return kContig ? 16 * kt + 4 * q4 + r : 8 * q4 + 2 * r + kt; };
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
  // kRescaleSlack (log2 units); it is then raised to the max over the four
  // lanes that hold each head, so all of a head's lanes agree.
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
    // y1).  With X_g / Y_g the words of lane group q4 = g, the target groups
    // hold (X0 X1), (X2 X3), (Y0 Y1), (Y2 Y3): a swap of the two lane halves
    // between X and Y, then of odd and even lane groups.
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
}

// Q^T of the G heads of one KV head as the B operand: column = head `col`
// (zero when col >= G), k-group q4 of k-step j = head-dimension chunk
// (q4 + 4j).  q points at the group's first head ([G][D], contiguous; global
// memory or LDS).
template <int D, int G, int AF>
__device__ __forceinline__ void q_operand(typename Mfma<AF>::vec (&qb)[D / 32], const uint16_t* q,
                                          int lane) {
  const int col = lane & 15;
  const int q4 = lane >> 4;
  const uint16_t* qrow = q + (col < G ? col : 0) * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * (q4 + 4 * j));
    if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
    qb[j] = __builtin_bit_cast(typename Mfma<AF>::vec, w);
  }
}

template <int AF>
__device__ __forceinline__ typename Mfma<AF>::vec ones_operand() {
  return __builtin_convertvector(f32x8{1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f},
                                 typename Mfma<AF>::vec);
}

// A wave's partial result for its G heads into LDS: lane (q4, col) holds
// O[head col][dim 16n + 4 q4 + r], and l in every row of the ones tile.
template <int D, int G>
__device__ __forceinline__ void put_wave_partial(float (*o)[D], float* m, float* l,
                                                 const f32x4 (&o_acc)[D / 16 + 1], float m_run,
                                                 int lane) {
  const int col = lane & 15;
  const int q4 = lane >> 4;
  if (col < G) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[col][16 * n + 4 * q4 + r] = o_acc[n][r];
    if (q4 == 0) {
      m[col] = m_run;
      l[col] = o_acc[D / 16][0];
    }
  }
}

// Combine the W wave partials of one (head, dim): m[w * ms], l[w * ms],
// o[w * os].  A wave without pages there left m = -inf, and its o and l are
// not read.
template <int W>
__device__ __forceinline__ void combine_waves(const float* m, const float* l, const float* o,
                                              int ms, int os, float& M, float& num, float& den) {
  M = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, m[w * ms]);
  num = 0.f;
  den = 0.f;
  if (M == -INFINITY) return;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float mw = m[w * ms];
    if (mw != -INFINITY) {
      const float f = fast_exp2(mw - M);
      num = fmaf(f, o[w * os], num);
      den = fmaf(f, l[w * ms], den);
    }
  }
}

// One element of the appended row in the cache format: the 16-bit value
// itself, its E4M3 code (scale = the tensor's scale) or its INT8 code
// (scale = the row's amax / 127).
template <int CF, int AF>
__device__ __forceinline__ uint32_t encode_elem(uint16_t x, float scale) {
  if constexpr (CF == FMT_I8) return i8_encode(lo16_to_f32<AF>(x), scale);
  else if constexpr (CF == FMT_E4M3) return e4m3_encode(lo16_to_f32<AF>(x), scale);
  else return x;
}

// Store element d of cache row `row` of the page at element offset `page`
// (balanced mode's appended row; non-temporal: nothing in the launch reads
// it back from memory).
template <int D, int CF>
__device__ __forceinline__ void store_row_elem(uint8_t* key_cache, uint8_t* value_cache,
                                               size_t page, int row, int d, uint32_t kq,
                                               uint32_t vq) {
  if constexpr (byte_fmt(CF)) {
    __builtin_nontemporal_store(static_cast<uint8_t>(kq), key_cache + page + k_page_off(row, d));
    __builtin_nontemporal_store(static_cast<uint8_t>(vq), value_cache + page + v_page_off(row, d, D));
  } else {
    __builtin_nontemporal_store(static_cast<uint16_t>(kq),
                                reinterpret_cast<uint16_t*>(key_cache) + page + k_page_off(row, d));
    __builtin_nontemporal_store(static_cast<uint16_t>(vq),
                                reinterpret_cast<uint16_t*>(value_cache) + page + v_page_off(row, d, D));
  }
}

// ---------------------------------------------------------------------------
// Grid mode: workgroup (s, g, b) reads split s of the pages of (sequence b,
// KV head g).  Pair mode (one split per sequence, the plan's choice for
// batches whose longest sequences would otherwise stream alone at the end):
// workgroup (0, g, b) also reads the tail of the (b', g) item that the
// batch's ranking pairs with b, when b is the shorter of the two
// (plan::pair_split).
//
// An item read by several workgroups (its splits, or its owner and its
// helper) is merged by the last of them to finish (finish_item).
//
// The decoded token's row (append mode) is loaded and encoded (as the writer
// encodes it) into LDS by every workgroup whose job holds its page; the wave
// that claims that page patches the row into its page registers and writes
// the lines that hold the row back to the cache whole (compute_page): no
// extra barrier, and nothing in the launch depends on the stores landing.

// Wave partial of an empty job: the combine skips m = -inf.
template <int G>
__device__ __forceinline__ void put_empty_partial(float* m, int lane) {
  if (lane < G) m[lane] = -INFINITY;
}

// The decoded token's row of (sequence, KV head) `src` (an index into
// new_key / new_value [B][Hkv][D]), lane-major: elements d = lane + 64 i.
template <int D>
__device__ __forceinline__ void load_new_row(uint16_t (&kr)[(D + 63) / 64],
                                             uint16_t (&vr)[(D + 63) / 64],
                                             const uint16_t* new_key, const uint16_t* new_value,
                                             size_t src, int lane) {
#pragma unroll
  for (int i = 0; i < (D + 63) / 64; ++i) {
    const int d = lane + 64 * i;
    kr[i] = d < D ? new_key[src * D + d] : 0;
    vr[i] = d < D ? new_value[src * D + d] : 0;
  }
}

// The row in the cache format, as the writer stores it: the 16-bit values,
// E4M3 codes (tensor scales) or INT8 codes with the row's own scales
// (amax / 127; a reduction over the wave, so every lane must take part).
template <int D, int CF, int AF>
__device__ __forceinline__ void encode_new_row(const uint16_t (&kr)[(D + 63) / 64],
                                               const uint16_t (&vr)[(D + 63) / 64],
                                               uint32_t (&kq)[(D + 63) / 64],
                                               uint32_t (&vq)[(D + 63) / 64], float k_enc_scale,
                                               float v_enc_scale, float& ks, float& vs) {
  constexpr int DPL = (D + 63) / 64;
  ks = k_enc_scale;
  vs = v_enc_scale;
  if constexpr (CF == FMT_I8) {
    float ka = 0.f, va = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      ka = fmaxf(ka, fabsf(lo16_to_f32<AF>(kr[i])));
      va = fmaxf(va, fabsf(lo16_to_f32<AF>(vr[i])));
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      ka = fmaxf(ka, shfl_xor_f(ka, m));
      va = fmaxf(va, shfl_xor_f(va, m));
    }
    ks = __fdiv_rn(ka, 127.f);
    vs = __fdiv_rn(va, 127.f);
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    kq[i] = encode_elem<CF, AF>(kr[i], ks);
    vq[i] = encode_elem<CF, AF>(vr[i], vs);
  }
}

// Finish one item (sequence bj, KV head g) of this workgroup: combine the W
// wave partials of job j from LDS; with one part that is the output.  With
// several, this part publishes its partial (agent-scope stores, complete
// before it counts itself in) and the last part of the item to count in
// merges all of them in slot order (merge_head, one wave per query head), so
// the output is the same bits whichever part merges.
template <int D, int G, int AF, int W, int NJ>
__device__ __forceinline__ void finish_item(
    int j, int bj, int g, int Hkv, int nparts, int slot, float v_scale,
    const float (&m_lds)[NJ][W][G], const float (&l_lds)[NJ][W][G],
    const float (&o_lds)[NJ][W][G][D], int* flag, uint16_t* __restrict__ out,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    int* __restrict__ ws_count, int nslots) {
  const int tid = threadIdx.x;
  const size_t head0 = (size_t)bj * Hkv * G + (size_t)g * G;
  for (int i = tid; i < G * D; i += 64 * W) {
    const int h = i / D;
    const int d = i - h * D;
    float M, num, den;
    combine_waves<W>(&m_lds[j][0][h], &l_lds[j][0][h], &o_lds[j][0][h][d], G, G * D, M, num, den);
    if (nparts == 1) {
      out[head0 * D + i] = static_cast<uint16_t>(f32_to_16<AF>(num * (v_scale / den)));
    } else {
      const size_t row = (head0 + h) * nslots + slot;
      ws_store(ws_o + row * D + d, num);
      if (d == 0) {
        ws_store(ws_m + row, M);
        ws_store(ws_l + row, den);
      }
    }
  }
  if (nparts == 1) return;
  // Count this part in; the last of the item merges.  The counter is back at
  // zero when the launch ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    int* cnt = ws_count + (size_t)bj * Hkv + g;
    const int arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = arrived == nparts - 1;
    if (arrived == nparts - 1) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*flag) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int h = wave; h < G; h += W)
    merge_head<D, AF>(out + (head0 + h) * D, nparts, v_scale, ws_m, ws_l, ws_o,
                      (head0 + h) * nslots, tid & 63);
}

template <int D, int G, int CF, int AF, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void decode_split(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, int B,
    int Hkv, int MBPS, int window, int len_cap, int S, int pair, float qk_scale_log2,
    float v_scale, float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    int* __restrict__ ws_count, const uint16_t* __restrict__ new_key,
    const uint16_t* __restrict__ new_value, float k_enc_scale, float v_enc_scale,
    float* __restrict__ key_scales, float* __restrict__ value_scales) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  constexpr int DPL = (D + 63) / 64;
  // Two jobs (own item, help) where their wave partials fit side by side.
  constexpr int NJ = plan::pair_fits(W, G, D) ? 2 : 1;
  typedef typename Mfma<AF>::vec vec;

  constexpr int TAB = 64 * W;             // pages of one job at most (plan)
  __shared__ float m_lds[NJ][W][G];
  __shared__ float l_lds[NJ][W][G];
  __shared__ __attribute__((aligned(16))) float o_lds[NJ][W][G][D];
  // Page ids (block * Hkv + g) of the jobs' pages: the own job's first,
  // then the help job's.
  __shared__ uint32_t pid_tab[NJ * TAB];
  __shared__ int next_idx;                // next unclaimed page index
  // Per job: the appended row, in the cache format, and (INT8) its scales.
  __shared__ __attribute__((aligned(16))) uint16_t row_lds[NJ][2][D];
  __shared__ float row_scale[NJ][2];
  // The help job's queries.
  __shared__ __attribute__((aligned(16))) uint16_t qh_lds[NJ > 1 ? G * D : 8];
  __shared__ int flag_lds[NJ];

  // The wave index is uniform across the wave; saying so keeps everything
  // derived from it (page counts, prefetch indices) in scalar registers.
  // A vector temporary there can be allocated to a register that an
  // in-flight page load targets, which forces a wait for every outstanding
  // load before the next page's loads are issued.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = Hkv * G;
  const bool append = new_key != nullptr;
  const bool paired = NJ > 1 && pair != 0;
  const int nslots = paired ? 2 : S;

  // --- first round: loads that need neither a length nor the plan --------
  // The own job's table entries go out with the length, for the split's
  // range at the longest length the plan allows (lane k: entry lo_spec +
  // wave + W k, clamped to the row): with one split per sequence that range
  // starts at page 0 whatever the length; with several it is the split's
  // range whenever the sequence is that long (a full ring, the common case
  // of a sliding-window batch).  Otherwise the entries are loaded again
  // after the plan; entries past the job are never used.
  const int p_cap = (int)((len_cap + kPage - 1) / kPage);
  const int lo_spec = S == 1 ? 0 : (int)((long long)s * p_cap / S);
  int bt_pre = 0;
  if (block_tables != nullptr)
    bt_pre = block_tables[(size_t)b * MBPS + min(lo_spec + wave + W * lane, MBPS - 1)];
  vec qb[KSTEPS];
  q_operand<D, G, AF>(qb, query + ((size_t)b * Hq + g * G) * D, lane);
  int lens_lane = 0;                      // pair mode: the batch's lengths (B <= 64)
  if (paired && lane < B) lens_lane = context_lens[lane];
  const int ctx = context_lens[b];
  uint16_t krow[DPL], vrow[DPL];          // wave 0: the own item's appended row
  if (append && wave == 0)
    load_new_row<D>(krow, vrow, new_key, new_value, (size_t)b * Hkv + g, lane);

  // --- the plan ----------------------------------------------------------
  // Lengths are clamped to the host's bound, which the plan was sized for
  // (at most 64 pages per wave).
  const int L = min(ctx, len_cap);
  const int P = L > 0 ? (L + kPage - 1) / kPage : 0;
  int own_lo = 0, own_hi = P;             // own job: pages [own_lo, own_hi) of sequence b
  int own_parts = 1, own_slot = 0;
  int hb = -1, help_lo = 0, help_hi = 0, Lh = 0, ctx_h = 0;  // help job on sequence hb
  if (paired) {
    // Rank the sequences by pages (ties by index), longest first; rank r
    // pairs with rank B - 1 - r.  Lane j's key, pages then 63 - j, orders
    // the batch that way with no two keys equal; this sequence's rank is
    // the count of larger keys (one ballot), and its partner's key the one
    // with exactly B - 1 - r larger keys, found bit by bit from the top
    // (one ballot per key bit; a loop over the B lengths with a lane read
    // per step took ~1 us of every wave's start).
    const int Lx = min(lens_lane, len_cap);
    const int Px = lane < B && Lx > 0 ? (Lx + kPage - 1) / kPage : 0;
    // Lengths within 3 pages of the first sequence's: no two differ by the
    // 2 kMinHelpPages pages a help needs, so nothing is paired (the ranking
    // below would find the same) and it is skipped.
    const int P0 = __builtin_amdgcn_readfirstlane(Px);
    const bool spread = __builtin_amdgcn_ballot_w64(
        lane < B && (Px > P0 + (plan::kMinHelpPages - 1) ||
                     Px + (plan::kMinHelpPages - 1) < P0)) != 0;
    if (spread) {
      const unsigned key = lane < B ? ((unsigned)Px << 6) | (unsigned)(63 - lane) : 0u;
      const unsigned kb = (unsigned)__builtin_amdgcn_readlane((int)key, b);
      const int r = (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(key > kb));
      const int pr = B - 1 - r;
      const int p_max = (int)(((long long)len_cap + kPage - 1) / kPage);   // >= every Px
      const int kbits = 32 - __builtin_clz((unsigned)max(p_max, 1)) + 6;
      unsigned prefix = 0;
      int above = pr;                        // larger keys still to pass
      for (int bit = kbits - 1; bit >= 0; --bit) {
        const unsigned hi = ~((1u << bit) - 1u);
        const unsigned cand = prefix | (1u << bit);
        const int n = (int)__builtin_popcountll(
            __builtin_amdgcn_ballot_w64(lane < B && (key & hi) == cand));
        if (above < n) {
          prefix = cand;
        } else {
          above -= n;
        }
      }
      const int partner = 63 - (int)(prefix & 63u);
      const int Pp = __builtin_amdgcn_readlane(Px, partner);
      if (r < pr) {
        own_hi = plan::pair_split(P, Pp);
        own_parts = own_hi < P ? 2 : 1;
      } else if (r > pr) {
        const int a = plan::pair_split(Pp, P);
        if (a < Pp) {
          hb = partner;
          help_lo = a;
          help_hi = Pp;
          ctx_h = __builtin_amdgcn_readlane(lens_lane, partner);
          Lh = min(ctx_h, len_cap);
        }
      }
    }
  } else if (S > 1) {
    own_lo = (int)((long long)s * P / S);
    own_hi = (int)((long long)(s + 1) * P / S);
    own_parts = S;
    own_slot = s;
  }
  if (P == 0) {
    // Empty context: zeros, written once (its splits all have no pages).
    own_parts = 1;
    if (s == 0)
      for (int i = threadIdx.x; i < G * D; i += 64 * W) out[((size_t)b * Hq + g * G) * D + i] = 0;
    if (hb < 0) return;
  }

  // The jobs' pages, as one list: index i < n0 is page own_lo + i of
  // sequence b, index n0 + j page help_lo + j of sequence hb.  Wave w starts
  // on index w (when the own job has that many pages); from then on each
  // wave claims the next unclaimed index (an LDS counter), so waves the
  // memory system serves faster take more pages and all finish close
  // together (with a static round-robin, the waves of one workgroup
  // finished up to ~8 us apart on the Mistral batch).
  const int n0 = P > 0 ? own_hi - own_lo : 0;      // <= TAB (plan)
  const int n1 = help_hi - help_lo;                // <= TAB
  const int N = n0 + n1;

  // Table entries: thread (wave, lane) holds index wave + W lane of each
  // job (the own job's from the first round when its range is the one
  // guessed there).
  const int ti = wave + W * lane;
  uint32_t own_pid = 0, help_pid = 0;
  if (ti < n0) {
    const int pg = own_lo + ti;
    own_pid = (uint32_t)(block_tables ? (own_lo == lo_spec ? bt_pre
                                                           : block_tables[(size_t)b * MBPS + pg])
                                      : b * MBPS + pg) * Hkv + g;
  }
  if (NJ > 1 && ti < n1) {
    const int pg = help_lo + ti;
    help_pid = (uint32_t)(block_tables ? block_tables[(size_t)hb * MBPS + pg]
                                       : hb * MBPS + pg) * Hkv + g;
  }
  // The help job's queries and appended row (second round).
  constexpr int QCH = G * D / 8;          // 16-byte chunks of the queries
  constexpr int QPT = (QCH + 64 * W - 1) / (64 * W);
  u32x4 qv[QPT];
  if (NJ > 1 && n1 > 0) {
    const uint16_t* src = query + ((size_t)hb * Hq + g * G) * D;
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int c = threadIdx.x + 64 * W * u;
      qv[u] = c < QCH ? *reinterpret_cast<const u32x4*>(src + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Appended rows: the own item's (cache row r0, list index i0) and the help
  // item's (r1, i1), when they lie in this workgroup's pages.
  int r0 = -1, r1 = -1;
  if (append && L > 0) {
    const int r = window > 0 ? (ctx - 1) % window : ctx - 1;
    if (r < L) r0 = r;
  }
  if (append && n1 > 0) {
    const int r = window > 0 ? (ctx_h - 1) % window : ctx_h - 1;
    if (r < Lh) r1 = r;
  }
  const int i0 = r0 >= 0 && r0 / kPage - own_lo >= 0 && r0 / kPage - own_lo < n0
                     ? r0 / kPage - own_lo : -1;
  const int i1 = r1 >= 0 && r1 / kPage - help_lo >= 0 && r1 / kPage - help_lo < n1
                     ? n0 + r1 / kPage - help_lo : -1;
  uint16_t hrow_k[DPL], hrow_v[DPL];      // wave 1 (0 if W == 1): the help row
  const int hwave = W > 1 ? 1 : 0;
  if (NJ > 1 && i1 >= 0 && wave == hwave)
    load_new_row<D>(hrow_k, hrow_v, new_key, new_value, (size_t)hb * Hkv + g, lane);

  // o_acc[NT] is the all-ones tile: every row holds the running sum l.
  float m_run = -INFINITY;
  f32x4 o_acc[NT + 1];
#pragma unroll
  for (int n = 0; n <= NT; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const vec ones = ones_operand<AF>();
  const bool stream_k = S == 1;
  auto fetch = [&](uint32_t pid, bool live, PageRegs<D, CF>& Pg) {
    load_page<D, CF>(Pg, key_cache, value_cache, key_scales, value_scales, pid, live, lane,
                     stream_k);
  };

  // The first page: index `wave`, its id in this wave's own table register.
  const bool first_live = wave < n0;
  PageRegs<D, CF> A, Bf;
  fetch(first_live ? __builtin_amdgcn_readlane(own_pid, 0) : 0u, first_live, A);
  asm volatile("" ::: "memory");

  // Tables, the help job's queries and the appended rows (encoded as the
  // writer encodes them) to LDS; then one barrier (LDS only: the page loads
  // in flight need not complete).
  if (ti < n0) pid_tab[ti] = own_pid;
  if (NJ > 1 && ti < n1) pid_tab[TAB * (NJ - 1) + ti] = help_pid;
  if (NJ > 1 && n1 > 0) {
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int c = threadIdx.x + 64 * W * u;
      if (c < QCH) *reinterpret_cast<u32x4*>(&qh_lds[8 * c]) = qv[u];
    }
  }
  auto stage_row = [&](int j, const uint16_t (&kr)[DPL], const uint16_t (&vr)[DPL]) {
    uint32_t kq[DPL], vq[DPL];
    float ks, vs;
    encode_new_row<D, CF, AF>(kr, vr, kq, vq, k_enc_scale, v_enc_scale, ks, vs);
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const int d = lane + 64 * u;
      if (d < D) {
        row_lds[j][0][d] = static_cast<uint16_t>(kq[u]);
        row_lds[j][1][d] = static_cast<uint16_t>(vq[u]);
      }
    }
    if (lane == 0) {
      row_scale[j][0] = ks;
      row_scale[j][1] = vs;
    }
  };
  if (i0 >= 0 && wave == 0) stage_row(0, krow, vrow);
  if (NJ > 1 && i1 >= 0 && wave == hwave) stage_row(NJ - 1, hrow_k, hrow_v);
  if (threadIdx.x == 0) next_idx = min(n0, W);
  asm volatile("" ::: "memory");
  wait_lgkmcnt0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // Claim the next index (>= N: none left).
  auto claim = [&]() {
    int k = 0;
    if (lane == 0) k = atomicAdd(&next_idx, 1);
    return __builtin_amdgcn_readfirstlane(k);
  };
  auto pid_of = [&](int i) {
    return __builtin_amdgcn_readfirstlane(i < n0 ? pid_tab[i] : pid_tab[TAB * (NJ - 1) + i - n0]);
  };
  int job = 0;                            // the job of the wave's current state
  bool had0 = false;                      // the wave attended an own-job page
  auto step = [&](PageRegs<D, CF>& Pg, int i) {
    const bool help = NJ > 1 && i >= n0;
    if (help && job == 0) {
      // First help page of this wave: keep the own job's wave partial (if
      // it read any), take the help job's queries and a fresh state.  An
      // opaque copy of the lane index keeps the LDS addresses from being
      // hoisted out of the page loop.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      if (had0)
        put_wave_partial<D, G>(o_lds[0][wave], m_lds[0][wave], l_lds[0][wave], o_acc, m_run, ln);
      m_run = -INFINITY;
#pragma unroll
      for (int n = 0; n <= NT; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      q_operand<D, G, AF>(qb, qh_lds, ln);
      job = 1;
    }
    had0 |= !help;
    const int jj = help ? NJ - 1 : 0;
    const int base = (help ? help_lo + i - n0 : own_lo + i) * kPage;
    const bool patch = i == (help ? i1 : i0);
    const int row = (help ? r1 : r0) % kPage;
    // The page that holds the appended row: compute_page patches the row
    // into the loaded page and stores it to the cache (INT8: its scales
    // here).
    constexpr int EB = byte_fmt(CF) ? 1 : 2;
    const size_t pid = patch ? (size_t)pid_of(i) : 0;
    if constexpr (CF == FMT_I8) {
      if (patch && lane == 0) {
        key_scales[pid * kPage + row] = row_scale[jj][0];
        value_scales[pid * kPage + row] = row_scale[jj][1];
      }
    }
    const size_t pbytes = pid * kPage * D * EB;
    compute_page<D, G, CF, AF>(Pg, m_run, o_acc, qb, ones, base, help ? Lh : L, patch, row,
                               row_lds[jj][0], row_lds[jj][1], row_scale[jj][0],
                               row_scale[jj][1], patch ? key_cache + pbytes : nullptr,
                               patch ? value_cache + pbytes : nullptr, qk_scale_log2, lane);
  };

  // Two register buffers: the current page is computed while the next
  // claimed one loads.
  int cur = first_live ? wave : claim();
  if (!first_live && cur < N) fetch(pid_of(cur), true, A);
  if (cur < N) {
    for (;;) {
      const int nx = claim();
      const bool more = nx < N;
      fetch(more ? pid_of(nx) : 0u, more, Bf);
      step(A, cur);
      if (!more) break;
      cur = nx;
      const int ny = claim();
      const bool more2 = ny < N;
      fetch(more2 ? pid_of(ny) : 0u, more2, A);
      step(Bf, cur);
      if (!more2) break;
      cur = ny;
    }
  }

  // Wave partials of the last job; a job this wave read no page of gets an
  // empty partial.
  if (job == 1)
    put_wave_partial<D, G>(o_lds[NJ - 1][wave], m_lds[NJ - 1][wave], l_lds[NJ - 1][wave], o_acc,
                           m_run, lane);
  else if (had0)
    put_wave_partial<D, G>(o_lds[0][wave], m_lds[0][wave], l_lds[0][wave], o_acc, m_run, lane);
  if (!had0) put_empty_partial<G>(m_lds[0][wave], lane);
  if (NJ > 1 && n1 > 0 && job == 0) put_empty_partial<G>(m_lds[NJ - 1][wave], lane);
  __syncthreads();

  // The help job first (its owner is waiting to merge it), then the own job.
  if (NJ > 1 && n1 > 0)
    finish_item<D, G, AF, W, NJ>(NJ - 1, hb, g, Hkv, 2, 1, v_scale, m_lds, l_lds, o_lds,
                                 &flag_lds[NJ - 1], out, ws_m, ws_l, ws_o, ws_count, nslots);
  if (P > 0)
    finish_item<D, G, AF, W, NJ>(0, b, g, Hkv, own_parts, own_slot, v_scale, m_lds,
                                 l_lds, o_lds, &flag_lds[0], out, ws_m, ws_l, ws_o, ws_count,
                                 nslots);
}

// ---------------------------------------------------------------------------
// Balanced mode: the pages of the whole batch, item (b, g) = b * Hkv + g
// after item b * Hkv + g - 1, are cut into equal ranges of c pages, one per
// workgroup, so that every CU reads the same number of bytes whatever the
// mix of context lengths.  A range covers the tail of one item, whole items
// and the head of another; its waves take the range's pages round-robin
// (switching query and softmax state where an item ends) and their partials
// are combined per item through LDS.  An item wholly inside a range is
// written straight to the output; an item cut by range boundaries is
// combined across its workgroups through the workspace (as the splits of
// grid mode).  Items are handled in rounds of at most SEGS items (the LDS
// holds one partial per wave and item of a round).

constexpr int kMaxBalancedB = plan::kMaxBalancedB;

template <int D, int G, int W>
constexpr int balanced_segs() {
  constexpr int s = 98304 / (W * G * D * 4);
  return s < 1 ? 1 : (s > W ? W : s);
}

template <int D, int G, int CF, int AF, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void decode_balanced(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, int B,
    int Hkv, int MBPS, int window, int len_cap, int Smax, int stream_k, float qk_scale_log2,
    float v_scale,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    int* __restrict__ ws_count, const uint16_t* __restrict__ new_key,
    const uint16_t* __restrict__ new_value, float k_enc_scale, float v_enc_scale,
    float* __restrict__ key_scales, float* __restrict__ value_scales) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int SEGS = balanced_segs<D, G, W>();
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  constexpr int DPL = (D + 63) / 64;       // row elements per lane
  constexpr int QCH = G * D / 8;           // 16-byte chunks of one item's queries
  constexpr int QPT = (SEGS * QCH + 64 * W - 1) / (64 * W);
  typedef typename Mfma<AF>::vec vec;

  __shared__ int pref[kMaxBalancedB + 1];  // pages of sequences 0 .. b-1 (per KV head)
  __shared__ int ctx_lds[kMaxBalancedB];
  __shared__ int wsum[W];
  __shared__ int pmax_lds;
  __shared__ float m_lds[SEGS][W][G];
  __shared__ float l_lds[SEGS][W][G];
  __shared__ __attribute__((aligned(16))) float o_lds[SEGS][W][G][D];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[SEGS][G * D];
  __shared__ __attribute__((aligned(16))) uint16_t newk_lds[SEGS][D];
  __shared__ __attribute__((aligned(16))) uint16_t newv_lds[SEGS][D];
  __shared__ float nks_lds[SEGS];
  __shared__ float nvs_lds[SEGS];
  __shared__ int seg_off[SEGS];    // first flat page of the item
  __shared__ int seg_len[SEGS];    // tokens the item attends to
  __shared__ int seg_new[SEGS];    // its appended row, when this range stores it, else -1
  __shared__ int seg_n[SEGS];      // workgroups sharing the item (0: no pages here)
  __shared__ int seg_slot[SEGS];   // this workgroup's partial among them
  __shared__ int seg_last[SEGS];
  __shared__ uint32_t pid_tab[64 * W];   // page ids of the round's pages
  __shared__ int seg_tab[64 * W];        // and their segments
  __shared__ int next_page;              // next unclaimed page of the round

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int Hq = Hkv * G;
  const int N = gridDim.x;
  const int wg = blockIdx.x;

  // Pages per sequence (min(len, window) tokens) and their prefix sums.
  if (threadIdx.x == 0) {
    pref[0] = 0;
    pmax_lds = 0;
  }
  __syncthreads();
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64 * W) {
    const int bi = b0 + (int)threadIdx.x;
    int P = 0;
    if (bi < B) {
      const int ctx = context_lens[bi];
      ctx_lds[bi] = ctx;
      // Clamped to the host's bound, which sized the ranges (at most 64 * W
      // pages each) and the partial slots per item.
      const int L = min(ctx, len_cap);
      P = L > 0 ? (L + kPage - 1) / kPage : 0;
    }
    int x = P, mx = P;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
      mx = max(mx, __shfl_xor(mx, o, 64));
    }
    if (lane == 63) wsum[wave] = x;
    if (lane == 0) atomicMax(&pmax_lds, mx);
    __syncthreads();
    int before = carry, tot = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const int v = wsum[w];
      if (w < wave) before += v;
      tot += v;
    }
    if (bi < B) pref[bi + 1] = before + x;
    carry += tot;
    __syncthreads();
  }
  const int T = Hkv * pref[B];           // pages of the batch (host: < 2^31)
  // Range size: equal shares of N, at least one page per wave, few enough
  // workgroups per item for the workspace (Smax partials), and a multiple of
  // W (every wave of a one-round range gets c / W pages).
  const int c = plan::balanced_range_pages(T, N, pmax_lds, Smax, W);

  // Sequences with no context get zeros (their items hold no pages).
  for (int b = wg; b < B; b += N) {
    if (min(ctx_lds[b], len_cap) <= 0)
      for (int i = threadIdx.x; i < Hq * D; i += 64 * W) out[(size_t)b * Hq * D + i] = 0;
  }
  if ((long long)wg * c >= T) return;
  const int x0 = wg * c;
  const int x1 = min(x0 + c, T);

  // The items holding flat pages x0 and x1 - 1: in the last sequence whose
  // pages start at or before the page (the prefix sums do not decrease, so
  // the sequences that start at or before it are a prefix, counted with
  // ballots), then the head within it.
  int n0 = 0, n1 = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int v = b < B ? Hkv * pref[b] : T;
    n0 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v <= x0));
    n1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v <= x1 - 1));
  }
  auto item_at = [&](int b, int x) {
    return b * Hkv + (x - Hkv * pref[b]) / (pref[b + 1] - pref[b]);
  };
  const int i_first = item_at(n0 - 1, x0);
  const int i_end = item_at(n1 - 1, x1 - 1) + 1;
  const vec ones = ones_operand<AF>();

  for (int i0 = i_first; i0 < i_end; i0 += SEGS) {
    const int nseg = min(SEGS, i_end - i0);
    // Opaque copies of the thread index and of the divisors: what the
    // round's set-up derives from them is recomputed each round, not held in
    // registers across the page loop.
    int tid = threadIdx.x, hkv = Hkv, cr = c, win = window;
    asm volatile("" : "+v"(tid), "+s"(hkv), "+s"(cr), "+s"(win));
    const int ln = tid & 63;
    // Lane s < nseg describes segment s, item i0 + s: its first flat page
    // soff, its length sL (tokens to attend), the flat pages [slo, shi) of
    // it in this range, and the cache row of the appended token when this
    // workgroup holds that row's page (snew, else -1).
    int soff = 0, sL = 0, slo = 0, shi = 0, snew = -1;
    if (ln < nseg) {
      const int i = i0 + ln;
      const int sb = i / hkv;
      const int sg = i - sb * hkv;
      const int P = pref[sb + 1] - pref[sb];
      const int ctx = ctx_lds[sb];
      soff = hkv * pref[sb] + sg * P;
      sL = min(ctx, len_cap);
      slo = max(x0, soff);
      shi = min(x1, soff + P);
      if (new_key != nullptr && shi > slo) {
        const int r = win > 0 ? (ctx - 1) % win : ctx - 1;
        if (soff + r / kPage >= slo && soff + r / kPage < shi) snew = r;
      }
      if (wave == 0) {
        seg_off[ln] = soff;
        seg_len[ln] = sL;
        seg_new[ln] = snew;
        seg_n[ln] = shi > slo ? (soff + P - 1) / cr - soff / cr + 1 : 0;
        seg_slot[ln] = wg - soff / cr;
      }
    }
    const int rs = __builtin_amdgcn_readlane(slo, 0);
    const int re = __builtin_amdgcn_readlane(shi, nseg - 1);

    // Pages of the round, rs + k for k < span.  Wave w starts on page w;
    // from then on each wave claims the next unclaimed page (an LDS
    // counter), so waves that are served faster take more pages and all
    // finish close together.  Thread k tabulates page k's segment and page id
    // (block * Hkv + head) for the claims; a wave's first page is looked up
    // by the wave itself.
    const int span = re - rs;  // <= 64 * W (host plan)
    auto page_info = [&](int k, int& seg) -> uint32_t {
      const int p = rs + k;
      int s = 0, po = __builtin_amdgcn_readlane(soff, 0);
#pragma unroll
      for (int t = 1; t < SEGS; ++t) {
        const int so = __builtin_amdgcn_readlane(soff, t);
        if (t < nseg && p >= so) {
          s = t;
          po = so;
        }
      }
      const int i = i0 + s;
      const int b = i / hkv;
      const int j = p - po;
      const int phys = block_tables ? block_tables[(size_t)b * MBPS + j] : b * MBPS + j;
      seg = s;
      return (uint32_t)phys * hkv + (i - b * hkv);
    };
    int tab_seg = 0;
    uint32_t tab_pid = 0;
    if (tid < span) tab_pid = page_info(tid, tab_seg);
    int first_seg = 0;
    uint32_t first_pid = 0;
    if (wave < span) first_pid = __builtin_amdgcn_readfirstlane(page_info(wave, first_seg));

    // Queries of the round's items, bound for LDS.
    u32x4 qv[QPT];
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int t = tid + 64 * W * u;
      qv[u] = u32x4{0u, 0u, 0u, 0u};
      if (t < nseg * QCH) {
        const int s = t / QCH;
        const int i = i0 + s;
        const int b = i / hkv;
        qv[u] = *reinterpret_cast<const u32x4*>(
            query + ((size_t)b * Hq + (i - b * hkv) * G) * D + 8 * (t - s * QCH));
      }
    }
    // Append: wave s stores segment s's new row if this range holds its
    // page.  Its loads go out now, its stores after the first page's loads.
    const int my_new = wave < nseg ? __builtin_amdgcn_readlane(snew, wave) : -1;
    uint16_t krow[DPL], vrow[DPL];
    int new_phys = 0;
    if (my_new >= 0) {
      const int i = i0 + wave;
      const int b = i / hkv;
      const size_t src = (size_t)i * D;  // new_key [B][Hkv][D]
#pragma unroll
      for (int u = 0; u < DPL; ++u) {
        const int d = ln + 64 * u;
        krow[u] = d < D ? new_key[src + d] : 0;
        vrow[u] = d < D ? new_value[src + d] : 0;
      }
      new_phys = block_tables ? block_tables[(size_t)b * MBPS + my_new / kPage]
                              : b * MBPS + my_new / kPage;
    }

    auto fetch = [&](uint32_t pid, bool live, PageRegs<D, CF>& Pg) {
      load_page<D, CF>(Pg, key_cache, value_cache, key_scales, value_scales, pid, live, lane,
                       stream_k != 0);
    };
    PageRegs<D, CF> A, Bf;
    if (wave < span) fetch(first_pid, true, A);

    // Queries to LDS, empty partial slots, the appended rows; then one
    // barrier (LDS only: the global stores need not have completed).
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int t = tid + 64 * W * u;
      if (t < nseg * QCH) *reinterpret_cast<u32x4*>(&q_lds[0][0] + 8 * t) = qv[u];
    }
    for (int t = tid; t < SEGS * W * G; t += 64 * W) (&m_lds[0][0][0])[t] = -INFINITY;
    if (tid < span) {
      pid_tab[tid] = tab_pid;
      seg_tab[tid] = tab_seg;
    }
    if (tid == 0) next_page = W;
    if (my_new >= 0) {
      const int i = i0 + wave;
      const int row = my_new % kPage;
      const uint32_t pid = (uint32_t)new_phys * hkv + (i - (i / hkv) * hkv);
      const size_t page = (size_t)pid * kPage * D;
      float kes = k_enc_scale, ves = v_enc_scale;
      if constexpr (CF == FMT_I8) {
        // Row scales, amax / 127 as the writer computes them.
        float ka = 0.f, va = 0.f;
#pragma unroll
        for (int u = 0; u < DPL; ++u) {
          ka = fmaxf(ka, fabsf(lo16_to_f32<AF>(krow[u])));
          va = fmaxf(va, fabsf(lo16_to_f32<AF>(vrow[u])));
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          ka = fmaxf(ka, shfl_xor_f(ka, m));
          va = fmaxf(va, shfl_xor_f(va, m));
        }
        kes = __fdiv_rn(ka, 127.f);
        ves = __fdiv_rn(va, 127.f);
        if (ln == 0) {
          key_scales[(size_t)pid * kPage + row] = kes;
          value_scales[(size_t)pid * kPage + row] = ves;
          nks_lds[wave] = kes;
          nvs_lds[wave] = ves;
        }
      }
#pragma unroll
      for (int u = 0; u < DPL; ++u) {
        const int d = ln + 64 * u;
        if (d < D) {
          const uint32_t kq = encode_elem<CF, AF>(krow[u], kes);
          const uint32_t vq = encode_elem<CF, AF>(vrow[u], ves);
          store_row_elem<D, CF>(key_cache, value_cache, page, row, d, kq, vq);
          newk_lds[wave][d] = static_cast<uint16_t>(kq);
          newv_lds[wave][d] = static_cast<uint16_t>(vq);
        }
      }
    }
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    if (wave < span) {
      float m_run = -INFINITY;
      f32x4 o_acc[NT + 1];
      vec qb[KSTEPS];
      int cur = -1, cur_off = 0, cur_L = 0, cur_new = -1;
      float cur_ks = 0.f, cur_vs = 0.f;
      auto flush = [&]() {
        put_wave_partial<D, G>(o_lds[cur][wave], m_lds[cur][wave], l_lds[cur][wave], o_acc,
                               m_run, lane);
      };
      // Claim the next page: its round index (>= span: none left).
      auto claim = [&]() {
        int k = 0;
        if (lane == 0) k = atomicAdd(&next_page, 1);
        return __builtin_amdgcn_readfirstlane(k);
      };
      auto step = [&](PageRegs<D, CF>& Pg, int k, int s) {
        if (s != cur) {
          // A new item: keep the last one's partial, take this one's query.
          if (cur >= 0) flush();
          cur = s;
          m_run = -INFINITY;
#pragma unroll
          for (int n = 0; n <= NT; ++n) o_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
          q_operand<D, G, AF>(qb, q_lds[s], lane);
          cur_off = __builtin_amdgcn_readfirstlane(seg_off[s]);
          cur_L = __builtin_amdgcn_readfirstlane(seg_len[s]);
          cur_new = __builtin_amdgcn_readfirstlane(seg_new[s]);
          if constexpr (CF == FMT_I8) {
            if (cur_new >= 0) {
              cur_ks = nks_lds[s];
              cur_vs = nvs_lds[s];
            }
          }
        }
        const int j = rs + k - cur_off;
        compute_page<D, G, CF, AF>(Pg, m_run, o_acc, qb, ones, j * kPage, cur_L,
                                   cur_new >= 0 && j == cur_new / kPage, cur_new % kPage,
                                   newk_lds[cur], newv_lds[cur], cur_ks, cur_vs, nullptr,
                                   nullptr, qk_scale_log2, lane);
      };
      // Two register buffers: the current page is computed while the next
      // claimed one loads.
      int k = wave, s = __builtin_amdgcn_readfirstlane(first_seg);
      for (;;) {
        const int kn = claim();
        const bool more = kn < span;
        const int sn = more ? __builtin_amdgcn_readfirstlane(seg_tab[kn]) : 0;
        fetch(more ? __builtin_amdgcn_readfirstlane(pid_tab[kn]) : 0u, more, Bf);
        step(A, k, s);
        if (!more) break;
        k = kn;
        s = sn;
        const int km = claim();
        const bool more2 = km < span;
        const int sm = more2 ? __builtin_amdgcn_readfirstlane(seg_tab[km]) : 0;
        fetch(more2 ? __builtin_amdgcn_readfirstlane(pid_tab[km]) : 0u, more2, A);
        step(Bf, k, s);
        if (!more2) break;
        k = km;
        s = sm;
      }
      flush();
    }
    __syncthreads();

    // Combine each item's wave partials: the output when the item is
    // wholly in this range, else this workgroup's partial in the workspace.
    bool shared = false;
    tid = threadIdx.x;
    hkv = Hkv;
    asm volatile("" : "+v"(tid), "+s"(hkv));
    for (int t = tid; t < nseg * G * D; t += 64 * W) {
      const int s = t / (G * D);
      const int h = (t / D) % G;
      const int d = t % D;
      const int n = seg_n[s];
      if (n == 0) continue;
      const int i = i0 + s;
      const int b = i / hkv;
      const size_t head = (size_t)b * Hq + (i - b * hkv) * G + h;
      float M, num, den;
      combine_waves<W>(&m_lds[s][0][h], &l_lds[s][0][h], &o_lds[s][0][h][d], G, G * D, M, num,
                       den);
      if (n == 1) {
        out[head * D + d] = static_cast<uint16_t>(f32_to_16<AF>(num * (v_scale / den)));
      } else {
        const size_t row = head * Smax + seg_slot[s];
        ws_store(ws_o + row * D + d, num);
        if (d == 0) {
          ws_store(ws_m + row, M);
          ws_store(ws_l + row, den);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < SEGS; ++s) shared |= s < nseg && seg_n[s] > 1;
    if (shared) {
      // Count this workgroup in on every cut item; the last of an item's
      // workgroups to arrive merges its partials.  Counters are back at
      // zero when the launch ends.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid < nseg) {
        const int s = tid;
        const int n = seg_n[s];
        int last = 0;
        if (n > 1) {
          int* cnt = ws_count + i0 + s;
          const int arrived =
              __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last = arrived == n - 1;
          if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        seg_last[s] = last;
      }
      __syncthreads();
      for (int t = wave; t < nseg * G; t += W) {
        const int s = t / G;
        if (!seg_last[s]) continue;
        const int i = i0 + s;
        const int b = i / hkv;
        const size_t head = (size_t)b * Hq + (i - b * hkv) * G + (t - s * G);
        merge_head<D, AF>(out + head * D, seg_n[s], v_scale, ws_m, ws_l, ws_o, head * Smax, lane);
      }
    }
    __syncthreads();  // the LDS is reused by the next round
  }
}

template <int D, int G, int CF, int AF, int W>
hipError_t launch_grid(const DecodeArgs& a, float qk, float vs, hipStream_t stream) {
  if (a.pair && !plan::pair_fits(W, G, D)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split<D, G, CF, AF, W>), dim3(a.S, a.Hkv, a.B), dim3(64 * W), 0,
                     stream, (uint16_t*)a.out, (const uint16_t*)a.query, (uint8_t*)a.key_cache,
                     (uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.B, a.Hkv,
                     a.MBPS, a.window, a.len_cap, a.S, a.pair, qk, vs, a.ws_m, a.ws_l,
                     a.ws_o, a.ws_count, (const uint16_t*)a.new_key,
                     (const uint16_t*)a.new_value, a.k_scale, a.v_scale, a.key_scales,
                     a.value_scales);
  return hipGetLastError();
}

template <int D, int G, int CF, int AF>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const float qk = a.softmax_scale * (CF == FMT_E4M3 ? a.k_scale : 1.f) * LOG2E;
  const float vs = CF == FMT_E4M3 ? a.v_scale : 1.f;
  if (a.N > 0) {
    // Balanced mode is planned for byte-format caches only, with W = 8.
    if constexpr (byte_fmt(CF)) {
      if (a.W != 8) return hipErrorInvalidValue;
      hipLaunchKernelGGL((decode_balanced<D, G, CF, AF, 8>), dim3(a.N), dim3(512), 0, stream,
                         (uint16_t*)a.out, (const uint16_t*)a.query, (uint8_t*)a.key_cache,
                         (uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.B, a.Hkv,
                         a.MBPS, a.window, a.len_cap, a.S, a.stream_k, qk, vs, a.ws_m, a.ws_l, a.ws_o,
                         a.ws_count, (const uint16_t*)a.new_key, (const uint16_t*)a.new_value,
                         a.k_scale, a.v_scale, a.key_scales, a.value_scales);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (a.W == 8) return launch_grid<D, G, CF, AF, 8>(a, qk, vs, stream);
  if (a.W == 4) return launch_grid<D, G, CF, AF, 4>(a, qk, vs, stream);
  return hipErrorInvalidValue;
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
