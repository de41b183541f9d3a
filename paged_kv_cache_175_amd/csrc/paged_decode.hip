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
// Work split.  One 64-lane wave owns (sequence b, KV head g, partition p), a
// partition being `part_tok` consecutive tokens (whole 32-token pages).  The
// wave keeps the G query heads of the group as the rows of 16x16 MFMA tiles
// (rows G..15 are zero) and streams its pages, prefetching page n+1 into a
// second register buffer while it computes page n:
//
//   * S = Q K^T: two 16x16x32 tiles of 16 tokens, D/32 k-steps each.  The K
//     page layout [D/8][32][8] makes every B operand one 16-byte load
//     (8 bytes for E4M3).
//   * Online softmax in log2 units (scale * log2 e folded in): each MFMA
//     output row is one head, so the per-head page max and sum are 16-lane
//     row reductions done entirely in DPP.
//   * P goes through 1 KiB of LDS into the MFMA A-operand layout (the only
//     transpose), and O += P V runs as D/16 16x16x32 MFMAs whose B operands
//     are single loads from the transposed V page [D][32].
//
// A partition either writes the normalised output (when it is the only one
// of its sequence) or its unnormalised (m, l, o) to the workspace; a second
// kernel merges partitions: M = max m_p, w_p = 2^(m_p - M),
// out = sum w_p o_p / sum w_p l_p.

#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int PROW = kPage + 8;  // LDS row of P (16-bit elements), padded
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

template <int CF>
__device__ __forceinline__ Raw8<CF> load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  Raw8<CF> x;
  if constexpr (CF == FMT_E4M3) {
    x.w = buf_load8(r, voff, soff);
  } else {
    x.w = buf_load16(r, voff, soff);
  }
  return x;
}

// Eight cache elements as an MFMA operand in the activation format.  E4M3
// values are exact in bf16 and fp16, so the widening is exact.
template <int CF, int AF>
__device__ __forceinline__ typename Mfma<AF>::vec as_operand(const Raw8<CF>& r) {
  if constexpr (CF == FMT_E4M3) {
    return __builtin_bit_cast(typename Mfma<AF>::vec, e4m3x8_to_16<AF>(r.w));
  } else {
    return __builtin_bit_cast(typename Mfma<AF>::vec, r.w);
  }
}

// Registers of one page.  16-bit caches: K operand of token tile tt and
// k-step j is one 16-byte load (token col + 16 tt).  E4M3: one 16-byte load
// per k-step holds the 8-byte chunks of tokens 2 col and 2 col + 1, which are
// column col of token tiles 0 and 1.
template <int D, int CF>
struct PageRegs {
  Raw8<CF> k[2][D / 32];   // [token tile][k-step]
  Raw8<CF> v[D / 16];      // [output tile]
};
template <int D>
struct PageRegs<D, FMT_E4M3> {
  u32x4 k[D / 32];         // [k-step]: tile 0 in words 0-1, tile 1 in words 2-3
  Raw8<FMT_E4M3> v[D / 16];
};

// Token of a page held in MFMA column `col` of token tile `tt`.
template <int CF>
__device__ __forceinline__ int tile_token(int tt, int col) {
  return CF == FMT_E4M3 ? 2 * col + tt : col + 16 * tt;
}

template <int D, int G, int CF, int AF>
__global__ __launch_bounds__(64) void decode_pass1(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int Hkv, int MBPS, int window, int part_tok, int NP, float qk_scale_log2,
    float v_scale, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int EB = (CF == FMT_E4M3) ? 1 : 2;
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  typedef typename Mfma<AF>::vec vec;

  __shared__ __attribute__((aligned(16))) uint16_t p_lds[16 * PROW];

  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int r4 = lane >> 4;

  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = Hkv * G;

  int L = context_lens[b];
  if (window > 0) L = min(L, window);
  const int nparts = (L + part_tok - 1) / part_tok;

  if (L <= 0) {
    // Empty context: zeros, written once by partition 0.
    if (p == 0) {
      for (int i = lane; i < G * D; i += 64) out[((size_t)b * Hq + g * G) * D + i] = 0;
    }
    return;
  }
  if (p >= nparts) return;

  const int t0 = p * part_tok;
  const int t1 = min(L, t0 + part_tok);
  const int pg0 = t0 / kPage;
  const int pg1 = (t1 + kPage - 1) / kPage;

  // Q as the A operand: row = head `col` of the group (zero when col >= G),
  // k-group r4 of k-step j = head-dimension chunk (r4 + 4j).
  vec qa[KSTEPS];
  {
    const uint16_t* qrow = query + ((size_t)b * Hq + g * G + (col < G ? col : 0)) * D;
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * (r4 + 4 * j));
      if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
      qa[j] = __builtin_bit_cast(vec, w);
    }
  }

  const size_t page_elems = (size_t)kPage * D;
  const int32_t* bt = block_tables + (size_t)b * MBPS;

  // Per-lane byte offsets inside a page (loop invariant).  K operand of
  // k-step j, token tile tt: chunk (r4 + 4j), token tile_token(tt, col); V
  // operand of output tile n: dim 16n + col, tokens 8 r4 .. 8 r4 + 7.
  const int k_lane = ((r4 * kPage + tile_token<CF>(0, col)) * 8) * EB;
  const int v_lane = (col * kPage + 8 * r4) * EB;
  constexpr int K_J = 4 * kPage * 8 * EB;    // byte step between k-steps
  constexpr int K_TT = 16 * 8 * EB;          // byte step between token tiles (16-bit)
  constexpr int V_N = 16 * kPage * EB;       // byte step between output tiles
  constexpr uint32_t PAGE_BYTES = (uint32_t)kPage * D * EB;

  // Physical blocks of this partition, lane i holding page pg0 + i (a
  // partition spans at most 64 pages), so the page loop never waits on a
  // block-table load.
  const int npg = pg1 - pg0;
  const int bt_lane = bt[pg0 + (lane < npg ? lane : 0)];

  auto load_page = [&](int pg, PageRegs<D, CF>& P) {
    const int phys = __builtin_amdgcn_readlane(bt_lane, pg - pg0);
    const size_t base = ((size_t)phys * Hkv + g) * page_elems * EB;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(key_cache + base, PAGE_BYTES);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(value_cache + base, PAGE_BYTES);
    if constexpr (CF == FMT_E4M3) {
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) P.k[j] = buf_load16(kr, k_lane, j * K_J);
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) P.k[tt][j] = load8<CF>(kr, k_lane, j * K_J + tt * K_TT);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) P.v[n] = load8<CF>(vr, v_lane, n * V_N);
  };

  // K operand of token tile tt, k-step j.
  auto k_operand = [&](const PageRegs<D, CF>& P, int tt, int j) -> vec {
    if constexpr (CF == FMT_E4M3) {
      Raw8<CF> r;
      r.w = tt == 0 ? u32x2{P.k[j][0], P.k[j][1]} : u32x2{P.k[j][2], P.k[j][3]};
      return as_operand<CF, AF>(r);
    } else {
      return as_operand<CF, AF>(P.k[tt][j]);
    }
  };

  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_page = [&](const PageRegs<D, CF>& P, int pg) {
    // S = Q K^T; lane (r4, col) gets heads 4*r4 + r, tokens tok0 and tok1.
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j) s[tt] = Mfma<AF>::mma(qa[j], k_operand(P, tt, j), s[tt]);
    }
    const int base = pg * kPage;
    const int tok0 = tile_token<CF>(0, col);
    const int tok1 = tile_token<CF>(1, col);
    const bool live0 = base + tok0 < t1;
    const bool live1 = base + tok1 < t1;
    float sc[4][2], pm[4];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r][0] = live0 ? s[0][r] * qk_scale_log2 : -INFINITY;
      sc[r][1] = live1 ? s[1][r] * qk_scale_log2 : -INFINITY;
      pm[r] = row16_max(fmaxf(sc[r][0], sc[r][1]));
      grow |= pm[r] > m_run[r] + kRescaleSlack;
    }
    // The running reference max only moves when some row's page max exceeds
    // it by more than kRescaleSlack (log2 units); otherwise probabilities are
    // taken against the old reference (they stay below 2^kRescaleSlack) and
    // the output needs no rescaling.  The test is wave-uniform.
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m_new = fmaxf(m_run[r], pm[r]);
        const float alpha = fast_exp2(m_run[r] - m_new);
        l_run[r] *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n][r] *= alpha;
        m_run[r] = m_new;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e0 = fast_exp2(sc[r][0] - m_run[r]);
      const float e1 = fast_exp2(sc[r][1] - m_run[r]);
      l_run[r] += row16_sum(e0 + e1);
      if constexpr (CF == FMT_E4M3) {
        // Tokens 2 col and 2 col + 1: one 32-bit store.
        *reinterpret_cast<uint32_t*>(&p_lds[(4 * r4 + r) * PROW + tok0]) =
            (uint32_t)cvt16<AF>(e0) | ((uint32_t)cvt16<AF>(e1) << 16);
      } else {
        p_lds[(4 * r4 + r) * PROW + tok0] = cvt16<AF>(e0);
        p_lds[(4 * r4 + r) * PROW + tok1] = cvt16<AF>(e1);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // A operand: P[head col][tokens 8*r4 .. 8*r4 + 7].
    const vec pa = *reinterpret_cast<const vec*>(&p_lds[col * PROW + 8 * r4]);
    // Rows past the context end may hold anything (NaN included); their
    // probabilities are 0, but 0 * NaN is NaN, so those V values are zeroed
    // on the (uniform) last partial page.
    const bool partial = base + kPage > t1;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      vec vb = as_operand<CF, AF>(P.v[n]);
      if (partial) {
        u32x4 w = __builtin_bit_cast(u32x4, vb);
        const int tok = base + 8 * r4;  // this lane holds tokens tok .. tok + 7
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (tok + 2 * e < t1) ? 0xffffu : 0u;
          const uint32_t hi = (tok + 2 * e + 1 < t1) ? 0xffff0000u : 0u;
          w[e] &= (lo | hi);
        }
        vb = __builtin_bit_cast(vec, w);
      }
      acc[n] = Mfma<AF>::mma(pa, vb, acc[n]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  // Two register buffers: page pg is computed while page pg + 1 loads.  The
  // prefetch past the last page re-reads the last page (an L2 hit) so that
  // no load sits behind a branch.
  PageRegs<D, CF> A, Bf;
  load_page(pg0, A);
  for (int pg = pg0;;) {
    load_page(min(pg + 1, pg1 - 1), Bf);
    compute_page(A, pg);
    if (++pg >= pg1) break;
    load_page(min(pg + 1, pg1 - 1), A);
    compute_page(Bf, pg);
    if (++pg >= pg1) break;
  }

  // Lane (r4, col) holds O[head 4*r4 + r][dim 16n + col].
  if (nparts == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * r4 + r;
      if (h >= G) continue;
      const float inv = v_scale / l_run[r];
      uint16_t* o = out + ((size_t)b * Hq + g * G + h) * D + col;
#pragma unroll
      for (int n = 0; n < NT; ++n) o[16 * n] = static_cast<uint16_t>(f32_to_16<AF>(acc[n][r] * inv));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * r4 + r;
      if (h >= G) continue;
      const size_t row = ((size_t)b * Hq + g * G + h) * NP + p;
      float* o = ws_o + row * D + col;
#pragma unroll
      for (int n = 0; n < NT; ++n) o[16 * n] = acc[n][r];
      if (col == 0) {
        ws_m[row] = m_run[r];
        ws_l[row] = l_run[r];
      }
    }
  }
}

// Merge the partitions of one (sequence, query head): one wave.  Partitions
// are taken 16 at a time with every load of a group issued before any use, so
// a group costs one memory round trip; the running max is rescaled between
// groups.
constexpr int kMergeGroup = 16;

template <int D, int AF>
__global__ __launch_bounds__(64) void decode_pass2(
    uint16_t* __restrict__ out, const int32_t* __restrict__ context_lens, int Hq, int window,
    int part_tok, int NP, float v_scale, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const float* __restrict__ ws_o) {
  constexpr int DPT = (D + 63) / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = context_lens[b];
  if (window > 0) L = min(L, window);
  const int nparts = (L + part_tok - 1) / part_tok;
  if (nparts <= 1) return;  // written by pass 1
  const size_t row = ((size_t)b * Hq + h) * NP;
  int dk[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) dk[k] = min(lane + 64 * k, D - 1);

  float M = -INFINITY, den = 0.f, num[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) num[k] = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += kMergeGroup) {
    const int n = min(kMergeGroup, nparts - p0);
    float mp[kMergeGroup], lp[kMergeGroup], op[kMergeGroup][DPT];
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i) {
      const size_t r = row + p0 + min(i, n - 1);
      mp[i] = ws_m[r];
      lp[i] = ws_l[r];
#pragma unroll
      for (int k = 0; k < DPT; ++k) op[i][k] = ws_o[r * D + dk[k]];
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i)
      if (i < n) Mg = fmaxf(Mg, mp[i]);
    const float f = fast_exp2(M - Mg);
    den *= f;
#pragma unroll
    for (int k = 0; k < DPT; ++k) num[k] *= f;
#pragma unroll
    for (int i = 0; i < kMergeGroup; ++i) {
      const float w = i < n ? fast_exp2(mp[i] - Mg) : 0.f;
      den = fmaf(w, lp[i], den);
#pragma unroll
      for (int k = 0; k < DPT; ++k) num[k] = fmaf(w, op[i][k], num[k]);
    }
    M = Mg;
  }
  const float inv = v_scale / den;
  uint16_t* dst = out + ((size_t)b * Hq + h) * D;
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int d = lane + 64 * k;
    if (d < D) dst[d] = static_cast<uint16_t>(f32_to_16<AF>(num[k] * inv));
  }
}

template <int D, int G, int CF, int AF>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const float qk = a.softmax_scale * (CF == FMT_E4M3 ? a.k_scale : 1.f) * LOG2E;
  const float vs = CF == FMT_E4M3 ? a.v_scale : 1.f;
  dim3 grid1(a.NP, a.Hkv, a.B);
  hipLaunchKernelGGL((decode_pass1<D, G, CF, AF>), grid1, dim3(64), 0, stream,
                     (uint16_t*)a.out, (const uint16_t*)a.query, (const uint8_t*)a.key_cache,
                     (const uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.Hkv,
                     a.MBPS, a.window, a.part_tok, a.NP, qk, vs, a.ws_m, a.ws_l, a.ws_o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.NP <= 1) return e;
  dim3 grid2(a.Hkv * G, a.B);
  hipLaunchKernelGGL((decode_pass2<D, AF>), grid2, dim3(64), 0, stream, (uint16_t*)a.out,
                     a.context_lens, a.Hkv * G, a.window, a.part_tok, a.NP, vs, a.ws_m, a.ws_l,
                     a.ws_o);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_fmt(const DecodeArgs& a, hipStream_t s) {
  if (a.act == FMT_BF16) {
    if (a.cache == FMT_BF16) return launch_typed<D, G, FMT_BF16, FMT_BF16>(a, s);
    if (a.cache == FMT_E4M3) return launch_typed<D, G, FMT_E4M3, FMT_BF16>(a, s);
  } else if (a.act == FMT_F16) {
    if (a.cache == FMT_F16) return launch_typed<D, G, FMT_F16, FMT_F16>(a, s);
    if (a.cache == FMT_E4M3) return launch_typed<D, G, FMT_E4M3, FMT_F16>(a, s);
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
  return cache == act || cache == FMT_E4M3;
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
