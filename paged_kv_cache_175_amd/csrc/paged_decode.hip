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
// the current one.  Per wave and page:
//
//   * S = Q K^T: the G query heads of the group are the rows of 16x16x32
//     MFMA tiles (rows G..15 are zero), the page's 32 tokens two 16-column
//     tiles, D/32 k-steps.  The K page layout [D/8][32][8] makes every B
//     operand one 16-byte load (one 16-byte load covers two tokens for E4M3).
//   * Online softmax in log2 units (scale * log2 e folded in): each MFMA
//     output row is one head, so the per-head page max and sum are 16-lane
//     row reductions done entirely in DPP; the reference max moves lazily.
//   * P goes through 1 KiB of the wave's LDS into the MFMA A-operand layout,
//     and O += P V runs as D/16 MFMAs whose B operands are single loads from
//     the transposed V page [D][32].
//
// Append mode (pa_decode_append) also stores the decoded token's K/V into its
// cache row in the same launch; the wave reading that row takes it from LDS.
//
// The W partial results of a workgroup are combined through LDS.  When a
// sequence is one split (S == 1, the usual case once B * Hkv workgroups fill
// the GPU) that is the output; otherwise each split writes (m, l, o) to the
// workspace and a merge kernel combines the S splits: M = max m_s,
// w_s = 2^(m_s - M), out = sum w_s o_s / sum w_s l_s.

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

template <int D, int G, int CF, int AF, int W>
__global__ __launch_bounds__(64 * W) void decode_split(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    uint8_t* __restrict__ key_cache, uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int Hkv, int MBPS, int window, int S, float qk_scale_log2, float v_scale,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    const uint16_t* __restrict__ new_key, const uint16_t* __restrict__ new_value,
    float k_enc_scale, float v_enc_scale) {
  static_assert(D % 32 == 0 && D >= 32 && D <= 256, "head_dim");
  static_assert(G >= 1 && G <= 16, "group");
  constexpr int EB = (CF == FMT_E4M3) ? 1 : 2;
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;
  typedef typename Mfma<AF>::vec vec;

  __shared__ __attribute__((aligned(16))) uint16_t p_lds_all[W][16 * PROW];
  __shared__ float m_lds[W][G];
  __shared__ float l_lds[W][G];
  __shared__ __attribute__((aligned(16))) float o_lds[W][G][D];
  __shared__ __attribute__((aligned(16))) uint16_t newk_lds[D];
  __shared__ __attribute__((aligned(16))) uint16_t newv_lds[D];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int r4 = lane >> 4;
  uint16_t* p_lds = p_lds_all[wave];

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
  // is FP8) and stages the stored values in LDS; the one wave that reads the
  // page patches the row into its MFMA operands, so nothing in this launch
  // depends on the store becoming visible.
  int row_new = -1, k_new = -1, w_new = -1;
  if (new_key != nullptr) {
    const int ctx = context_lens[b];
    const int r_new = window > 0 ? (ctx - 1) % window : ctx - 1;
    const int pg_new = r_new / kPage;
    if (pg_new >= pa && pg_new < pb) {
      row_new = r_new - pg_new * kPage;
      w_new = (pg_new - pa) % W;
      k_new = (pg_new - pa) / W;
      const int phys = block_tables[(size_t)b * MBPS + pg_new];
      const size_t page = ((size_t)phys * Hkv + g) * (size_t)kPage * D;
      const size_t src = ((size_t)b * Hkv + g) * D;
      for (int d = threadIdx.x; d < D; d += 64 * W) {
        const uint16_t kx = new_key[src + d];
        const uint16_t vx = new_value[src + d];
        if constexpr (CF == FMT_E4M3) {
          const uint32_t kq = e4m3_encode(lo16_to_f32<AF>(kx), k_enc_scale);
          const uint32_t vq = e4m3_encode(lo16_to_f32<AF>(vx), v_enc_scale);
          key_cache[page + k_page_off(row_new, d)] = static_cast<uint8_t>(kq);
          value_cache[page + v_page_off(row_new, d)] = static_cast<uint8_t>(vq);
          newk_lds[d] = static_cast<uint16_t>(e4m3x2_to_16<AF, false>(kq) & 0xffffu);
          newv_lds[d] = static_cast<uint16_t>(e4m3x2_to_16<AF, false>(vq) & 0xffffu);
        } else {
          reinterpret_cast<uint16_t*>(key_cache)[page + k_page_off(row_new, d)] = kx;
          reinterpret_cast<uint16_t*>(value_cache)[page + v_page_off(row_new, d)] = vx;
          newk_lds[d] = kx;
          newv_lds[d] = vx;
        }
      }
    }
  }
  __syncthreads();

  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (npg > 0) {
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
    // Physical blocks of this wave's pages, lane k holding its k-th page, so
    // the page loop never waits on a block-table load.
    const int bt_lane = bt[pa + wave + W * (lane < npg ? lane : 0)];

    // Per-lane byte offsets inside a page (loop invariant).  K operand of
    // k-step j, token tile tt: chunk (r4 + 4j), token tile_token(tt, col); V
    // operand of output tile n: dim 16n + col, tokens 8 r4 .. 8 r4 + 7.
    const int k_lane = ((r4 * kPage + tile_token<CF>(0, col)) * 8) * EB;
    const int v_lane = (col * kPage + 8 * r4) * EB;
    constexpr int K_J = 4 * kPage * 8 * EB;    // byte step between k-steps
    constexpr int K_TT = 16 * 8 * EB;          // byte step between token tiles (16-bit)
    constexpr int V_N = 16 * kPage * EB;       // byte step between output tiles
    constexpr uint32_t PAGE_BYTES = (uint32_t)kPage * D * EB;

    auto load_page = [&](int k, PageRegs<D, CF>& Pg) {
      const int phys = __builtin_amdgcn_readlane(bt_lane, k);
      const size_t base = ((size_t)phys * Hkv + g) * page_elems * EB;
      const __amdgpu_buffer_rsrc_t kr = make_rsrc(key_cache + base, PAGE_BYTES);
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(value_cache + base, PAGE_BYTES);
      if constexpr (CF == FMT_E4M3) {
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) Pg.k[j] = buf_load16(kr, k_lane, j * K_J);
      } else {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < KSTEPS; ++j) Pg.k[tt][j] = load8<CF>(kr, k_lane, j * K_J + tt * K_TT);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) Pg.v[n] = load8<CF>(vr, v_lane, n * V_N);
    };

    // K operand of token tile tt, k-step j.
    auto k_operand = [&](const PageRegs<D, CF>& Pg, int tt, int j) -> vec {
      if constexpr (CF == FMT_E4M3) {
        Raw8<CF> r;
        r.w = tt == 0 ? u32x2{Pg.k[j][0], Pg.k[j][1]} : u32x2{Pg.k[j][2], Pg.k[j][3]};
        return as_operand<CF, AF>(r);
      } else {
        return as_operand<CF, AF>(Pg.k[tt][j]);
      }
    };

    auto compute_page = [&](const PageRegs<D, CF>& Pg, int k) {
      // Is this the page holding the appended row?  (Wave-uniform.)
      const bool patch = wave == w_new && k == k_new;
      // S = Q K^T; lane (r4, col) gets heads 4*r4 + r, tokens tok0 and tok1.
      f32x4 sc4[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sc4[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) {
          vec kop = k_operand(Pg, tt, j);
          if (patch && tile_token<CF>(tt, col) == row_new)
            kop = *reinterpret_cast<const vec*>(&newk_lds[8 * (r4 + 4 * j)]);
          sc4[tt] = Mfma<AF>::mma(qa[j], kop, sc4[tt]);
        }
      }
      const int base = (pa + wave + W * k) * kPage;
      const int tok0 = tile_token<CF>(0, col);
      const int tok1 = tile_token<CF>(1, col);
      const bool live0 = base + tok0 < L;
      const bool live1 = base + tok1 < L;
      float sc[4][2], pm[4];
      bool grow = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r][0] = live0 ? sc4[0][r] * qk_scale_log2 : -INFINITY;
        sc[r][1] = live1 ? sc4[1][r] * qk_scale_log2 : -INFINITY;
        pm[r] = row16_max(fmaxf(sc[r][0], sc[r][1]));
        grow |= pm[r] > m_run[r] + kRescaleSlack;
      }
      // The running reference max only moves when some row's page max
      // exceeds it by more than kRescaleSlack (log2 units); otherwise
      // probabilities are taken against the old reference (they stay below
      // 2^kRescaleSlack) and the output needs no rescaling.  The test is
      // wave-uniform.
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
      // Only this wave touches its P buffer: a wave-local ordering point.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // A operand: P[head col][tokens 8*r4 .. 8*r4 + 7].
      const vec pa_op = *reinterpret_cast<const vec*>(&p_lds[col * PROW + 8 * r4]);
      // Rows past the context end may hold anything (NaN included); their
      // probabilities are 0, but 0 * NaN is NaN, so those V values are
      // zeroed on the (uniform) last partial page.
      const bool partial = base + kPage > L;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        vec vb = as_operand<CF, AF>(Pg.v[n]);
        if (partial) {
          u32x4 w = __builtin_bit_cast(u32x4, vb);
          const int tok = base + 8 * r4;  // this lane holds tokens tok .. tok + 7
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (tok + 2 * e < L) ? 0xffffu : 0u;
            const uint32_t hi = (tok + 2 * e + 1 < L) ? 0xffff0000u : 0u;
            w[e] &= (lo | hi);
          }
          vb = __builtin_bit_cast(vec, w);
        }
        if (patch && r4 == (row_new >> 3)) {
          // Element row_new % 8 of this lane's 8 tokens is the appended row.
          u32x4 w = __builtin_bit_cast(u32x4, vb);
          const uint32_t x = newv_lds[16 * n + col];
          const int e = row_new & 7;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q == (e >> 1))
              w[q] = (e & 1) ? ((w[q] & 0xffffu) | (x << 16)) : ((w[q] & 0xffff0000u) | x);
          }
          vb = __builtin_bit_cast(vec, w);
        }
        acc[n] = Mfma<AF>::mma(pa_op, vb, acc[n]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // Two register buffers: page k is computed while page k + 1 loads.  The
    // prefetch past the last page re-reads the last page (an L2 hit) so that
    // no load sits behind a branch.
    PageRegs<D, CF> A, Bf;
    load_page(0, A);
    for (int k = 0;;) {
      load_page(min(k + 1, npg - 1), Bf);
      compute_page(A, k);
      if (++k >= npg) break;
      load_page(min(k + 1, npg - 1), A);
      compute_page(Bf, k);
      if (++k >= npg) break;
    }
  }

  // Combine the W waves through LDS.  Lane (r4, col) holds O[head 4*r4 + r]
  // [dim 16n + col]; waves without pages contribute (-inf, 0, 0).
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * r4 + r;
    if (h < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n) o_lds[wave][h][16 * n + col] = acc[n][r];
      if (col == 0) {
        m_lds[wave][h] = m_run[r];
        l_lds[wave][h] = l_run[r];
      }
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
      ws_o[row * D + d] = num;
      if (d == 0) {
        ws_m[row] = M;
        ws_l[row] = den;
      }
    }
  }
}

// Merge the S split partials of one (sequence, query head): one wave.
// Partials are taken 16 at a time with every load of a group issued before
// any use, so a group costs one memory round trip; the running max is
// rescaled between groups.  Empty splits carry m = -inf and weigh nothing.
constexpr int kMergeGroup = 16;

template <int D, int AF>
__global__ __launch_bounds__(64) void decode_merge(
    uint16_t* __restrict__ out, const int32_t* __restrict__ context_lens, int Hq, int window,
    int S, float v_scale, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o) {
  constexpr int DPT = (D + 63) / 64;  // dims per lane
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = context_lens[b];
  if (window > 0) L = min(L, window);
  if (L <= 0) return;  // zeros written by the split kernel
  const size_t row = ((size_t)b * Hq + h) * S;
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
      mp[i] = ws_m[r];
      lp[i] = ws_l[r];
#pragma unroll
      for (int k = 0; k < DPT; ++k) op[i][k] = ws_o[r * D + dk[k]];
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
  dim3 grid(a.S, a.Hkv, a.B);
  if (a.W == 8) {
    hipLaunchKernelGGL((decode_split<D, G, CF, AF, 8>), grid, dim3(512), 0, stream,
                       (uint16_t*)a.out, (const uint16_t*)a.query, (uint8_t*)a.key_cache,
                       (uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.Hkv,
                       a.MBPS, a.window, a.S, qk, vs, a.ws_m, a.ws_l, a.ws_o,
                       (const uint16_t*)a.new_key, (const uint16_t*)a.new_value, a.k_scale,
                       a.v_scale);
  } else if (a.W == 4) {
    hipLaunchKernelGGL((decode_split<D, G, CF, AF, 4>), grid, dim3(256), 0, stream,
                       (uint16_t*)a.out, (const uint16_t*)a.query, (uint8_t*)a.key_cache,
                       (uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.Hkv,
                       a.MBPS, a.window, a.S, qk, vs, a.ws_m, a.ws_l, a.ws_o,
                       (const uint16_t*)a.new_key, (const uint16_t*)a.new_value, a.k_scale,
                       a.v_scale);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S <= 1) return e;
  dim3 grid2(a.Hkv * G, a.B);
  hipLaunchKernelGGL((decode_merge<D, AF>), grid2, dim3(64), 0, stream, (uint16_t*)a.out,
                     a.context_lens, a.Hkv * G, a.window, a.S, vs, a.ws_m, a.ws_l, a.ws_o);
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
