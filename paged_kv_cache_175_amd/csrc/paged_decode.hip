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
// Work split.  One 64-lane wave owns (sequence b, KV head g, partition p),
// where a partition is `part_tok` consecutive tokens (a multiple of the
// 32-token page).  The wave streams its pages one at a time:
//
//   * S = Q_g K^T on MFMA (v_mfma_f32_16x16x32, bf16 or f16): the G query
//     heads of the group are the 16-row A operand (zero rows pad G up to 16),
//     the page's 32 tokens are two 16-column B tiles.  K is loaded straight
//     into the B-operand layout: lane i reads token (i%16 [+16]) and the
//     8-element chunk (i/16 + 4j) of the head dimension.
//   * Online softmax on the 16x32 score tile: each lane of row 0 holds the
//     scores of one token column for four heads, so the per-head page max and
//     sum are 16-lane row reductions.  Scores are kept in log2 units
//     (scale * log2(e) folded in) so exp is a single v_exp_f32.
//   * O += P V on the vector ALU: V is read fully coalesced (lane i reads
//     8 elements of token i/(D/8) + (64/(D/8))*s), the probabilities travel
//     through 32*G floats of LDS, and each lane keeps G x 8 fp32 partial
//     outputs for its chunk of the head dimension.
//
// A partition either writes the normalised output (when it is the only one
// of its sequence) or its unnormalised (m, l, o) to the workspace; a second
// kernel merges partitions: M = max m_p, w_p = 2^(m_p - M),
// out = sum w_p o_p / sum w_p l_p.

#include "common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr int BS = 32;          // tokens per page
constexpr float LOG2E = 1.4426950408889634f;

template <int CF>
struct CacheElem {
  static constexpr int bytes = 2;
};
template <>
struct CacheElem<FMT_E4M3> {
  static constexpr int bytes = 1;
};

// The 8 cache elements a lane needs, as raw words: 4 words for 16-bit
// formats, 2 words for E4M3.
template <int CF>
struct Raw8 {
  u32x4 w;
};
template <>
struct Raw8<FMT_E4M3> {
  u32x2 w;
};

template <int CF>
__device__ __forceinline__ Raw8<CF> load8(const uint8_t* p) {
  Raw8<CF> r;
  if constexpr (CF == FMT_E4M3) {
    r.w = *reinterpret_cast<const u32x2*>(p);
  } else {
    r.w = *reinterpret_cast<const u32x4*>(p);
  }
  return r;
}

// Widen 8 cache elements to fp32.
template <int CF>
__device__ __forceinline__ void widen8(const Raw8<CF>& r, float (&x)[8]) {
  if constexpr (CF == FMT_E4M3) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      f32x2 a = e4m3x2_to_f32<false>(r.w[w]);
      f32x2 b = e4m3x2_to_f32<true>(r.w[w]);
      x[4 * w + 0] = a[0];
      x[4 * w + 1] = a[1];
      x[4 * w + 2] = b[0];
      x[4 * w + 3] = b[1];
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w + 0] = lo16_to_f32<CF>(r.w[w]);
      x[2 * w + 1] = hi16_to_f32<CF>(r.w[w]);
    }
  }
}

// MFMA operand type for an activation format.
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

// 8 cache elements as an MFMA operand in the activation format.  For a
// 16-bit cache the bits are used as they are; E4M3 values are exact in both
// bf16 and fp16, so the widened fp32 values convert without rounding.
template <int CF, int AF>
__device__ __forceinline__ typename Mfma<AF>::vec as_operand(const Raw8<CF>& r) {
  u32x4 w;
  if constexpr (CF == FMT_E4M3) {
    float x[8];
    widen8<CF>(r, x);
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pack2<AF>(x[2 * k], x[2 * k + 1]);
  } else {
    w = r.w;
  }
  return __builtin_bit_cast(typename Mfma<AF>::vec, w);
}

template <int D, int G, int CF, int AF>
__global__ __launch_bounds__(64) void decode_pass1(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    int Hkv, int MBPS, int window, int part_tok, int NP, float qk_scale_log2,
    float v_scale, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o) {
  static_assert(D % 32 == 0 && (D == 64 || D == 128), "head_dim");
  static_assert(G >= 1 && G <= 8, "group");
  constexpr int EB = CacheElem<CF>::bytes;
  constexpr int KSTEPS = D / 32;        // MFMA k-steps per token tile
  constexpr int CPR = D / 8;            // 8-element chunks per token row
  constexpr int TPI = 64 / CPR;         // tokens per V load instruction
  constexpr int VLOADS = BS / TPI;      // V load instructions per page
  constexpr int HROWS = (G + 3) / 4;    // MFMA output rows of 16 lanes holding heads
  typedef typename Mfma<AF>::vec vec;

  __shared__ float p_lds[BS * G];

  const int lane = threadIdx.x;
  const int col = lane & 15;            // MFMA: token column / A row (head)
  const int r4 = lane >> 4;             // MFMA: k-group / output row group
  const int vc = lane % CPR;            // V chunk owned by this lane
  const int vq = lane / CPR;            // V token sub-index

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
      for (int h = 0; h < G; ++h) {
        uint16_t* o = out + ((size_t)b * Hq + g * G + h) * D;
        for (int d = lane; d < D; d += 64) o[d] = 0;
      }
    }
    return;
  }
  if (p >= nparts) return;

  const int t0 = p * part_tok;
  const int t1 = min(L, t0 + part_tok);
  const int pg0 = t0 / BS;
  const int pg1 = (t1 + BS - 1) / BS;

  // Q as the MFMA A operand: row = head (col < G), k chunk (r4 + 4j).
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

  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  const size_t page_elems = (size_t)BS * D;
  const int32_t* bt = block_tables + (size_t)b * MBPS;

  for (int pg = pg0; pg < pg1; ++pg) {
    const int phys = bt[pg];
    const size_t page_off = ((size_t)phys * Hkv + g) * page_elems;
    const uint8_t* kp = key_cache + page_off * EB;
    const uint8_t* vp = value_cache + page_off * EB;

    // Issue every load of the page up front.
    Raw8<CF> kr[2][KSTEPS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        kr[tt][j] = load8<CF>(kp + ((size_t)(col + 16 * tt) * D + 8 * (r4 + 4 * j)) * EB);
    Raw8<CF> vr[VLOADS];
#pragma unroll
    for (int s = 0; s < VLOADS; ++s)
      vr[s] = load8<CF>(vp + ((size_t)(vq + TPI * s) * D + 8 * vc) * EB);

    // S = Q K^T for tokens [16tt, 16tt+16) of the page.
    f32x4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KSTEPS; ++j)
        sacc[tt] = Mfma<AF>::mma(qa[j], as_operand<CF, AF>(kr[tt][j]), sacc[tt]);
    }

    // Online softmax.  Lane (r4, col) holds heads 4*r4 + r for token col (+16).
    const int base = pg * BS;
    float alpha[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s0 = sacc[0][r] * qk_scale_log2;
      float s1 = sacc[1][r] * qk_scale_log2;
      if (base + col >= t1) s0 = -INFINITY;
      if (base + col + 16 >= t1) s1 = -INFINITY;
      const float pm = row16_max(fmaxf(s0, s1));
      const float m_new = fmaxf(m_run[r], pm);
      alpha[r] = fast_exp2(m_run[r] - m_new);
      const float e0 = fast_exp2(s0 - m_new);
      const float e1 = fast_exp2(s1 - m_new);
      l_run[r] = l_run[r] * alpha[r] + row16_sum(e0 + e1);
      m_run[r] = m_new;
      const int h = 4 * r4 + r;
      if (r4 < HROWS && h < G) {
        p_lds[col * G + h] = e0;
        p_lds[(col + 16) * G + h] = e1;
      }
    }
    __syncthreads();

    // Rescale the running output, then accumulate P V.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[h & 3]), 16 * (h >> 2)));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= a;
    }
    // Rows past the end of the context may hold anything (NaN included):
    // their probabilities are 0, but 0 * NaN is NaN, so their values are
    // zeroed on the (uniform) last, partial page.
    const bool partial_page = base + BS > t1;
#pragma unroll
    for (int s = 0; s < VLOADS; ++s) {
      float x[8];
      widen8<CF>(vr[s], x);
      const int tok = vq + TPI * s;
      if (partial_page && base + tok >= t1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = p_lds[tok * G + h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], x[e], acc[h][e]);
    }
    __syncthreads();
  }

  // Sum the partial outputs of the lanes that share a chunk.
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, 64);

  // Per-head running max / sum, uniform across the wave.
  float mh[G], lh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mh[h] = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_run[h & 3]), 16 * (h >> 2)));
    lh[h] = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_run[h & 3]), 16 * (h >> 2)));
  }

  // Lane (vq, vc) writes heads h = vq, vq + TPI, ... of chunk vc.
  if (nparts == 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if ((h % TPI) != vq) continue;
      const float inv = v_scale / lh[h];
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = pack2<AF>(acc[h][2 * k] * inv, acc[h][2 * k + 1] * inv);
      *reinterpret_cast<u32x4*>(out + ((size_t)b * Hq + g * G + h) * D + 8 * vc) = w;
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if ((h % TPI) != vq) continue;
      const size_t row = ((size_t)b * Hq + g * G + h) * NP + p;
      f32x4* o = reinterpret_cast<f32x4*>(ws_o + row * D + 8 * vc);
      o[0] = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      o[1] = f32x4{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
      if (vc == 0) {
        ws_m[row] = mh[h];
        ws_l[row] = lh[h];
      }
    }
  }
}

// Merge the partitions of each (sequence, query head).
template <int D, int AF>
__global__ __launch_bounds__(64) void decode_pass2(
    uint16_t* __restrict__ out, const int32_t* __restrict__ context_lens, int Hq, int window,
    int part_tok, int NP, float v_scale, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const float* __restrict__ ws_o) {
  constexpr int DPT = D / 64;  // dims per lane
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int L = context_lens[b];
  if (window > 0) L = min(L, window);
  const int nparts = (L + part_tok - 1) / part_tok;
  if (nparts <= 1) return;  // written by pass 1
  const size_t row = ((size_t)b * Hq + h) * NP;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ws_m[row + p]);
  float num[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) num[k] = 0.f;
  float den = 0.f;
  const int d0 = threadIdx.x * DPT;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(ws_m[row + p] - M);
    den = fmaf(w, ws_l[row + p], den);
    const float* o = ws_o + (row + p) * D + d0;
#pragma unroll
    for (int k = 0; k < DPT; ++k) num[k] = fmaf(w, o[k], num[k]);
  }
  const float inv = v_scale / den;
  uint16_t* dst = out + ((size_t)b * Hq + h) * D + d0;
#pragma unroll
  for (int k = 0; k < DPT; ++k) dst[k] = static_cast<uint16_t>(f32_to_16<AF>(num[k] * inv));
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_supported(int D, int G, int act, int cache) {
  if (D != 64 && D != 128) return false;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (act != FMT_BF16 && act != FMT_F16) return false;
  return cache == act || cache == FMT_E4M3;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_group<64>(a, s);
    case 128: return launch_group<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
