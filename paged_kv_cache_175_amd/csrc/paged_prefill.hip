// paged_prefill.hip -- causal chunked prefill over a paged (possibly shared)
// KV cache, on MFMA.
//
// A chunk of C new tokens of a sequence attends causally over everything the
// sequence has cached, its own chunk included: query j sits at absolute
// position ctx - C + j and sees keys 0 .. ctx - C + j.  The keys and values
// are reached through the block table, so prefix blocks shared by several
// sequences are simply the same physical pages in several tables
// ("PagedAttention in mistral.rs": prefix caching works with the paged cache,
// and prefill runs as a separate attention kernel when FlashAttention is on).
//
// Work split.  A workgroup of 4 waves owns 128 consecutive queries of one
// (sequence, query head); each wave owns 32 of them as two 16-row MFMA tiles.
// The workgroup walks the key pages of the sequence (32 tokens each) up to
// the last position its queries can see:
//
//   * the 256 threads copy the page into LDS as K [32][D] and V [D][32] (the
//     cache pages are K [D/8][32][8] and V [D][32], so both copies move
//     16-byte chunks and both MFMA operands become 16-byte LDS reads); rows
//     at or past the context end are zeroed, and E4M3 codes are widened to
//     the activation format (exactly) on the way in;
//   * each wave: S = Q K^T (v_mfma_f32_16x16x32), causal mask, online softmax
//     in log2 units, P rounded to the activation format and passed through
//     LDS into the A-operand layout, O += P V.
// The output is O / l, rounded to the activation format.

#include "common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

constexpr int BS = 32;
constexpr int QT = 128;          // queries per workgroup
constexpr int QW = 32;           // queries per wave
constexpr float LOG2E_P = 1.4426950408889634f;

template <int D, int CF, int AF>
__global__ __launch_bounds__(256) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const int32_t* __restrict__ cu_q_lens, const uint8_t* __restrict__ key_cache,
    const uint8_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int Hq, int Hkv, int MBPS,
    float qk_scale_log2, float v_scale) {
  constexpr int KSTEPS = D / 32;
  constexpr int NT = D / 16;            // 16-wide output column tiles
  constexpr int KROW = D + 8;           // padded LDS row of K (elements)
  constexpr int VROW = BS + 8;          // padded LDS row of transposed V
  constexpr int EB = (CF == FMT_E4M3) ? 1 : 2;
  constexpr int CPR = D / 8;            // 8-element chunks per token row
  typedef typename Mfma<AF>::vec vec;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[BS * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VROW];
  __shared__ __attribute__((aligned(16))) uint16_t p_lds[4][QW * (BS + 8)];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int r4 = lane >> 4;

  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = Hq / Hkv;
  const int g = h / G;

  const int q_begin = cu_q_lens[b];
  const int C = cu_q_lens[b + 1] - q_begin;
  if (tile * QT >= C) return;
  const int ctx = context_lens[b];
  const int first_pos = ctx - C;                    // absolute position of query 0
  const int j_wave = tile * QT + wave * QW;         // first query of this wave
  const int j_last_wg = min(C, tile * QT + QT) - 1;
  const int last_pos_wg = first_pos + j_last_wg;
  const int npages = last_pos_wg / BS + 1;

  // Q of this wave as A operands: tile mt, row 16mt + col, k chunk r4 + 4j.
  vec qa[2][KSTEPS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int j = j_wave + 16 * mt + col;
    const bool live = j < C;
    const uint16_t* qrow = query + ((size_t)(q_begin + (live ? j : 0)) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * (r4 + 4 * s));
      if (!live) w = u32x4{0u, 0u, 0u, 0u};
      qa[mt][s] = __builtin_bit_cast(vec, w);
    }
  }

  float m_run[2][4], l_run[2][4];
  f32x4 o_acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_run[mt][r] = -INFINITY;
      l_run[mt][r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) o_acc[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Absolute positions of the rows this lane holds in the S/O layout.
  int row_pos[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) row_pos[mt][r] = first_pos + j_wave + 16 * mt + 4 * r4 + r;
  const int wave_last_pos = first_pos + min(C - 1, j_wave + QW - 1);
  const bool wave_live = j_wave < C;

  const int32_t* bt = block_tables + (size_t)b * MBPS;
  uint16_t* pw = p_lds[wave];

  for (int pg = 0; pg < npages; ++pg) {
    const int phys = bt[pg];
    const size_t page_off = ((size_t)phys * Hkv + g) * (size_t)BS * D;
    const int base = pg * BS;

    // Stage K (row-major [32][D]) and V (transposed [D][32]) of the page in
    // LDS.  Cache pages are K [D/8][32][8] and V [D][32], so both copies are
    // 8-element chunks.  Rows at or past the context end are zeroed.
    for (int c = tid; c < BS * CPR; c += 256) {
      // K chunk: token t, dims 8*dc .. 8*dc + 7.
      const int t = c % BS;
      const int dc = c / BS;
      u32x4 kw = u32x4{0u, 0u, 0u, 0u};
      if (base + t < ctx) {
        const size_t src = (page_off + (size_t)(dc * BS + t) * 8) * EB;
        if constexpr (CF == FMT_E4M3) {
          kw = e4m3x8_to_16<AF>(*reinterpret_cast<const u32x2*>(key_cache + src));
        } else {
          kw = *reinterpret_cast<const u32x4*>(key_cache + src);
        }
      }
      *reinterpret_cast<u32x4*>(&k_lds[t * KROW + 8 * dc]) = kw;
      // V chunk: dim d, tokens 8*tq .. 8*tq + 7.
      const int d = c / 4;
      const int tq = c % 4;
      const size_t vsrc = (page_off + (size_t)d * BS + 8 * tq) * EB;
      u32x4 vw;
      if constexpr (CF == FMT_E4M3) {
        vw = e4m3x8_to_16<AF>(*reinterpret_cast<const u32x2*>(value_cache + vsrc));
      } else {
        vw = *reinterpret_cast<const u32x4*>(value_cache + vsrc);
      }
      const int tok = base + 8 * tq;
      if (tok + 8 > ctx) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (tok + 2 * e < ctx) ? 0xffffu : 0u;
          const uint32_t hi = (tok + 2 * e + 1 < ctx) ? 0xffff0000u : 0u;
          vw[e] &= (lo | hi);
        }
      }
      *reinterpret_cast<u32x4*>(&v_lds[d * VROW + 8 * tq]) = vw;
    }
    __syncthreads();

    if (wave_live && base <= wave_last_pos) {
      // S = Q K^T for the two 16-token tiles of the page.
      f32x4 s_acc[2][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        vec kb[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          kb[s] = *reinterpret_cast<const vec*>(&k_lds[(16 * tt + col) * KROW + 8 * (r4 + 4 * s)]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          s_acc[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s)
            s_acc[mt][tt] = Mfma<AF>::mma(qa[mt][s], kb[s], s_acc[mt][tt]);
        }
      }

      // Causal mask + online softmax; lane holds rows (mt, 4*r4 + r), token col (+16).
      float alpha[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lim = min(row_pos[mt][r], ctx - 1);
          float s0 = s_acc[mt][0][r] * qk_scale_log2;
          float s1 = s_acc[mt][1][r] * qk_scale_log2;
          if (base + col > lim) s0 = -INFINITY;
          if (base + col + 16 > lim) s1 = -INFINITY;
          const float pm = row16_max(fmaxf(s0, s1));
          const float m_new = fmaxf(m_run[mt][r], pm);
          // m_new is finite: key 0 is visible to every query.
          alpha[mt][r] = fast_exp2(m_run[mt][r] - m_new);
          const float e0 = fast_exp2(s0 - m_new);
          const float e1 = fast_exp2(s1 - m_new);
          l_run[mt][r] = l_run[mt][r] * alpha[mt][r] + row16_sum(e0 + e1);
          m_run[mt][r] = m_new;
          const int q = 16 * mt + 4 * r4 + r;
          pw[q * (BS + 8) + col] = (uint16_t)f32_to_16<AF>(e0);
          pw[q * (BS + 8) + col + 16] = (uint16_t)f32_to_16<AF>(e1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

      // O = alpha * O + P V.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) o_acc[mt][n][r] *= alpha[mt][r];
        const vec pa = *reinterpret_cast<const vec*>(&pw[(16 * mt + col) * (BS + 8) + 8 * r4]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const vec vb = *reinterpret_cast<const vec*>(&v_lds[(16 * n + col) * VROW + 8 * r4]);
          o_acc[mt][n] = Mfma<AF>::mma(pa, vb, o_acc[mt][n]);
        }
      }
    }
    __syncthreads();
  }

  if (!wave_live) return;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j_wave + 16 * mt + 4 * r4 + r;
      if (j >= C) continue;
      const float inv = v_scale / l_run[mt][r];
      uint16_t* dst = out + ((size_t)(q_begin + j) * Hq + h) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) dst[16 * n + col] = (uint16_t)f32_to_16<AF>(o_acc[mt][n][r] * inv);
    }
  }
}

template <int D, int CF, int AF>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const float qk = a.softmax_scale * (CF == FMT_E4M3 ? a.k_scale : 1.f) * LOG2E_P;
  const float vs = CF == FMT_E4M3 ? a.v_scale : 1.f;
  dim3 grid((a.max_chunk + QT - 1) / QT, a.Hq, a.B);
  hipLaunchKernelGGL((prefill_kernel<D, CF, AF>), grid, dim3(256), 0, s, (uint16_t*)a.out,
                     (const uint16_t*)a.query, a.cu_q_lens, (const uint8_t*)a.key_cache,
                     (const uint8_t*)a.value_cache, a.block_tables, a.context_lens, a.Hq,
                     a.Hkv, a.MBPS, qk, vs);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  if (a.act == FMT_BF16) {
    if (a.cache == FMT_BF16) return launch_t<D, FMT_BF16, FMT_BF16>(a, s);
    if (a.cache == FMT_E4M3) return launch_t<D, FMT_E4M3, FMT_BF16>(a, s);
  } else if (a.act == FMT_F16) {
    if (a.cache == FMT_F16) return launch_t<D, FMT_F16, FMT_F16>(a, s);
    if (a.cache == FMT_E4M3) return launch_t<D, FMT_E4M3, FMT_F16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int D, int G, int act, int cache) {
  if (D != 64 && D != 96 && D != 128) return false;
  if (G < 1 || G > 16) return false;
  if (act != FMT_BF16 && act != FMT_F16) return false;
  return cache == act || cache == FMT_E4M3;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.max_chunk <= 0) return hipSuccess;
  switch (a.D) {
    case 64: return launch_d<64>(a, s);
    case 96: return launch_d<96>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
