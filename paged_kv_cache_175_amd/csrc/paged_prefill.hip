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
// Work split.  The query rows of one (sequence, KV head) are the pairs
// (position j, head h in the KV head's group), numbered row = j * G + h, so a
// staged K/V page serves all G query heads that read it.  A workgroup of 8
// waves (two per SIMD) owns 128 * NQ consecutive rows; each wave owns NQ
// tiles of 16 rows.
// The workgroup walks the sequence's key pages (32 tokens each) up to the last
// position its rows can see.  Pages of a 16-bit cache go from global memory
// straight into LDS (global_load_lds_dwordx4, no registers) two at a time:
// four LDS page buffers hold the pair being computed and the next pair in
// flight, with one barrier per pair.  E4M3 and INT8 pages are widened to the
// activation format on the way, so they pass through registers, one page
// ahead, through two buffers.  An INT8 page ("libmir-metal 0.2.0,
// src/native/trace/kv.rs", fn build: per-token/head codes with fp32 scales)
// also stages its 32 K and 32 V row scales; the K scales multiply the scores
// and the V scales the P of the V MFMAs (the running sum takes the unscaled
// P).
//
// Per wave and page, everything is computed transposed so that the
// probabilities never leave registers:
//   S^T = K Q^T   (v_mfma_f32_16x16x32; K from LDS as the A operand, Q held
//                  in registers as the B operand).  The two 16-key A tiles of
//                  a page take the keys with bit 2 clear and set: tile kt row
//                  x is key 8 * (x / 4) + 4 * kt + x % 4.  Lane l then holds,
//                  for query column l % 16, the eight consecutive keys
//                  8 * (l / 16) .. 8 * (l / 16) + 7;
//   P^T = exp2(S^T * c - m), rounded to the activation format: those eight
//                  values per lane are exactly a B operand over the page's
//                  keys in natural order;
//   O^T += V^T P^T (A operand = V^T: eight consecutive tokens of one head
//                  dimension, one 16-byte LDS read).
// LDS pages hold K as [D/8][32] chunks of 8 elements and V as [D][4] chunks
// (dimension, 8-token group) with the 16-byte chunks of each row
// XOR-swizzled so that both operand reads are free of bank conflicts.
// The running sum l of each query is taken from the same rounded P that
// weights V: each lane adds its eight P values to a per-lane partial sum
// with four two-element dot products against ones (v_dot2c_f32_bf16 or
// _f16, exact products, fp32 sums), rescaled with O; the four lanes that
// hold a query are added up at the end.  The running maximum m is only
// raised when a new score exceeds it by more than 2^8 (any lane, checked
// with a ballot), so the cross-lane maximum and the rescale of O run on a
// few pages only.  Probabilities therefore stay below 2^8, which fp32
// accumulation and the 16-bit P operand both hold without loss of relative
// precision.
//
// Rows at or past the context end in a sequence's last page hold stale data.
// Their scores are always masked (every query sits before the context end),
// and on that page the V operand is zeroed there, so no Inf or NaN reaches
// the accumulators through a zero probability.
//
// Sliding-window layers (WIN): the cache is a ring of W rows, position i in
// row i mod W ("Rolling buffer cache", opening post), and the chunk has not
// been written into it yet, since its later tokens would overwrite rows its
// earlier queries still need.  Query i attends to positions i - W + 1 .. i:
// those before the chunk come from the ring pages, the chunk's own from its
// K/V activations, staged through registers into the same LDS layout, one
// page ahead, two buffers.  A byte ring's page is held in registers as its
// raw codes and widened to the activation format when it is stored to LDS;
// an INT8 ring's rows are staged as their codes times their row scales,
// rounded to the activation format; over an E4M3 ring the tensor scales
// fold into the score and output scales and the chunk's rows are divided
// by them.
//
// Workgroup order: workgroups are dispatched to the 8 XCDs round-robin, so
// the flat workgroup id is remapped to give each XCD a contiguous range of
// (KV head, sequence, row tile) items.  The workgroups that read one KV
// head's shared prefix pages then run on one XCD, close in time, and hit in
// its L2.

#include <cfloat>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

constexpr int BS = 32;
// Eight waves share each staged page: against four (two workgroups per CU),
// half the re-reads of the pages from L2 and half the staging work per wave
// (measured: sliding-window prefill 752 -> 623 us, E4M3 ring 930 -> 830;
// causal shared-prefix prefill unchanged).
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr float LOG2E_P = 1.4426950408889634f;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedTrans = 0x400;
// Scores (in log2 units) may exceed the running maximum by this much before
// the maximum is raised.
constexpr float kSlack = 8.0f;

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, v), mask, 64));
}

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Eight INT8 codes times their scales (s[k] for code k), rounded to the
// activation format.
template <int AF>
__device__ __forceinline__ u32x4 i8x8_scaled(u32x2 c, f32x8 s) {
  f32x8 f;
#pragma unroll
  for (int w = 0; w < 2; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[4 * w + i] = static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(c[w] >> (8 * i))));
  f *= s;
  typedef typename Mfma<AF>::vec v8;
  return __builtin_bit_cast(u32x4, __builtin_convertvector(f, v8));
}

// acc + w.lo + w.hi for two packed values of an activation format: a
// two-element dot product against ones (the products are exact).
template <int AF>
__device__ __forceinline__ float add_pair(uint32_t w, float acc);
template <>
__device__ __forceinline__ float add_pair<FMT_BF16>(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         bf16x2{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}
template <>
__device__ __forceinline__ float add_pair<FMT_F16>(uint32_t w, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
}

// Four 16-bit values of an activation format (hardware conversion, round to
// nearest even).
template <int AF>
struct Vec4;
template <>
struct Vec4<FMT_BF16> {
  typedef __bf16 type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec4<FMT_F16> {
  typedef _Float16 type __attribute__((ext_vector_type(4)));
};

// Eight values of an activation format times m, clamped to +-448 (the E4M3
// range) and rounded back to the format.
template <int AF>
__device__ __forceinline__ u32x4 mul_clamp(u32x4 w, float m) {
  typedef typename Mfma<AF>::vec v8;
  f32x8 f = __builtin_convertvector(__builtin_bit_cast(v8, w), f32x8) * m;
  f = __builtin_elementwise_min(__builtin_elementwise_max(f, (f32x8)(-448.f)), (f32x8)(448.f));
  return __builtin_bit_cast(u32x4, __builtin_convertvector(f, v8));
}

// LDS chunk slots (16-byte chunks, in chunk units within one page).  Both
// maps are involutions on the row index bits they touch, so the same
// functions map a slot back to its cache chunk.
__device__ __forceinline__ int k_slot(int dc, int t) { return dc * BS + (t ^ (((t >> 3) & 1) << 2)); }
__device__ __forceinline__ int v_slot(int d, int tq) { return d * 4 + (tq ^ ((d >> 1) & 3)); }

// Workgroup barrier that does not wait for outstanding global loads (a
// __syncthreads would drain the LDS-direct loads still in flight for later
// pages).  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int CF, int AF, int NQ, bool WIN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
    const int32_t* __restrict__ cu_q_lens, const uint8_t* __restrict__ key_cache,
    const uint8_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int Hq, int Hkv, int G, int B, int MBPS,
    int row_tiles, float qk_scale_log2, float v_scale, const float* __restrict__ key_scales,
    const float* __restrict__ value_scales, const uint16_t* __restrict__ key_act,
    const uint16_t* __restrict__ value_act, int window, float chunk_k_mul,
    float chunk_v_mul) {
  constexpr int KS = D / 32;              // k-steps of S^T (32 head dims each)
  constexpr int NT = D / 16;              // 16-dim tiles of O^T
  constexpr int PAGE = BS * D;            // elements of one K (or V) page
  constexpr bool kDma = !byte_fmt(CF) && !WIN;
  constexpr bool kI8 = CF == FMT_I8;
  // Per-key scales staged beside each page: the INT8 row scales of the
  // causal path.
  constexpr bool kScaled = kI8 && !WIN;
  // Window path over an INT8 ring: each ring row is staged as its codes
  // times its scales, rounded to the activation format.
  constexpr bool kWinI8 = WIN && kI8;
  constexpr bool kWinByte = WIN && byte_fmt(CF);
  // Window path over an E4M3 ring: a ring row on a row-by-row page is
  // staged as raw codes too and widened when stored.
  constexpr bool kWinDefer = WIN && CF == FMT_E4M3;
  // Window path over an E4M3 ring: the ring's tensor scales fold into the
  // score and output scales, and the chunk's own rows are staged divided
  // by them (clamped to the E4M3 range, which holds them whenever the
  // scales cover the chunk, as they must for the ring it is written to).
  constexpr bool kFoldWin = WIN && CF == FMT_E4M3;
  // LDS-direct staging works on pairs of pages: the pair being computed
  // and the next one in flight, four buffers.
  constexpr int NBUF = kDma ? 4 : 2;
  constexpr int EB = kDma ? 2 : 1;        // cache bytes per element
  constexpr int NCH = PAGE / 8;           // 8-element chunks per page (K or V)
  constexpr int RW = 16 * NQ * kWaves;    // rows per workgroup
  // LDS-direct loads: 64 chunks (1 KiB) per wave instruction; the K and V
  // pages together are D / 8 such units, up to UPW per wave (at D = 96 the
  // last two waves have none).
  constexpr int UPW = (D / 8 + kWaves - 1) / kWaves;
  // Register staging (E4M3, INT8): chunks per thread.
  constexpr int ST = (NCH + kThreads - 1) / kThreads;
  typedef typename Mfma<AF>::vec vec;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NBUF][PAGE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NBUF][PAGE];
  __shared__ __attribute__((aligned(16))) float ks_lds[kScaled ? NBUF : 1][BS];  // row scales
  __shared__ __attribute__((aligned(16))) float vs_lds[kScaled ? NBUF : 1][BS];

  // --- which (KV head, sequence, row tile) this workgroup owns -----------
  const int n_items = row_tiles * Hkv * B;
  const int per_xcd = (n_items + kXcds - 1) / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= n_items) return;
  const int x = item % row_tiles;
  const int b = (item / row_tiles) % B;
  const int g = item / (row_tiles * B);

  const int q_begin = cu_q_lens[b];
  const int C = cu_q_lens[b + 1] - q_begin;
  const int rows = C * G;
  if (x * RW >= rows) return;
  // A full cache holds at most MBPS * BS positions (the table row); a length
  // above that is clamped so no table read leaves the row.  The window path
  // indexes its ring modulo the window, inside the row whatever the length.
  const int ctx = WIN ? context_lens[b] : min(context_lens[b], MBPS * BS);
  const int first_pos = ctx - C;               // absolute position of query 0
  const int last_row_wg = min(rows, x * RW + RW) - 1;
  // Key pages [p_lo, p_lo + npages): from the earliest key any row of the
  // workgroup sees (0, or the start of its earliest query's window) to its
  // latest query.
  const int p_lo = WIN ? max(0, first_pos + (x * RW) / G - window + 1) / BS : 0;
  const int npages = (first_pos + last_row_wg / G) / BS + 1 - p_lo;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int q4 = lane >> 4;

  const int row0 = x * RW + wave * 16 * NQ;    // first row of this wave
  const bool wave_live = row0 < rows;
  const int pos_lo = first_pos + row0 / G;                              // earliest query
  const int pos_hi = first_pos + min(rows - 1, row0 + 16 * NQ - 1) / G;  // latest query

  // Q^T operands and the query position of each tile column this lane holds.
  vec qb[NQ][KS];
  int qpos[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int r = row0 + 16 * t + col;
    const bool live = r < rows;
    const int j = live ? r / G : C - 1;
    const int hq = g * G + (live ? r - j * G : 0);
    qpos[t] = first_pos + j;
    const uint16_t* qrow = query + ((size_t)(q_begin + j) * Hq + hq) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * q4);
      if (!live) w = u32x4{0u, 0u, 0u, 0u};
      qb[t][s] = __builtin_bit_cast(vec, w);
    }
  }

  // Per tile: the running maximum m_run, the lane's partial running sum
  // l_acc (its eight keys of each page), and O^T.  The raw scores are tested
  // against a raw threshold: a raw score above m_thr is more than kSlack
  // above m_run once scaled (m_thr = (m_run + kSlack) / scale; the scale is
  // > 0, checked by the host), which saves a multiply and an add per tile
  // and page.
  float m_run[NQ];
  float m_thr[NQ];
  float l_acc[NQ];
  f32x4 o_acc[NT][NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    // A window row can meet pages that lie wholly below its window before
    // its first live key: a finite floor keeps exp2(s - m) at 0 there.
    m_run[t] = WIN ? -1.0e30f : -INFINITY;
    m_thr[t] = -INFINITY;
    l_acc[t] = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o_acc[n][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Operand offsets (elements) inside a staged page.  K: chunk row
  // (4s + q4), key row 8 * (col / 4) + 4 * kt + col % 4.  V: head dim
  // 16n + col, token chunk q4.
  int k_off[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) k_off[kt] = k_slot(q4, 8 * (col >> 2) + 4 * kt + (col & 3)) * 8;
  const int v_off = v_slot(col, q4) * 8;       // + 16 * 4 * 8 * n (the swizzle ignores d / 16)

  // --- page staging ------------------------------------------------------
  // Without a table the map is the identity: logical block j of sequence b
  // is physical block b * MBPS + j.
  const bool ident = block_tables == nullptr;
  const int32_t* bt = block_tables + (size_t)b * MBPS;
  // Physical blocks of pages 0..63 (the window path indexes its ring itself).
  int bt_reg = !WIN && !ident && lane < npages ? bt[lane] : 0;
  const size_t head_off = (size_t)g * PAGE;
  const size_t blk_stride = (size_t)Hkv * PAGE;
  auto phys_of = [&](int q) {
    if (ident) return b * MBPS + q;
    if ((q & 63) == 0 && q > 0) bt_reg = q + lane < npages ? bt[q + lane] : 0;
    return __builtin_amdgcn_readlane(bt_reg, q & 63);
  };

  // LDS-direct path: source byte offset (inside a page) of this lane's chunk
  // in each of the wave's units.
  int dma_src[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int u = min(wave * UPW + i, D / 8 - 1);   // unused past D / 8
    if (u < D / 16) {
      const int s = u * 64 + lane;             // K slot
      dma_src[i] = k_slot(s >> 5, s & 31) * 16;
    } else {
      // V slot s = (d, x) holds the chunk of token group x ^ swizzle(d),
      // which the cache keeps at chunk (group * D + d).
      const int s = (u - D / 16) * 64 + lane;
      const int d = s >> 2;
      const int tq = (s & 3) ^ ((d >> 1) & 3);
      dma_src[i] = (tq * D + d) * 16;
    }
  }
  auto dma_page = [&](int phys, int buf) {
    const size_t page = ((size_t)phys * blk_stride + head_off) * EB;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int u = wave * UPW + i;
      if (u >= D / 8) continue;
      const bool is_k = u < D / 16;
      const uint8_t* src = (is_k ? key_cache : value_cache) + page + dma_src[i];
      uint16_t* dst = is_k ? &k_lds[buf][u * 512] : &v_lds[buf][(u - D / 16) * 512];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0,
                                       0);
    }
  };

  // Register path (E4M3, INT8): chunk c of the K page is (d / 8, t) =
  // (c / 32, c % 32) and chunk c of the V page is (d, t / 8) = (c % D, c / D).
  // Threads 0..31 also carry the page's K row scales, 32..63 its V scales.
  u32x2 kreg[kDma ? 1 : ST], vreg[kDma ? 1 : ST];
  float sreg = 0.f;
  auto load_regs = [&](int phys) {
    const size_t page = ((size_t)phys * blk_stride + head_off) * EB;
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      const int c = tid + i * kThreads;
      if (NCH % kThreads == 0 || c < NCH) {
        kreg[i] = *reinterpret_cast<const u32x2*>(key_cache + page + (size_t)c * 8);
        vreg[i] = *reinterpret_cast<const u32x2*>(value_cache + page + (size_t)c * 8);
      }
    }
    if constexpr (kI8) {
      const size_t srow = ((size_t)phys * Hkv + g) * BS;
      if (tid < BS) sreg = key_scales[srow + tid];
      else if (tid < 2 * BS) sreg = value_scales[srow + tid - BS];
    }
  };
  auto widen = [&](u32x2 c) -> u32x4 {
    if constexpr (kI8) {
      return i8x8_to_16<AF>(c);
    } else {
      return e4m3x8_to_16<AF>(c);
    }
  };
  auto store_regs = [&](int buf, int base) {
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      const int c = tid + i * kThreads;
      if (NCH % kThreads == 0 || c < NCH) {
        *reinterpret_cast<u32x4*>(&k_lds[buf][k_slot(c >> 5, c & 31) * 8]) = widen(kreg[i]);
        *reinterpret_cast<u32x4*>(&v_lds[buf][v_slot(c % D, c / D) * 8]) = widen(vreg[i]);
      }
    }
    if constexpr (kI8) {
      // Stale rows past the context end get scale 0 (their scores are
      // masked anyway; a NaN V scale would survive a zero probability).
      const int row = tid & (BS - 1);
      const float sv = base + row < ctx ? sreg : 0.f;
      if (tid < BS) ks_lds[buf][row] = sv;
      else if (tid < 2 * BS) vs_lds[buf][row] = sv;
    }
  };

  // Window path: item (r, c) = row r, head-dimension chunk c of a page.  A
  // row before the chunk comes from the ring (its ring page holds rows
  // pos mod W; the ring has every position from max(0, start - W) on); a
  // row of the chunk from the activations; any other row is zero (never
  // visible to a query).  A quantised ring's rows are held as raw codes
  // and widened when the page is stored to LDS (E4M3 exactly; INT8 as codes
  // times their row scales, rounded to the activation format), except an
  // INT8 ring's rows on a row-by-row page, which are scaled in registers
  // of their own as they arrive.  Over an E4M3 ring the chunk's rows are
  // divided by the tensor scales when they are stored.
  constexpr int NIT = (BS * (D / 8) + kThreads - 1) / kThreads;
  u32x4 wk[WIN ? NIT : 1], wv[WIN ? NIT : 1];
  // A byte ring's native page: raw codes, widened when stored (and an INT8
  // ring's scales: the K chunk's row, the V chunk's eight rows).
  u32x2 wkc[kWinByte ? NIT : 1], wvc[kWinByte ? NIT : 1];
  float wks[kWinI8 ? NIT : 1];
  f32x4 wvs0[kWinI8 ? NIT : 1], wvs1[kWinI8 ? NIT : 1];
  // Item class: 0 a zero row or a native page, 1 a byte ring's row on a
  // row-by-row page (E4M3: widened when stored; INT8: scaled while staging,
  // held apart from the chunk rows' registers), 2 a chunk row (E4M3 ring:
  // divided when stored).  One variable, so that the branches that set it
  // store values, not flags in different places.  On a row-by-row page the
  // chunk rows' loads then write registers that nothing else writes, and
  // no load is waited for before the page's products (a merge of loaded
  // and computed values into one register waits for the load).
  int wcl[WIN ? NIT : 1];
  // An E4M3 ring's row on a row-by-row page: the K codes in wkc, the V
  // codes one byte per register (gathered from eight V chunks).
  uint32_t wvb[kWinDefer ? NIT : 1][8];
  const uint16_t* vc16 = reinterpret_cast<const uint16_t*>(value_cache);
  // Eight elements of a 16-bit ring's K (or V) starting at element `off`
  // of the cache: one 16-byte load.
  auto ring_chunk = [&](const uint8_t* cache, size_t off) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(cache) + off);
  };
  // A page wholly before the chunk is all ring rows, every one written
  // (the ring holds max(0, start - W) .. start - 1, all W rows once
  // start >= W): it is staged as native page chunks, V included, with no
  // per-row choice.  Other pages go row by row.
  bool win_native = false;
  auto load_win = [&](int base) {
    const int ring_lo = max(0, first_pos - window);
    const int ring_blk = (base % window) / BS;
    const int phys = base >= first_pos ? 0 : ident ? b * MBPS + ring_blk : bt[ring_blk];
    const size_t page = (size_t)phys * blk_stride + head_off;
    win_native = base + BS <= first_pos;
    if (win_native) {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int item = tid + i * kThreads;
        wcl[i] = 0;
        if (item < NCH) {
          if constexpr (kWinByte) {
            wkc[i] = *reinterpret_cast<const u32x2*>(key_cache + page + (size_t)item * 8);
            wvc[i] = *reinterpret_cast<const u32x2*>(value_cache + page + (size_t)item * 8);
            if constexpr (kWinI8) {
              const size_t srow = ((size_t)phys * Hkv + g) * BS;
              wks[i] = key_scales[srow + (item & (BS - 1))];
              const f32x4* vsp = reinterpret_cast<const f32x4*>(value_scales + srow + 8 * (item / D));
              wvs0[i] = vsp[0];
              wvs1[i] = vsp[1];
            }
            // Every staged register is written on both paths, so that no
            // loaded value has to be copied where the paths join.
            wk[i] = u32x4{0u, 0u, 0u, 0u};
            wv[i] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (kWinDefer) {
#pragma unroll
              for (int e = 0; e < 8; ++e) wvb[i][e] = 0u;
            }
          } else {
            wk[i] = ring_chunk(key_cache, page + (size_t)item * 8);
            wv[i] = ring_chunk(value_cache, page + (size_t)item * 8);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int item = tid + i * kThreads;
      u32x4 kw = u32x4{0u, 0u, 0u, 0u}, vw = u32x4{0u, 0u, 0u, 0u};
      wcl[i] = 0;
      if constexpr (kWinByte) {
        wkc[i] = u32x2{0u, 0u};
        wvc[i] = u32x2{0u, 0u};
        if constexpr (kWinDefer) {
#pragma unroll
          for (int e = 0; e < 8; ++e) wvb[i][e] = 0u;
        }
        if constexpr (kWinI8) {
          wks[i] = 0.f;
          wvs0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
          wvs1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (item < NCH) {
        const int r = item & (BS - 1);
        const int c = item / BS;
        const int pos = base + r;
        if (pos >= ring_lo && pos < first_pos) {
          if constexpr (kWinDefer) {
            wkc[i] = *reinterpret_cast<const u32x2*>(key_cache + page + (size_t)(c * BS + r) * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              wvb[i][e] = value_cache[page + ((size_t)(r >> 3) * D + 8 * c + e) * 8 + (r & 7)];
            wcl[i] = 1;
          } else if constexpr (kWinI8) {
            // The INT8 ring row's scaled K and V go into the native page's
            // scale registers (unused on row-by-row pages), not into the
            // registers the chunk rows' loads write.
            const size_t srow = ((size_t)phys * Hkv + g) * BS + r;
            wvs0[i] = __builtin_bit_cast(
                f32x4, i8x8_scaled<AF>(*reinterpret_cast<const u32x2*>(key_cache + page +
                                                                       (size_t)(c * BS + r) * 8),
                                       (f32x8)(key_scales[srow])));
            u32x2 vq = u32x2{0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              vq[e >> 2] |= (uint32_t)value_cache[page + ((size_t)(r >> 3) * D + 8 * c + e) * 8 +
                                                  (r & 7)]
                            << (8 * (e & 3));
            wvs1[i] = __builtin_bit_cast(f32x4, i8x8_scaled<AF>(vq, (f32x8)(value_scales[srow])));
            wcl[i] = 1;
          } else {
            kw = ring_chunk(key_cache, page + (size_t)(c * BS + r) * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const size_t at = page + ((size_t)(r >> 3) * D + 8 * c + 2 * e) * 8 + (r & 7);
              vw[e] = (uint32_t)vc16[at] | ((uint32_t)vc16[at + 8] << 16);
            }
          }
        } else if (pos >= first_pos && pos < ctx) {
          const size_t row = ((size_t)(q_begin + pos - first_pos) * Hkv + g) * D + 8 * c;
          kw = *reinterpret_cast<const u32x4*>(key_act + row);
          vw = *reinterpret_cast<const u32x4*>(value_act + row);
          wcl[i] = 2;
        }
      }
      wk[i] = kw;
      wv[i] = vw;
    }
  };
  // Native: chunk `item` of the K page is (d / 8, t) = (item / 32, item % 32)
  // and of the V page (d, t / 8) = (item % D, item / D).  Row by row: item
  // (t, d / 8) = (item % 32, item / 32) for both, V transposed here.
  auto store_win = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int item = tid + i * kThreads;
      if (item < NCH) {
        const int r = item & (BS - 1);
        const int c = item / BS;
        if constexpr (kFoldWin) {
          if (!win_native && wcl[i] == 2) {
            wk[i] = mul_clamp<AF>(wk[i], chunk_k_mul);
            wv[i] = mul_clamp<AF>(wv[i], chunk_v_mul);
          }
        }
        if constexpr (kWinByte) {
          if (win_native) {
            if constexpr (kWinI8) {
              const f32x4 s0 = wvs0[i], s1 = wvs1[i];
              wk[i] = i8x8_scaled<AF>(wkc[i], (f32x8)(wks[i]));
              wv[i] = i8x8_scaled<AF>(wvc[i], f32x8{s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]});
            } else {
              wk[i] = widen(wkc[i]);
              wv[i] = widen(wvc[i]);
            }
          } else if (kWinI8 && wcl[i] == 1) {
            wk[i] = __builtin_bit_cast(u32x4, wvs0[i]);
            wv[i] = __builtin_bit_cast(u32x4, wvs1[i]);
          } else if (kWinDefer && wcl[i] == 1) {
            u32x2 vq;
#pragma unroll
            for (int h = 0; h < 2; ++h)
              vq[h] = wvb[i][4 * h] | (wvb[i][4 * h + 1] << 8) | (wvb[i][4 * h + 2] << 16) |
                      (wvb[i][4 * h + 3] << 24);
            wk[i] = widen(wkc[i]);
            wv[i] = widen(vq);
          }
        }
        *reinterpret_cast<u32x4*>(&k_lds[buf][k_slot(c, r) * 8]) = wk[i];
        if (win_native) {
          *reinterpret_cast<u32x4*>(&v_lds[buf][v_slot(item % D, item / D) * 8]) = wv[i];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 8 * c + e;
            v_lds[buf][v_slot(d, r >> 3) * 8 + (r & 7)] =
                static_cast<uint16_t>(wv[i][e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  };

  if constexpr (WIN) {
    load_win(p_lo * BS);
    store_win(0);
    __syncthreads();
  } else if constexpr (kDma) {
    // The first pair.
    if (npages > 0) dma_page(phys_of(0), 0);
    if (npages > 1) dma_page(phys_of(1), 1);
    wait_vmcnt<0>();
    lds_barrier();
  } else {
    load_regs(phys_of(0));
    store_regs(0, 0);
    __syncthreads();
  }

  int cur = 0;
  for (int p = 0; p < npages; ++p) {
    const int base = (p_lo + p) * BS;
    if constexpr (WIN) {
      if (p + 1 < npages) load_win(base + BS);
    } else if constexpr (kDma) {
      // Page p sits in buffer p mod 4.  At the first page of a pair the next
      // pair goes into the buffers of the previous pair, which every wave
      // finished before the last barrier.
      cur = p & 3;
      if ((p & 1) == 0) {
        if (p + 2 < npages) dma_page(phys_of(p + 2), (p + 2) & 3);
        if (p + 3 < npages) dma_page(phys_of(p + 3), (p + 3) & 3);
      }
    } else {
      if (p + 1 < npages) load_regs(phys_of(p + 1));
    }

    // A wave computes a page if some key of it lies in some row's window.
    const bool in_window = !WIN || base + BS - 1 >= pos_lo - window + 1;
    if (wave_live && base <= pos_hi && in_window) {
      auto page = [&](auto masked) {
      const uint16_t* kb = k_lds[cur];
      const uint16_t* vb = v_lds[cur];
      // S^T = K Q^T: the two 16-key tiles of the page.
      f32x4 s_acc[2][NQ];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int t = 0; t < NQ; ++t) s_acc[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const vec ka = *reinterpret_cast<const vec*>(&kb[k_off[kt] + s * 4 * BS * 8]);
#pragma unroll
          for (int t = 0; t < NQ; ++t) s_acc[kt][t] = Mfma<AF>::mma(ka, qb[t][s], s_acc[kt][t]);
        }
      }

      // The causal mask and P.  Lane element (kt, r) is key
      // base + 8 * q4 + 4 * kt + r.  The scores stay unscaled: the maxima
      // are scaled once per lane and the softmax scale (in log2 units) goes
      // into the exponent's FMA, which saves a multiply per score.  The mask
      // is needed only where the page reaches past the earliest query of the
      // wave; the two cases are separate instantiations so that the common,
      // unmasked one carries no per-score compares and selects.
      {
        if constexpr (kScaled) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const f32x4 ks4 = *reinterpret_cast<const f32x4*>(&ks_lds[cur][8 * q4 + 4 * kt]);
#pragma unroll
            for (int t = 0; t < NQ; ++t) s_acc[kt][t] *= ks4;
          }
        }
        if constexpr (decltype(masked)::value) {
#pragma unroll
          for (int t = 0; t < NQ; ++t)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int kp = base + 8 * q4 + 4 * kt + r;
                if (kp > qpos[t] || (WIN && kp <= qpos[t] - window)) s_acc[kt][t][r] = -INFINITY;
              }
        }
        // The running maxima.  Raising one is rare (a ballot finds a score
        // more than kSlack above it); it is then raised to the maximum over
        // the four lanes that hold the query (never lowered), and unchanged
        // maxima keep their accumulators as they are.
        // The lane's maxima use the NaN-propagating maximum (gfx950's
        // three-input v_maximum3_f32): fmaxf must quiet signalling NaNs in
        // IEEE mode, which costs a canonicalising max per MFMA result.
        // Scores here are finite or -inf, so both give the same value.  The
        // maxima stay raw until a raise; the test compares them with m_thr.
        float lmax[NQ];
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          const f32x4 a = s_acc[0][t], c = s_acc[1][t];
          const float m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[0], a[1]), a[2]);
          const float m2 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[3], c[0]), c[1]);
          const float m3 = __builtin_elementwise_maximum(c[2], c[3]);
          lmax[t] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m1, m2), m3);
        }
        auto raise_max = [&](int t) {
          const float lm = qk_scale_log2 * lmax[t];
          float cm = fmaxf(lm, shfl_xor_f(lm, 16));
          cm = fmaxf(cm, shfl_xor_f(cm, 32));
          const float m_new = fmaxf(m_run[t], cm);
          const float alpha = m_new == m_run[t] ? 1.f : fast_exp2(m_run[t] - m_new);
#pragma unroll
          for (int n = 0; n < NT; ++n) o_acc[n][t] *= alpha;
          l_acc[t] *= alpha;
          m_run[t] = m_new;
          m_thr[t] = (m_new + kSlack) / qk_scale_log2;
        };
        // One test for all tiles, so that the block after it holds every
        // tile's exponentials and V MFMAs.
        bool raise = false;
#pragma unroll
        for (int t = 0; t < NQ; ++t) raise |= lmax[t] > m_thr[t];
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
          for (int t = 0; t < NQ; ++t) raise_max(t);
        }
      }

      // P and O^T += V^T P^T.  On the sequence's last page, tokens at or past
      // the context end are zeroed in the V operand.
      u32x4 keep = u32x4{~0u, ~0u, ~0u, ~0u};
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tok = base + 8 * q4 + 2 * e;
          keep[e] = (tok < ctx ? 0xffffu : 0u) | (tok + 1 < ctx ? 0xffff0000u : 0u);
        }
      }
      auto v_operand = [&](int n) {
        u32x4 vw = *reinterpret_cast<const u32x4*>(&vb[v_off + n * 16 * 4 * 8]);
        if constexpr (decltype(masked)::value) vw &= keep;
        return __builtin_bit_cast(vec, vw);
      };
      // P of tile t (and, beside the unscaled P, the P that weights V when
      // the keys carry V scales); the lane's partial l adds the unscaled P.
      auto p_operand = [&](int t) -> vec {
        f32x8 pv;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            pv[4 * kt + r] = fast_exp2(fmaf(s_acc[kt][t][r], qk_scale_log2, -m_run[t]));
        vec pb = __builtin_convertvector(pv, vec);
        const u32x4 pw = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int e = 0; e < 4; ++e) l_acc[t] = add_pair<AF>(pw[e], l_acc[t]);
        if constexpr (kScaled) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const f32x4 vs4 = *reinterpret_cast<const f32x4*>(&vs_lds[cur][8 * q4 + 4 * kt]);
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[4 * kt + r] *= vs4[r];
          }
          pb = __builtin_convertvector(pv, vec);
        }
        return pb;
      };
      // One query tile at a time; all V operands stay in registers.
      vec va[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) va[n] = v_operand(n);
      if constexpr (!decltype(masked)::value && !kScaled) {
        // Software-pipelined over the tiles: tile t's P and tile t - 1's V
        // MFMAs form one scheduling region, inside which group barriers
        // interleave them (an MFMA, two exponentials, two other VALU
        // instructions, ...) so that the matrix core works while the VALU
        // computes P.  Left to itself the scheduler issues every
        // exponential of the page first and every V MFMA after them.
        vec p_prev = p_operand(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 1; t < NQ; ++t) {
          const vec pb = p_operand(t);
#pragma unroll
          for (int n = 0; n < NT; ++n)
            o_acc[n][t - 1] = Mfma<AF>::mma(va[n], p_prev, o_acc[n][t - 1]);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedTrans, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 2, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          p_prev = pb;
        }
#pragma unroll
        for (int n = 0; n < NT; ++n)
          o_acc[n][NQ - 1] = Mfma<AF>::mma(va[n], p_prev, o_acc[n][NQ - 1]);
      } else {
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          const vec pb = p_operand(t);
#pragma unroll
          for (int n = 0; n < NT; ++n) o_acc[n][t] = Mfma<AF>::mma(va[n], pb, o_acc[n][t]);
        }
      }
      };
      // Masked where the page reaches past the earliest query, or (window)
      // below the window of the latest one.
      if (base + BS - 1 > pos_lo || (WIN && base <= pos_hi - window)) {
        page(std::true_type{});
      } else {
        page(std::false_type{});
      }
    }
    if constexpr (kDma) {
      // After the second page of a pair: this wave's share of the next pair
      // has landed; the barrier publishes every wave's share and retires
      // the pair just computed for reuse.
      if ((p & 1) == 1 && p + 1 < npages) {
        wait_vmcnt<0>();
        lds_barrier();
      }
    } else {
      if constexpr (WIN) {
        if (p + 1 < npages) store_win(cur ^ 1);
      } else {
        if (p + 1 < npages) store_regs(cur ^ 1, base + BS);
      }
      __syncthreads();
      cur ^= 1;
    }
  }

  if (!wave_live) return;
  // l of each query: the partial sums of the four lanes that hold it.
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    l_acc[t] += shfl_xor_f(l_acc[t], 16);
    l_acc[t] += shfl_xor_f(l_acc[t], 32);
  }
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int r = row0 + 16 * t + col;
    if (r >= rows) continue;
    const int j = r / G;
    const int hq = g * G + r - j * G;
    const float inv = v_scale / l_acc[t];
    uint16_t* dst = out + ((size_t)(q_begin + j) * Hq + hq) * D + 4 * q4;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const f32x4 o = o_acc[n][t] * inv;
      *reinterpret_cast<u32x2*>(dst + 16 * n) =
          __builtin_bit_cast(u32x2, __builtin_convertvector(o, typename Vec4<AF>::type));
    }
  }
}

// Query tiles of 16 rows per wave: as many as fit in 256 VGPRs at two waves
// per SIMD (the byte formats keep their widening temporaries live too, INT8
// its row scales and a second P operand, the window path its staged
// activation rows, and over a quantised ring both).
template <int D, int CF, bool WIN>
constexpr int query_tiles() {
  if (D <= 64) return 4;
  if (D <= 96) return WIN && byte_fmt(CF) ? 2 : byte_fmt(CF) || WIN ? 3 : 4;
  return byte_fmt(CF) || WIN ? 2 : 3;
}

template <int D, int CF, int AF, bool WIN>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  constexpr int NQ = query_tiles<D, CF, WIN>();
  constexpr int RW = 16 * NQ * kWaves;
  const int G = a.Hq / a.Hkv;
  const long long row_tiles = ((long long)a.max_chunk * G + RW - 1) / RW;
  const long long items = row_tiles * a.Hkv * a.B;
  const long long per_xcd = (items + kXcds - 1) / kXcds;
  if (per_xcd * kXcds > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // An E4M3 cache's tensor scales fold into the score and output scales
  // (in the window path the chunk's own rows are staged divided by them).
  constexpr bool kFold = CF == FMT_E4M3;
  const float qk = a.softmax_scale * (kFold ? a.k_scale : 1.f) * LOG2E_P;
  const float vs = kFold ? a.v_scale : 1.f;
  // The chunk rows' multipliers of the window path over an E4M3 ring
  // (1 / scale, capped to a finite value for denormal scales).
  const float kmul = WIN && kFold ? fminf(1.f / a.k_scale, FLT_MAX) : 1.f;
  const float vmul = WIN && kFold ? fminf(1.f / a.v_scale, FLT_MAX) : 1.f;
  hipLaunchKernelGGL((prefill_kernel<D, CF, AF, NQ, WIN>), dim3((unsigned)(per_xcd * kXcds)),
                     dim3(kThreads), 0, s, (uint16_t*)a.out, (const uint16_t*)a.query,
                     a.cu_q_lens, (const uint8_t*)a.key_cache, (const uint8_t*)a.value_cache,
                     a.block_tables, a.context_lens, a.Hq, a.Hkv, G, a.B, a.MBPS,
                     (int)row_tiles, qk, vs, a.key_scales, a.value_scales,
                     (const uint16_t*)a.key_act, (const uint16_t*)a.value_act, a.window,
                     kmul, vmul);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  if (a.window > 0) {
    if (a.act == FMT_BF16) {
      if (a.cache == FMT_BF16) return launch_t<D, FMT_BF16, FMT_BF16, true>(a, s);
      if (a.cache == FMT_E4M3) return launch_t<D, FMT_E4M3, FMT_BF16, true>(a, s);
      if (a.cache == FMT_I8) return launch_t<D, FMT_I8, FMT_BF16, true>(a, s);
    } else if (a.act == FMT_F16) {
      if (a.cache == FMT_F16) return launch_t<D, FMT_F16, FMT_F16, true>(a, s);
      if (a.cache == FMT_E4M3) return launch_t<D, FMT_E4M3, FMT_F16, true>(a, s);
      if (a.cache == FMT_I8) return launch_t<D, FMT_I8, FMT_F16, true>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.act == FMT_BF16) {
    if (a.cache == FMT_BF16) return launch_t<D, FMT_BF16, FMT_BF16, false>(a, s);
    if (a.cache == FMT_E4M3) return launch_t<D, FMT_E4M3, FMT_BF16, false>(a, s);
    if (a.cache == FMT_I8) return launch_t<D, FMT_I8, FMT_BF16, false>(a, s);
  } else if (a.act == FMT_F16) {
    if (a.cache == FMT_F16) return launch_t<D, FMT_F16, FMT_F16, false>(a, s);
    if (a.cache == FMT_E4M3) return launch_t<D, FMT_E4M3, FMT_F16, false>(a, s);
    if (a.cache == FMT_I8) return launch_t<D, FMT_I8, FMT_F16, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int D, int G, int act, int cache) {
  if (D != 64 && D != 96 && D != 128) return false;
  if (G < 1 || G > 16) return false;
  if (act != FMT_BF16 && act != FMT_F16) return false;
  return cache == act || cache == FMT_E4M3 || cache == FMT_I8;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.max_chunk <= 0 || a.B <= 0) return hipSuccess;
  switch (a.D) {
    case 64: return launch_d<64>(a, s);
    case 96: return launch_d<96>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
