// plan.hpp -- the decode plan: how the pages of a batch are shared out between
// workgroups, and the layout of the decode workspace.  Plain C++: the C ABI
// computes the plan on the host, the balanced kernel calls
// balanced_range_pages() on the device (a constexpr function), and a
// host-only program checks the invariants the kernels rely on over a sweep
// of shapes.
#pragma once

#include <stddef.h>

#include "../../include/pa.h"

namespace pa {
namespace plan {

constexpr int kBlock = 32;
// Grid mode aims at this many resident waves (8 per CU on the 256 CUs of an
// MI355X).
constexpr long long kTargetWaves = 2048;
// Below this many tokens every sequence is one split: one launch, no
// workspace (a split's merge costs more than it saves there).
constexpr long long kMinSplitContext = 1024;
// The last split to finish merges the partials 16 per memory round trip;
// more than 16 automatic splits cost more in that merge than they gain
// (single sequence, 8192 tokens: 16 splits 12.9 us, 32 splits 15.5 us).
constexpr long long kMaxAutoSplits = 16;
// Balanced mode: the kernel keeps the batch's page prefix sums in LDS, for
// at most kMaxBalancedB sequences.
constexpr int kMaxBalancedB = 1024;
constexpr long long kMinBalancedSlots = 16;
// A wave holds the table entries of its pages in one 64-lane register.
constexpr long long kPagesPerWave = 64;
constexpr size_t kAlign = 256;
constexpr size_t kMinCounters = PA_DECODE_MIN_COUNTERS;

template <typename T>
constexpr T max_of(T a, T b) { return a > b ? a : b; }
template <typename T>
constexpr T min_of(T a, T b) { return a < b ? a : b; }

constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Decode plan, a dispatch by cache format and context length.
//
// Grid mode (decode_split): a workgroup of W waves handles one split of the
// pages of one (sequence, KV head).  Below kMinSplitContext tokens every
// sequence is one split.  From kMinSplitContext on, the automatic choice
// aims at kTargetWaves resident waves: W = 8 while B * Hkv <= 256, else
// W = 4; S splits per sequence so that B * Hkv * S * W ~ kTargetWaves, with
// at least one page per wave on the longest sequence and at most
// kMaxAutoSplits.  A split spans at most kPagesPerWave * W pages.
// partition_tokens > 0 forces S = ceil(len / partition_tokens).
//
// Balanced mode (decode_balanced), for E4M3 and INT8 caches from
// kMinSplitContext tokens on (partition_tokens == 0) where the grid plan is
// not pair mode: the batch's pages are cut into equal ranges, one per
// workgroup (W = 8, a multiple of the CU count of workgroups), whatever the
// mix of context lengths; S is then the number of partial slots per
// (sequence, KV head).  Against the grid plan without pairs, on the FP8
// decode shape (B = 64, 1024..8192 tokens): INT8 131 -> 118 us, E4M3 118.5
// -> 117.4 us; pair mode beats both there (E4M3 107.7 us, INT8 104.3 us),
// so a byte cache takes balanced mode only where pairs do not apply (more
// than kMaxPairB sequences, or several splits per sequence).  With 16-bit
// caches the grid plan stayed faster (Mistral batch 57.6 vs 59.9 us;
// rolling batch 27.6 vs 29.8 us): its prefix scan and the merges of the
// sequences cut between ranges cost more than the balance gains there.
struct Plan {
  int S;          // grid mode: splits per sequence; balanced: partial slots per item
  int W;
  bool balanced;  // one equal range of the batch's pages per workgroup
  bool pair;      // grid mode, one split: short sequences help long ones (below)
  int slots;      // workspace partials per (sequence, query head)
};

// Pair mode: one split per (sequence, KV head) leaves the longest sequences
// streaming alone at the end, at one CU's rate.  Every workgroup ranks the
// sequences by pages (B <= kMaxPairB, one wave) and pairs rank r with rank
// B - 1 - r; the workgroup of the shorter sequence of a pair also reads the
// tail of the longer one (pair_split), for the same KV head.  Its wave
// partials of the two jobs sit side by side in LDS, beside a copy of the
// help job's queries per wave; pair mode is built where these take at most
// 48 KiB (two workgroups of 4 waves still fit a CU).
constexpr int kMaxPairB = 64;
constexpr bool pair_fits(int W, int G, int D) {
  return 2 * W * G * D * 4 + W * G * D * 2 <= 49152;
}
// A help job shorter than this is not worth its merge.
constexpr int kMinHelpPages = 4;

// The longer item of a pair (Pl >= Ps pages) keeps pages [0, a); its helper
// reads [a, Pl), so that the two workgroups read the same number of pages.
// No help (a = Pl) when fewer than kMinHelpPages would move.
constexpr int pair_split(int Pl, int Ps) {
  const int a = (Pl + Ps + 1) / 2;
  return Pl - a >= kMinHelpPages ? a : Pl;
}

// Tokens a sequence may attend to at most (the kernels clamp each length to
// it): max_context_len, capped at the window.
constexpr long long len_cap(long long max_len, int window) {
  return window > 0 ? min_of<long long>(window, max_len) : max_len;
}

inline bool make_plan(int B, int Hkv, int G, int D, int max_len, int window,
                      int partition_tokens, bool byte_cache, Plan* p) {
  long long L = len_cap(max_len, window);
  if (L < 1) L = 1;
  if (partition_tokens < 0 || partition_tokens % kBlock != 0) return false;
  const long long pages = (L + kBlock - 1) / kBlock;
  const long long pairs = (long long)B * Hkv;
  // The grid plan.
  const int W = pairs > 256 ? 4 : 8;
  long long S;
  if (partition_tokens > 0) {
    S = (L + partition_tokens - 1) / partition_tokens;
  } else if (L < kMinSplitContext) {
    S = 1;
  } else {
    S = pairs > 0 ? kTargetWaves / (pairs * W) : 1;
    S = min_of(S, pages / W);
    S = min_of(S, kMaxAutoSplits);
    S = max_of(S, 1LL);
  }
  // A wave holds at most kPagesPerWave pages.
  S = max_of(S, (pages + kPagesPerWave * W - 1) / (kPagesPerWave * W));
  const bool pair = S == 1 && partition_tokens == 0 && L >= kMinSplitContext &&
                    B <= kMaxPairB && pair_fits(W, G, D);
  if (byte_cache && !pair && partition_tokens == 0 && L >= kMinSplitContext &&
      B <= kMaxBalancedB && pairs * pages < (1LL << 31)) {
    // Balanced mode: ranges of at most kPagesPerWave * W pages, and partial
    // slots enough that no item spans more of them.
    p->balanced = true;
    p->pair = false;
    p->W = 8;
    p->S = (int)max_of(kMinBalancedSlots,
                       (pages + kPagesPerWave * p->W - 1) / (kPagesPerWave * p->W) + 1);
    p->slots = p->S;
    return true;
  }
  if (S > 65535) return false;
  p->balanced = false;
  p->S = (int)S;
  p->W = W;
  p->pair = pair;
  p->slots = p->pair ? 2 : p->S;
  return true;
}

// Balanced mode: workgroups of the launch.  One range per CU, or a multiple
// of the CU count so that no range exceeds kPagesPerWave * W pages.
inline long long balanced_workgroups(int B, int Hkv, long long max_len, int window,
                                     long long cus, int W) {
  const long long L = len_cap(max_len, window);
  const long long tmax = (long long)B * Hkv * ((L + kBlock - 1) / kBlock);
  return cus * max_of(1LL, (tmax + cus * kPagesPerWave * W - 1) / (cus * kPagesPerWave * W));
}

// Balanced mode: pages per range, given the batch's T pages (all heads), the
// N workgroups, the longest item's pmax pages and the Smax partial slots:
// equal shares of N, at least one page per wave, few enough workgroups per
// item for the partial slots (an item of P pages meets at most ceil(P/c) + 1
// ranges), and a multiple of W.
constexpr int balanced_range_pages(int T, int N, int pmax, int Smax, int W) {
  int c = (T + N - 1) / N;
  c = max_of(c, (pmax + Smax - 2) / (Smax - 1));
  c = max_of(c, W);
  return (c + W - 1) / W * W;
}

// Workspace of a split plan.  The split arrival counters come first, at
// offset 0: max(B*Hkv, kMinCounters) int32, so that the counter region starts
// and (up to kMinCounters pairs) ends at the same place whatever the shape,
// and the partials of one call never land on a counter of a later call.
// Then m and l [B*Hq*S] and o [B*Hq*S*D] fp32; each region 256-byte aligned.
inline size_t counter_bytes(int B, int Hkv) {
  return round_up(max_of((size_t)B * Hkv, kMinCounters) * sizeof(int), kAlign);
}

struct WsLayout {
  size_t m, l, o, total;  // byte offsets of the regions, and the size
};

inline WsLayout ws_layout(int B, int Hq, int Hkv, int D, int S) {
  const size_t rows = (size_t)B * Hq * S;
  WsLayout w;
  w.m = counter_bytes(B, Hkv);
  w.l = w.m + round_up(rows * sizeof(float), kAlign);
  w.o = w.l + round_up(rows * sizeof(float), kAlign);
  w.total = w.o + round_up(rows * D * sizeof(float), kAlign);
  return w;
}

inline size_t workspace_for(int B, int Hq, int Hkv, int D, const Plan& p) {
  if (p.slots <= 1) return 0;
  return ws_layout(B, Hq, Hkv, D, p.slots).total;
}

}  // namespace plan
}  // namespace pa
