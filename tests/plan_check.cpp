// plan_check.cpp -- host-only check of the decode plan's invariants
// (paged_kv_cache_175_amd/csrc/plan.hpp), which the kernels rely on for
// staying inside their buffers:
//
//   grid mode     the splits cover the item; every wave of every split holds at most
//                 kPagesPerWave pages (its table register), for every length
//                 up to the length cap; at most 65535 splits;
//   pair mode     every page of every item is read exactly once (by its own
//                 workgroup or its one helper), and every job fits a wave;
//                 the kernel's ballot ranking gives the same ranks and partners;
//   balanced mode a range spans at most kPagesPerWave * W pages, the ranges
//                 cover the batch, and no item meets more ranges than it has
//                 partial slots, for random length mixes up to the cap;
//   workspace     the counter region at offset 0 holds B*Hkv counters and
//                 is the same region for every shape with B*Hkv <=
//                 kMinCounters; the partial regions follow it, disjoint.
//
// Built with g++ and run by tests/test_plan_host.py.  Prints one line and
// exits 0 when every case holds, 1 (naming the case) otherwise.

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../paged_kv_cache_175_amd/csrc/plan.hpp"

using namespace pa::plan;

static long long g_cases = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      std::printf("FAIL %s: ", #cond);                     \
      std::printf(__VA_ARGS__);                            \
      std::printf("\n");                                   \
      std::exit(1);                                        \
    }                                                      \
  } while (0)

static long long pages_of(long long L) { return L > 0 ? (L + kBlock - 1) / kBlock : 0; }

static long long wave_pages(long long n, int w, int W) { return n > w ? (n - w + W - 1) / W : 0; }

static void check_grid(int B, int Hkv, int max_len, int window, int part, const Plan& p) {
  const long long cap = len_cap(max_len, window);
  CHECK(p.S >= 1 && p.S <= 65535, "S=%d", p.S);
  CHECK(p.W == 4 || p.W == 8, "W=%d", p.W);
  CHECK(p.slots == (p.pair ? 2 : p.S), "slots=%d", p.slots);
  CHECK(!p.pair || (p.S == 1 && B <= kMaxPairB), "pair mode with S=%d B=%d", p.S, B);
  // Lengths the kernel may meet after clamping: a spread over [1, cap].
  std::vector<long long> lens = {1, 2, 31, 32, 33, 63, 64, 65, cap, cap - 1, cap - 31, cap / 2,
                                 cap / 3 + 7};
  for (long long L : lens) {
    if (L < 1 || L > cap) continue;
    const int P = (int)pages_of(L);
    long long covered = 0;
    for (int s = 0; s < p.S; ++s) {
      // Split s of the kernel: pages [s P / S, (s + 1) P / S).
      const int a = (int)((long long)s * P / p.S), b = (int)((long long)(s + 1) * P / p.S);
      CHECK(a <= b && (s > 0 || a == 0) && (s + 1 < p.S || b == P), "split %d: [%d, %d) of %d",
            s, a, b, P);
      covered += b - a;
      for (int w = 0; w < p.W; ++w) {
        const long long npg = wave_pages(b - a, w, p.W);
        CHECK(npg <= kPagesPerWave, "B=%d Hkv=%d max_len=%d window=%d part=%d L=%lld s=%d npg=%lld",
              B, Hkv, max_len, window, part, L, s, npg);
      }
    }
    CHECK(covered == P, "splits cover %lld of %d pages", covered, P);
    ++g_cases;
  }
}

// The kernel's ranking, restated on the host: lane j's key is its pages then
// 63 - j; a sequence's rank is the count of larger keys, and its partner's
// key the one with exactly B - 1 - r larger keys, found bit by bit from the
// top with one count per bit (the kernel counts with ballots).
static void kernel_rank(const std::vector<int>& P, int B, int b, int p_max, int* r,
                        int* partner) {
  unsigned key[64];
  for (int l = 0; l < 64; ++l) key[l] = l < B ? ((unsigned)P[l] << 6) | (unsigned)(63 - l) : 0u;
  int rr = 0;
  for (int l = 0; l < 64; ++l) rr += key[l] > key[b];
  int kbits = 6;
  for (unsigned m = (unsigned)(p_max > 1 ? p_max : 1); m; m >>= 1) ++kbits;
  unsigned prefix = 0;
  int above = B - 1 - rr;
  for (int bit = kbits - 1; bit >= 0; --bit) {
    const unsigned hi = ~((1u << bit) - 1u);
    const unsigned cand = prefix | (1u << bit);
    int n = 0;
    for (int l = 0; l < B; ++l) n += (key[l] & hi) == cand;
    if (above < n) prefix = cand;
    else above -= n;
  }
  *r = rr;
  *partner = 63 - (int)(prefix & 63u);
}

// Pair mode: rank by pages (ties by index), pair rank r with B - 1 - r, the
// shorter item's workgroup reads [a, Pl) of the longer one (pair_split), as
// the kernel computes it from the batch's lengths.  Every page of every item
// is read exactly once, no workgroup helps more than one item, every job
// fits a wave's table register, and an item is divided in two at most.
static void check_pairs(std::mt19937_64& rng, const Plan& p, int B, long long cap) {
  for (int trial = 0; trial < 8; ++trial) {
    std::vector<int> P(B);
    for (int b = 0; b < B; ++b) {
      long long L = trial == 0 ? cap : trial == 1 ? (b % 2 ? cap : 0)
                  : trial == 2 ? cap - std::uniform_int_distribution<long long>(0, 3 * kBlock)(rng)
                  : std::uniform_int_distribution<long long>(0, cap)(rng);
      P[b] = (int)pages_of(L < 0 ? 0 : L);
    }
    std::vector<int> rank(B, 0);
    for (int i = 0; i < B; ++i)
      for (int j = 0; j < B; ++j) rank[i] += P[j] > P[i] || (P[j] == P[i] && j < i);
    std::vector<int> by_rank(B);
    for (int i = 0; i < B; ++i) by_rank[rank[i]] = i;
    // The kernel skips the ranking when every length is within
    // kMinHelpPages - 1 pages of the first one's: then no pair may help.
    bool near = true;
    for (int b = 0; b < B; ++b) near &= std::abs(P[b] - P[0]) <= kMinHelpPages - 1;
    if (near)
      for (int i = 0; i < B; ++i)
        for (int j = 0; j < B; ++j)
          if (P[i] >= P[j]) CHECK(pair_split(P[i], P[j]) == P[i], "a help within the shortcut");
    const int p_max = (int)pages_of(cap);
    for (int b = 0; b < B; ++b) {
      int kr, kp;
      kernel_rank(P, B, b, p_max, &kr, &kp);
      CHECK(kr == rank[b] && kp == by_rank[B - 1 - rank[b]],
            "kernel ranking of item %d: rank %d partner %d, want %d %d", b, kr, kp, rank[b],
            by_rank[B - 1 - rank[b]]);
    }
    std::vector<long long> read(B, 0);
    std::vector<int> helped_by(B, -1);
    for (int b = 0; b < B; ++b) {
      const int r = rank[b], pr = B - 1 - r, partner = by_rank[pr];
      int own_hi = P[b];
      if (r < pr) own_hi = pair_split(P[b], P[partner]);
      read[b] += own_hi;
      for (int w = 0; w < p.W; ++w)
        CHECK(wave_pages(own_hi, w, p.W) <= kPagesPerWave, "own job too long");
      if (r > pr) {
        const int a = pair_split(P[partner], P[b]);
        if (a < P[partner]) {
          CHECK(helped_by[partner] < 0, "item %d helped twice", partner);
          helped_by[partner] = b;
          read[partner] += P[partner] - a;
          for (int w = 0; w < p.W; ++w)
            CHECK(wave_pages(P[partner] - a, w, p.W) <= kPagesPerWave, "help job too long");
        }
      }
    }
    for (int b = 0; b < B; ++b)
      CHECK(read[b] == P[b], "item %d: %lld of %d pages read", b, read[b], P[b]);
    ++g_cases;
  }
}

static void check_balanced(std::mt19937_64& rng, int B, int Hkv, int max_len, int window,
                           const Plan& p) {
  const long long cap = len_cap(max_len, window);
  CHECK(p.W == 8 && p.S >= 2, "W=%d S=%d", p.W, p.S);
  for (long long cus : {1LL, 80LL, 256LL, 304LL}) {
    const long long N = balanced_workgroups(B, Hkv, max_len, window, cus, p.W);
    CHECK(N >= 1 && N % cus == 0 && N < (1LL << 31), "N=%lld", N);
    for (int trial = 0; trial < 6; ++trial) {
      // Length mixes: all at the cap, one long among short ones, uniform.
      std::vector<long long> P(B);
      for (int b = 0; b < B; ++b) {
        long long L;
        if (trial == 0) L = cap;
        else if (trial == 1) L = b == 0 ? cap : 1;
        else if (trial == 2) L = b == B - 1 ? cap : 0;
        else L = std::uniform_int_distribution<long long>(0, cap)(rng);
        P[b] = pages_of(L);
      }
      long long T = 0, pmax = 0;
      for (long long x : P) {
        T += Hkv * x;
        pmax = x > pmax ? x : pmax;
      }
      CHECK(T < (1LL << 31), "T=%lld", T);
      const long long c = balanced_range_pages((int)T, (int)N, (int)pmax, p.S, p.W);
      CHECK(c >= p.W && c % p.W == 0, "c=%lld", c);
      CHECK(c <= kPagesPerWave * p.W, "B=%d Hkv=%d max_len=%d window=%d cus=%lld c=%lld", B, Hkv,
            max_len, window, cus, c);
      CHECK(N * c >= T, "ranges do not cover the batch: N=%lld c=%lld T=%lld", N, c, T);
      long long off = 0;
      for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g, off += P[b]) {
          if (P[b] == 0) continue;
          const long long ranges = (off + P[b] - 1) / c - off / c + 1;
          CHECK(ranges <= p.S, "item (%d,%d) of %lld pages meets %lld ranges, %d slots", b, g,
                P[b], ranges, p.S);
        }
      }
      ++g_cases;
    }
  }
}

static void check_workspace(int B, int Hq, int Hkv, int D, const Plan& p) {
  const size_t need = workspace_for(B, Hq, Hkv, D, p);
  if (p.slots <= 1) {
    CHECK(need == 0, "one part per item needs no workspace");
    return;
  }
  const WsLayout w = ws_layout(B, Hq, Hkv, D, p.slots);
  const size_t rows = (size_t)B * Hq * p.slots;
  CHECK(w.m >= (size_t)B * Hkv * 4, "counters");
  CHECK(w.m >= kMinCounters * 4, "counter region below its minimum");
  if ((size_t)B * Hkv <= kMinCounters) CHECK(w.m == counter_bytes(1, 1), "counter region moved");
  CHECK(w.l >= w.m + rows * 4 && w.o >= w.l + rows * 4 && w.total >= w.o + rows * D * 4,
        "regions overlap");
  CHECK(w.m % kAlign == 0 && w.l % kAlign == 0 && w.o % kAlign == 0, "alignment");
  CHECK(need == w.total, "size");
}

int main() {
  std::mt19937_64 rng(12345);
  const int Bs[] = {1, 2, 3, 8, 32, 64, 129, 1024, 2048};
  const int Hkvs[] = {1, 2, 8, 32};
  const int lens[] = {0, 1, 31, 32, 33, 512, 1000, 1023, 1024, 1025, 2048, 4096, 8191, 8192,
                      32768, 65536, 131072, 1 << 20};
  const int windows[] = {0, 32, 1024, 4096, 65536};
  const int parts[] = {0, 32, 256, 1024, 4096};
  for (int B : Bs)
    for (int Hkv : Hkvs)
      for (int max_len : lens)
        for (int window : windows)
          for (int part : parts)
            for (int byte_cache = 0; byte_cache < 2; ++byte_cache) {
             for (int G : {1, 4, 16}) {
              Plan p{};
              if (!make_plan(B, Hkv, G, 128, max_len, window, part, byte_cache != 0, &p))
                continue;
              if (p.balanced) {
                CHECK(byte_cache && part == 0 && B <= kMaxBalancedB, "balanced for B=%d", B);
                if ((long long)B * Hkv * pages_of(len_cap(max_len, window)) < (1LL << 26))
                  check_balanced(rng, B, Hkv, max_len, window, p);
              } else {
                check_grid(B, Hkv, max_len, window, part, p);
                if (p.pair) {
                  CHECK(pair_fits(p.W, G, 128), "pair mode without room in LDS");
                  check_pairs(rng, p, B, len_cap(max_len, window));
                }
              }
              check_workspace(B, G * Hkv, Hkv, 128, p);
             }
            }
  std::printf("ok %lld cases\n", g_cases);
  return 0;
}
