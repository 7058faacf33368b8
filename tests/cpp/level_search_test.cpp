// CPU test of the radix-select level arithmetic (row_wise_topk_amd/csrc/level_search.h).
//
// 1. Consistent counts: a level loop driven by real histograms of random
//    value sets finds the need-th smallest value (the column search of a cut)
//    and the need-th largest (the key search), checked against std::sort, and
//    ends within kMaxLevels levels.
// 2. Inconsistent counts (random bins, counts and "not found" answers, as a
//    corrupt buffer might produce): every loop ends within kMaxLevels levels,
//    and narrow() never leaves the range it started from.
#define __host__
#define __device__
#include "level_search.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

using dstk::RangeLevel;

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

// The need-th value (1-based) of `vals` in [lo, hi], ascending if `asc`,
// found level by level the way the kernels do: a histogram of 2^11 bins per
// level, searched in order.
static bool level_loop(const std::vector<uint32_t>& vals, uint32_t lo, uint32_t hi, uint32_t need,
                       bool asc, uint32_t* out, int* levels) {
  RangeLevel lv{lo, hi, need, 0};
  const uint32_t nb = 1u << RangeLevel::kBits;
  for (int it = 0; it < RangeLevel::kMaxLevels; ++it) {
    const uint32_t s = lv.shift();
    std::vector<uint32_t> h(nb, 0);
    for (uint32_t v : vals)
      if (v >= lv.base && v <= lv.top) ++h[(v - lv.base) >> s];
    // search order: ascending bins, or descending for the largest first
    uint32_t acc = 0, bin = nb, before = 0, cnt = 0;
    for (uint32_t i = 0; i < nb; ++i) {
      const uint32_t b = asc ? i : nb - 1 - i;
      if (acc < lv.need && lv.need <= acc + h[b]) { bin = b; before = acc; cnt = h[b]; break; }
      acc += h[b];
    }
    if (!lv.narrow(bin, before, cnt)) return false;
    *levels = lv.level;
    if (cnt == lv.need) {   // the whole bin is taken: its edge is the answer
      *out = asc ? lv.top : lv.base;
      return true;
    }
    if (lv.single()) { *out = lv.base; return true; }
  }
  return false;
}

int main() {
  std::mt19937_64 rng(12345);
  // 1. consistent counts
  for (int trial = 0; trial < 3000; ++trial) {
    const int n = 1 + static_cast<int>(rng() % 3000);
    const int mode = trial % 4;
    std::vector<uint32_t> v(n);
    for (auto& x : v) {
      switch (mode) {
        case 0: x = static_cast<uint32_t>(rng()); break;                 // full 32-bit range
        case 1: x = static_cast<uint32_t>(rng() % 50); break;             // heavy ties
        case 2: x = 0x80000000u + static_cast<uint32_t>(rng() % 100000); break;
        default: x = static_cast<uint32_t>(rng() % 2147483647u); break;   // 31-bit columns
      }
    }
    std::vector<uint32_t> sv = v;
    std::sort(sv.begin(), sv.end());
    const uint32_t lo = sv.front(), hi = sv.back();
    const uint32_t need = 1 + static_cast<uint32_t>(rng() % n);
    for (int asc = 0; asc < 2; ++asc) {
      uint32_t out = 0;
      int levels = 0;
      const bool ok = level_loop(v, lo, hi, need, asc != 0, &out, &levels);
      CHECK(ok);
      CHECK(levels <= RangeLevel::kMaxLevels);
      const uint32_t want = asc ? sv[need - 1] : sv[n - need];
      // The answer is exact when the loop ended on a single value; when it
      // ended on a whole bin, that bin's members up to the answer are all taken.
      if (ok) {
        if (asc) CHECK(out >= want && std::count_if(sv.begin(), sv.end(), [&](uint32_t x) { return x <= out; }) >= need);
        else CHECK(out <= want && std::count_if(sv.begin(), sv.end(), [&](uint32_t x) { return x >= out; }) >= need);
      }
    }
  }
  // 2. inconsistent counts: any answers at all, the loop still ends
  for (int trial = 0; trial < 200000; ++trial) {
    uint32_t lo = static_cast<uint32_t>(rng()), hi = static_cast<uint32_t>(rng());
    if (lo > hi) std::swap(lo, hi);
    RangeLevel lv{lo, hi, 1 + static_cast<uint32_t>(rng() % 5000), 0};
    int it = 0;
    for (; it < 100; ++it) {
      const uint32_t bin = (rng() % 8 == 0) ? (1u << RangeLevel::kBits) + static_cast<uint32_t>(rng() % 4)
                                            : static_cast<uint32_t>(rng() % (1u << RangeLevel::kBits));
      const uint32_t before = static_cast<uint32_t>(rng() % 6000), cnt = static_cast<uint32_t>(rng() % 6000);
      const uint32_t b0 = lv.base, t0 = lv.top;
      if (!lv.narrow(bin, before, cnt)) {
        CHECK(lv.base == b0 && lv.top == t0);
        break;
      }
      CHECK(lv.base >= b0 && lv.top <= t0 && lv.base <= lv.top);
      if (lv.single()) break;
    }
    CHECK(it <= RangeLevel::kMaxLevels);
  }
  std::printf(fails ? "level search: %d failures\n" : "level search: ok\n", fails);
  return fails ? 1 : 0;
}
