// The range arithmetic of one MSD radix-select level, shared by the streaming
// kernel's cuts (host and device, so that it is tested on the CPU).
//
// A level bins an unsigned range [base, top] into 2^kBits bins of 2^shift
// values each, shift = max(0, bit_length(top - base) - kBits).  A histogram
// search then names the bin that holds the need-th member in search order,
// with `before` members ranked ahead of that bin and `count` in it.  narrow()
// moves the range to that bin.  A 32-bit range is resolved in at most
// kMaxLevels levels (11 + 11 + 10 bits); narrow() refuses a further level,
// and refuses counts that no buffer can produce (no bin found, or a bin that
// cannot hold the rest), so that a caller's level loop always ends.
#pragma once

#include <stdint.h>

namespace dstk {

struct RangeLevel {
  static constexpr int kBits = 11;
  static constexpr int kMaxLevels = 3;

  uint32_t base;   // lowest value of the range
  uint32_t top;    // highest value of the range
  uint32_t need;   // members still to take, in search order, inside the range
  int level;       // levels narrowed so far

  __host__ __device__ uint32_t shift() const {
    const uint32_t span = top - base;
    const uint32_t bl = span ? 32u - static_cast<uint32_t>(__builtin_clz(span)) : 0u;
    return bl > static_cast<uint32_t>(kBits) ? bl - static_cast<uint32_t>(kBits) : 0u;
  }

  // Narrow to bin `bin` (ascending, 0 = the bin holding `base`).  Returns
  // false, and leaves the range as it was, when the level is not possible.
  __host__ __device__ bool narrow(uint32_t bin, uint32_t before, uint32_t count) {
    if (level >= kMaxLevels) return false;
    if (bin >= (1u << kBits)) return false;            // the search found no bin
    if (before >= need || count < need - before) return false;
    const uint32_t s = shift();
    const uint64_t lo = static_cast<uint64_t>(base) + (static_cast<uint64_t>(bin) << s);
    if (lo > top) return false;                        // a bin past the range
    const uint64_t hi = lo + ((uint64_t{1} << s) - 1u);
    base = static_cast<uint32_t>(lo);
    top = hi < top ? static_cast<uint32_t>(hi) : top;
    need -= before;
    ++level;
    return true;
  }

  // The range is a single value (the search is over).
  __host__ __device__ bool single() const { return base == top; }
};

}  // namespace dstk
