// Row-wise TopK kernels for MI355X (gfx950, wave64).
//
// Method (narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for
// sparse attention and sampling", method paragraph): keep a threshold T that
// starts at -inf and never falls; read the row once in contiguous blocks of B
// elements visited in a random order; append the values that pass T to a
// candidate buffer; when the buffer reaches k + B2 entries, radix-select it back
// to k and raise T.  The pages' CUDA design is prior art only; what follows is
// laid out for CDNA4, where a wave64 vector instruction occupies its 16-lane
// SIMD for 4 cycles and a workgroup has few waves per SIMD, so the cost of every
// step is close to its instruction count:
//
//  * one workgroup (256 or 512 lanes) streams a row, or a share of a row's
//    blocks when several workgroups cooperate on one row;
//  * a block is B = 4096 elements; every lane issues 16-byte loads, and the
//    loads of the next 3 blocks are always in flight (a register ring whose
//    loads are issued unconditionally, so the compiler waits for exactly the
//    block being filtered);
//  * the first whole block sets T from histograms of its values held in
//    registers (one per wave), so the buffer never has to hold a block
//    admitted at -inf; a workgroup with a short share of a row starts from
//    an estimate of the row's 1.5k-th to 3k-th value instead, checked by the
//    merge or by the final count (should it fail, the row is read again from
//    a valid bound);
//  * the filter compares raw fp32 values (bf16 widened by a shift) with a
//    wave-wide early-out on each lane's running maximum; survivors are
//    compacted into LDS with ballot / mbcnt and one LDS atomic per wave;
//  * a candidate is one 64-bit composite in LDS, so the cut (radix select) is
//    an 11-bit histogram over the high word in the live range [T, max], refined
//    only when the boundary bin is too full, and keeping a candidate is one
//    64-bit compare; exact ties on a key are cut by column the same way;
//  * several workgroups on one row share T through a 64-bit atomicMax in
//    device memory; the last to finish merges the others' survivors (fp32
//    rows shared this way run 512-lane workgroups, one per CU);
//  * the epilogue orders the k results by value or by column (histogram
//    grouping, in-bin rank, re-binning of large bins) and writes indices,
//    values and status.
//
// Order and tie-break (xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！",
// Q&A on stable results): larger value first, then lower column.  A value v at
// column i has the composite  (key(v) << 32) | ~i,  where key() maps fp32
// sign-magnitude onto unsigned offset binary so that -0.0 and +0.0 share one
// key.  The threshold T is a composite too: an element is admitted iff its
// composite is > T, so T can sit between two equal values with different
// columns.  Every published T leaves at least k composites of the row above it.
// Output values are rebuilt from the key (exact for every non-NaN value but a
// zero, whose sign is read back from the input).
//
// NaN (narracomm.com, NaN paragraph): always checked over [0, end); a NaN sets
// a status bit for the row instead of trapping.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ds_topk.h"
#include "level_search.h"
#include "topk_internal.h"

namespace dstk {
namespace {

constexpr int kRadixBits = 11;
constexpr int kBins = 1 << kRadixBits;
static_assert(kRadixBits == RangeLevel::kBits, "the cuts and their level arithmetic use one bin width");
constexpr uint32_t kBias = 0x80000000u;
constexpr uint32_t kQNaN32 = 0x7FC00000u;
constexpr uint32_t kNegInf32 = 0xFF800000u;

// 16 bytes of a row: one vector load per lane.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

// ---------------------------------------------------------------- keys
__device__ __forceinline__ uint32_t key_of_bits(uint32_t b) {
  const uint32_t mag = b & 0x7FFFFFFFu;
  return (b & 0x80000000u) ? kBias - mag : kBias + mag;
}

// Inverse of key_of_bits for keys of non-NaN values ([0x00800000, 0xFF800000]);
// the key of both zeros gives +0.0.
__device__ __forceinline__ uint32_t bits_of_key(uint32_t key) {
  return key >= kBias ? key - kBias : ((kBias - key) | 0x80000000u);
}

__device__ __forceinline__ u64 comp_of(uint32_t key, uint32_t col) {
  return (static_cast<u64>(key) << 32) | static_cast<uint32_t>(~col);
}
__device__ __forceinline__ uint32_t key_of(u64 c) { return static_cast<uint32_t>(c >> 32); }
__device__ __forceinline__ uint32_t col_of(u64 c) { return ~static_cast<uint32_t>(c); }

// T = -inf with "greater or equal": just below the key of -inf, all columns.
constexpr u64 kThrInit = (static_cast<u64>(0x00800000u - 1u) << 32) | 0xFFFFFFFFull;
constexpr uint32_t kNegInfKey = 0x00800000u;   // key of -inf, the lowest of any non-NaN value

// The threshold in the form the filter uses: admit v iff v > f, or v == f and
// column < idx_lim.  With idx_lim == ~0u this is simply v >= f.
struct Filter {
  float f;
  uint32_t idx_lim;
};

__device__ __forceinline__ Filter filter_of(u64 thr) {
  const uint32_t K = static_cast<uint32_t>(thr >> 32);
  const uint32_t low = static_cast<uint32_t>(thr);
  if (low == 0xFFFFFFFFu) return {__uint_as_float(bits_of_key(K + 1u)), 0xFFFFFFFFu};
  return {__uint_as_float(bits_of_key(K)), ~low};
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ u64 ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t mbcnt64(u64 m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// A value every lane holds the same copy of (read from LDS after a barrier,
// say), moved to a scalar register so that branches on it are scalar.
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}
__device__ __forceinline__ u64 uniform64(u64 v) {
  return (static_cast<u64>(uniform(static_cast<uint32_t>(v >> 32))) << 32) |
         uniform(static_cast<uint32_t>(v));
}

// DPP move: lanes whose source is outside the row, or whose row is masked off,
// receive IDENT.
template <int CTRL, int ROW_MASK, uint32_t IDENT>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(IDENT), static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Inclusive scan over the 64 lanes of a wave (all lanes active): row_shr
// 1/2/4/8 inside each 16-lane row, then row_bcast 15 and 31 across rows.
template <typename Op, uint32_t IDENT>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, Op op) {
  x = op(x, dpp<0x111, 0xF, IDENT>(x));
  x = op(x, dpp<0x112, 0xF, IDENT>(x));
  x = op(x, dpp<0x114, 0xF, IDENT>(x));
  x = op(x, dpp<0x118, 0xF, IDENT>(x));
  x = op(x, dpp<0x142, 0xA, IDENT>(x));
  x = op(x, dpp<0x143, 0xC, IDENT>(x));
  return x;
}

struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };

__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  return wave_scan<OpAdd, 0u>(x, OpAdd{});
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(wave_scan<OpMax, 0u>(x, OpMax{})), 63));
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(
      static_cast<int>(wave_scan<OpMin, 0xFFFFFFFFu>(x, OpMin{})), 63));
}

template <int CTRL, int ROW_MASK, u64 IDENT>
__device__ __forceinline__ u64 dpp64(u64 v) {
  const uint32_t lo = dpp<CTRL, ROW_MASK, static_cast<uint32_t>(IDENT)>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp<CTRL, ROW_MASK, static_cast<uint32_t>(IDENT >> 32)>(static_cast<uint32_t>(v >> 32));
  return (static_cast<u64>(hi) << 32) | lo;
}

template <bool MAX>
__device__ __forceinline__ u64 wave_extreme64(u64 x) {
  constexpr u64 I = MAX ? 0ull : ~0ull;
  auto op = [](u64 a, u64 b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = op(x, dpp64<0x111, 0xF, I>(x));
  x = op(x, dpp64<0x112, 0xF, I>(x));
  x = op(x, dpp64<0x114, 0xF, I>(x));
  x = op(x, dpp64<0x118, 0xF, I>(x));
  x = op(x, dpp64<0x142, 0xA, I>(x));
  x = op(x, dpp64<0x143, 0xC, I>(x));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), 63));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), 63));
  return (static_cast<u64>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t bit_length(uint32_t v) { return v ? 32u - __clz(v) : 0u; }
__device__ __forceinline__ uint32_t bit_length64(u64 v) { return v ? 64u - __clzll(v) : 0u; }

__device__ __forceinline__ uint32_t shift_for_span(uint32_t span) {
  const uint32_t b = bit_length(span);
  return b > kRadixBits ? b - kRadixBits : 0u;
}

// ---------------------------------------------------------------- device-memory sharing
// Relaxed agent-scope accesses: coherent across the XCDs' L2 caches without
// any cache write-back or invalidate.
__device__ __forceinline__ u64 load_thr(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_thr(u64* p, u64 v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename W>
__device__ __forceinline__ void st_agent(W* p, W v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename W>
__device__ __forceinline__ W ld_agent(const W* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this wave has issued is complete.  Used
// before the arrival counter of a row moves: the survivors were written with
// agent-scope atomic stores, so once complete they are visible to the
// workgroup that reads them after seeing the counter.
__device__ __forceinline__ void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- block order
// A bijection on [0, nb): a mixing bijection on [0, 2^m) (odd multipliers and
// xor-shifts) restricted to [0, nb) by cycle walking.  Seeded per row.
struct BlockOrder {
  uint32_t nb, mask, c1, sh;
  bool ident;

  __device__ BlockOrder(uint32_t nb_, uint32_t seed, uint32_t row, bool in_order) {
    nb = nb_;
    ident = in_order || nb_ <= 2;
    const uint32_t m = nb_ <= 1 ? 1u : bit_length(nb_ - 1u);
    mask = m >= 32 ? 0xFFFFFFFFu : ((1u << m) - 1u);
    sh = (m + 1u) / 2u;
    uint32_t h = seed * 0x9E3779B9u ^ (row + 0x7F4A7C15u) * 0x85EBCA6Bu;
    h ^= h >> 16;
    h *= 0x7FEB352Du;
    h ^= h >> 15;
    c1 = h;
  }
  __device__ __forceinline__ uint32_t mix(uint32_t x) const {
    x = (x * 0x9E3779B1u + c1) & mask;
    x ^= x >> sh;
    x = (x * 0x85EBCA77u) & mask;
    x ^= x >> sh;
    return x;
  }
  __device__ __forceinline__ uint32_t operator()(uint32_t j) const {
    if (ident) return j;
    uint32_t y = mix(j);
    while (y >= nb) y = mix(y);
    return y;
  }
};

// ---------------------------------------------------------------- LDS
template <int CAP, int NT>
struct Smem {
  u64 comp[CAP];              // candidate composites
  alignas(16) uint32_t hist[kBins];   // zero whenever not in use
  uint32_t wsum[NT / 64];
  uint32_t res[5];
  uint32_t cnt[2];            // append counters; cur receives appends, cur^1 the next cut
  uint32_t snap[2][NT / 64];  // per-wave count after its last append, by step parity
  uint32_t hikey;             // upper bound of every candidate key
  uint32_t flags;             // row status bits
  uint32_t is_last;
  uint32_t nwork;             // epilogue sort: number of pending segments
  uint32_t nside;             // cut: members of a small boundary bin
  uint32_t kept;              // cut: candidates above the new threshold
  u64 rng[2];                 // epilogue sort: min / max order key of a segment
  u64 thr;                    // the workgroup's threshold (composite)
  u64 xv;                     // a cut's second answer: a bound with >= need2 candidates above
  uint32_t bt[5];             // first-block start: min key, max key, t0 key, t2 key, ring count
  u64 specmax;                // merge: the largest estimated start used on the row (0: none)
  u64 tvalid;                 // merge: the largest bound known to leave k of the row above it
  uint32_t n_cut;             // statistics: cuts made by this workgroup
  uint32_t n_reread;          // statistics: whole-row re-reads by this workgroup
};

// A thread's own run of BPT consecutive bins, read and written 16 bytes at a
// time (BPT is a multiple of 4): one wide access instead of BPT narrow ones
// that would all fall on a few LDS banks.
template <int BPT, int NT, int CAP>
__device__ __forceinline__ void own_bins_read(const Smem<CAP, NT>& sm, uint32_t (&h)[BPT]) {
  static_assert(BPT % 4 == 0, "bins per thread");
  const u32x4* p = reinterpret_cast<const u32x4*>(sm.hist + threadIdx.x * BPT);
#pragma unroll
  for (int i = 0; i < BPT / 4; ++i) {
    const u32x4 v = p[i];
    h[4 * i] = v.x;
    h[4 * i + 1] = v.y;
    h[4 * i + 2] = v.z;
    h[4 * i + 3] = v.w;
  }
}
template <int BPT, int NT, int CAP>
__device__ __forceinline__ void own_bins_write(Smem<CAP, NT>& sm, const uint32_t (&h)[BPT]) {
  u32x4* p = reinterpret_cast<u32x4*>(sm.hist + threadIdx.x * BPT);
#pragma unroll
  for (int i = 0; i < BPT / 4; ++i) p[i] = u32x4{h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]};
}
template <int BPT, int NT, int CAP>
__device__ __forceinline__ void own_bins_zero(Smem<CAP, NT>& sm) {
  u32x4* p = reinterpret_cast<u32x4*>(sm.hist + threadIdx.x * BPT);
#pragma unroll
  for (int i = 0; i < BPT / 4; ++i) p[i] = u32x4{0u, 0u, 0u, 0u};
}

// Suffix search over hist (higher bins first), which it leaves zeroed.  Finds
// b* with  sum_{b > b*} hist[b] < need <= sum_{b >= b*} hist[b].
// res = {b*, sum above b*, hist[b*], total}; res[0] = kBins when total < need.
// With need2 > 0 the same search for need2 goes to res[4] (kBins if none).
template <int NT, int CAP>
__device__ __forceinline__ void hist_find_top(Smem<CAP, NT>& sm, uint32_t need,
                                              uint32_t need2 = 0) {
  constexpr int BPT = kBins / NT;
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t h[BPT];
  own_bins_read<BPT>(sm, h);
  own_bins_zero<BPT>(sm);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) s += h[i];
  const uint32_t p = wave_prefix_sum(s);   // inclusive, within the wave
  if (lane == 63) sm.wsum[w] = p;
  if (t == 0) {
    sm.res[0] = kBins;
    sm.res[4] = kBins;
  }
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) {
    const uint32_t ws = sm.wsum[w2];
    tot += ws;
    if (w2 < w) before += ws;
  }
  const uint32_t excl_above = tot - (before + p);   // bins owned by threads > t
  const uint32_t incl_above = excl_above + s;
  if (excl_above < need && need <= incl_above) {
    uint32_t acc = excl_above;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (acc + h[i] >= need) {
        sm.res[0] = t * BPT + i;
        sm.res[1] = acc;
        sm.res[2] = h[i];
        break;
      }
      acc += h[i];
    }
  }
  if (need2 != 0 && excl_above < need2 && need2 <= incl_above) {
    uint32_t acc = excl_above;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (acc + h[i] >= need2) {
        sm.res[4] = t * BPT + i;
        break;
      }
      acc += h[i];
    }
  }
  if (t == 0) sm.res[3] = tot;
  __syncthreads();
}

// In place: hist[b] <- sum_{b' < b} hist[b'].  Returns the total.
template <int NT, int CAP>
__device__ __forceinline__ uint32_t hist_exclusive_scan(Smem<CAP, NT>& sm) {
  constexpr int BPT = kBins / NT;
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t h[BPT];
  own_bins_read<BPT>(sm, h);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) s += h[i];
  const uint32_t p = wave_prefix_sum(s);
  if (lane == 63) sm.wsum[w] = p;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) {
    const uint32_t ws = sm.wsum[w2];
    tot += ws;
    if (w2 < w) before += ws;
  }
  uint32_t run = before + p - s;
  uint32_t o[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    o[i] = run;
    run += h[i];
  }
  own_bins_write<BPT>(sm, o);
  __syncthreads();
  return tot;
}

template <int NT, int CAP>
__device__ __forceinline__ void hist_zero_own(Smem<CAP, NT>& sm) {
  own_bins_zero<kBins / NT>(sm);
}

// ---------------------------------------------------------------- the cut
// Candidates are visited in groups of G slots per thread (slot e of thread t
// is buffer position t + e * NT): a group's LDS reads are issued back to
// back, unconditionally at a clamped address, and waited for once.  Slots
// past the count read as 0, which is below every threshold and outside every
// key range.  Whole groups of 16 are followed by one last group of 4, 8 or 16
// slots, whichever covers the rest, so a short buffer is not read 16 deep.
constexpr int kGroup = 16;

template <int G>
struct GroupSize {
  static constexpr int value = G;
};

template <int NT, typename Body>
__device__ __forceinline__ void for_groups(uint32_t c, Body&& body) {
  const uint32_t slots = (c + NT - 1) / NT;   // uniform
  uint32_t e0 = 0;
#pragma unroll 1
  for (; e0 + kGroup < slots; e0 += kGroup) body(GroupSize<kGroup>{}, e0);
  const uint32_t rest = slots - e0;
  if (rest > 8) body(GroupSize<16>{}, e0);
  else if (rest > 4) body(GroupSize<8>{}, e0);
  else if (rest > 0) body(GroupSize<4>{}, e0);
}

template <int G, int NT, int CAP>
__device__ __forceinline__ void read_group(const Smem<CAP, NT>& sm, uint32_t e0, uint32_t c,
                                           u64 (&v)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t i = threadIdx.x + (e0 + g) * NT;
    v[g] = sm.comp[i < CAP ? i : CAP - 1];
  }
  // All reads are issued before any result is used; without this fence the
  // scheduler can give every read the same destination and wait for each.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t i = threadIdx.x + (e0 + g) * NT;
    v[g] = i < c ? v[g] : 0ull;
  }
}

// Among the candidates with key E_key and composite > T, the column of the
// need-th smallest column (need >= 1 and at least need such candidates).  At
// most three levels (31-bit columns); if a level's counts disagree with the
// cut's (no buffer can make them), the row is flagged DS_ROW_INTERNAL and
// the top of the current range is returned, so the loop always ends.
template <int NT, int CAP>
__device__ __noinline__ uint32_t index_cut(Smem<CAP, NT>& sm, uint32_t c, uint32_t E_key,
                                           uint32_t need, u64 T, uint32_t n_cols) {
  RangeLevel lv{0u, n_cols > 0 ? n_cols - 1u : 0u, need, 0};
  for (int it = 0; it < RangeLevel::kMaxLevels; ++it) {
    const uint32_t shift = lv.shift();
    const uint32_t ibase = lv.base, span = lv.top - lv.base;
    for_groups<NT>(c, [&](auto gs, uint32_t e0) {
      constexpr int G = decltype(gs)::value;
      u64 v[G];
      read_group<G>(sm, e0, c, v);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t ci = col_of(v[g]) - ibase;
        if ((key_of(v[g]) == E_key) & (ci <= span) & (v[g] > T))
          atomicAdd(&sm.hist[(kBins - 1) - (ci >> shift)], 1u);
      }
    });
    __syncthreads();
    hist_find_top(sm, lv.need);
    // Bin in ascending column order (wraps past the bins when none was found,
    // which narrow() refuses).
    const uint32_t b = (kBins - 1) - uniform(sm.res[0]);
    const uint32_t below = uniform(sm.res[1]), bc = uniform(sm.res[2]);
    if (!lv.narrow(b, below, bc)) break;
    if (bc == lv.need) return lv.top;   // the whole bin is taken
    if (lv.single()) return lv.base;
  }
  if (threadIdx.x == 0) atomicOr(&sm.flags, static_cast<uint32_t>(DS_ROW_INTERNAL));
  __syncthreads();
  return lv.top;
}

// Compaction into counter `nxt`, one group of slots at a time: all threads
// read the group, then the kept entries (composite > keep_above) go to
// positions reserved with one LDS atomic per wave.  The write cursor never
// passes the number of positions read so far, so a write never lands on an
// unread entry.  With SIDE, the members of a small boundary bin
// (side_lo < composite <= keep_above) go to the idle, zero histogram memory,
// counted in sm.nside.
template <int NT, int CAP, bool SIDE>
__device__ __forceinline__ void compact_buffer(Smem<CAP, NT>& sm, uint32_t c, int nxt,
                                               u64 keep_above, u64 side_lo) {
  const int lane = threadIdx.x & 63;
  u64* side = reinterpret_cast<u64*>(sm.hist);
  if (SIDE && threadIdx.x == 0) sm.nside = 0u;
  for_groups<NT>(c, [&](auto gs, uint32_t e0) {
    constexpr int G = decltype(gs)::value;
    u64 v[G];
    read_group<G>(sm, e0, c, v);
    u64 mk[G], ms[G];
    uint32_t total = 0, nsd = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mk[g] = ballot(v[g] > keep_above);
      total += static_cast<uint32_t>(__popcll(mk[g]));
      if (SIDE) {
        ms[g] = ballot((v[g] > side_lo) & (v[g] <= keep_above));
        nsd += static_cast<uint32_t>(__popcll(ms[g]));
      }
    }
    __syncthreads();
    if (total) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&sm.cnt[nxt], total);
      base = uniform(base);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if ((mk[g] >> lane) & 1ull) sm.comp[base + mbcnt64(mk[g])] = v[g];
        base += static_cast<uint32_t>(__popcll(mk[g]));
      }
    }
    if (SIDE && nsd) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&sm.nside, nsd);
      base = uniform(base);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if ((ms[g] >> lane) & 1ull) side[base + mbcnt64(ms[g])] = v[g];
        base += static_cast<uint32_t>(__popcll(ms[g]));
      }
    }
  });
}

constexpr uint32_t kSmallBin = 64;   // largest boundary bin ranked directly
static_assert(kSmallBin == static_cast<uint32_t>(kStreamSlotSlack), "survivor slots per workgroup: k + kSmallBin");
constexpr int kSmallCutG = 4;   // candidates per thread of the small cut
// small_cut: candidates per thread, within the buffer's room
constexpr int small_cut_g(int cap, int nt) {
  return kSmallCutG * nt + static_cast<int>(kSmallBin) <= cap ? kSmallCutG
                                                               : (cap - static_cast<int>(kSmallBin)) / nt;
}

// The n = sm.nside (<= kSmallBin) members of a small boundary bin sit in the
// histogram memory as composites.  Each wave counts, for every member, how
// many members of its share are larger; the member with exactly need - 1
// larger members is the last one kept (composites are distinct).  Kept
// members are appended to counter `nxt`.  Returns the new threshold and
// leaves the histogram memory zeroed.
template <int NT, int CAP>
__device__ __noinline__ u64 resolve_small_bin(Smem<CAP, NT>& sm, int nxt, uint32_t need) {
  constexpr int NW = NT / 64;
  constexpr uint32_t PART = (kSmallBin + NW - 1) / NW;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  u64* side = reinterpret_cast<u64*>(sm.hist);
  uint32_t* rank = sm.hist + 2 * kSmallBin;   // kSmallBin counters, zero
  __syncthreads();
  const uint32_t n = uniform(sm.nside);
  const u64 mine = side[static_cast<uint32_t>(lane) < n ? lane : 0];
  u64 other[PART];
#pragma unroll
  for (uint32_t j = 0; j < PART; ++j) {
    const uint32_t q = w * PART + j;
    other[j] = side[q < n ? q : 0];
  }
  uint32_t r = 0;
#pragma unroll
  for (uint32_t j = 0; j < PART; ++j) r += ((w * PART + j < n) & (other[j] > mine)) ? 1u : 0u;
  if (static_cast<uint32_t>(lane) < n && r) atomicAdd(&rank[lane], r);
  __syncthreads();
  if (w == 0 && static_cast<uint32_t>(lane) < n && rank[lane] + 1u == need) sm.rng[0] = mine;
  __syncthreads();
  const u64 kth = uniform64(sm.rng[0]);
  if (w == 0) {
    const bool keep = (static_cast<uint32_t>(lane) < n) & (mine >= kth);
    const u64 m = ballot(keep);
    uint32_t base = 0;
    if (lane == 0 && m) base = atomicAdd(&sm.cnt[nxt], static_cast<uint32_t>(__popcll(m)));
    base = uniform(base);
    if (keep) sm.comp[base + mbcnt64(m)] = mine;
  }
  __syncthreads();
  for (uint32_t j = t; j < 3 * kSmallBin; j += NT) sm.hist[j] = 0u;
  return kth - 1u;
}

// Cut the candidate buffer: keep every candidate with composite > T_new, where
// T_new >= sm.thr leaves between k and keep_max candidates (or all of them if
// no more than keep_max are above sm.thr).  keep_max == k gives the exact
// top-k.  Returns the new append counter index.
// With need2 > 0 it also leaves in sm.xv a composite with at least need2 of
// the candidates above it (0 if there are fewer than need2 above sm.thr).
// sm.kept receives the number of candidates above the new threshold.  With
// find_only the buffer is left as it is (the caller reads it filtered by
// sm.thr); keep_max must then be at least k + kSmallBin, so that a boundary
// bin small enough to rank is always kept whole.
template <int NT, int CAP>
__device__ __noinline__ int cut_buffer(Smem<CAP, NT>& sm, int cur, uint32_t k,
                                       uint32_t keep_max, uint32_t n_cols, uint32_t hi_key,
                                       uint32_t need2 = 0, bool find_only = false) {
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t hk = wave_max(hi_key);
  if (lane == 0) atomicMax(&sm.hikey, hk);
  if (t == 0) {
    sm.cnt[cur ^ 1] = 0u;
    sm.n_cut += 1u;
  }
  __syncthreads();
  const uint32_t c = min(uniform(sm.cnt[cur]), static_cast<uint32_t>(CAP));
  const u64 T = uniform64(sm.thr);
  const uint32_t hi = uniform(sm.hikey);
  const uint32_t K = static_cast<uint32_t>(T >> 32);
  const bool key_only = static_cast<uint32_t>(T) == 0xFFFFFFFFu;   // T = "key >= K + 1"
  const uint32_t klo = key_only ? K + 1u : K;

  u64 newT = T;
  u64 xv = 0;
  uint32_t kept = 0;
  // Small boundary bin: its members (composite in (sb_lo, newT]) are
  // collected during the compaction and ranked exactly; the sb_need-th
  // largest of them is the last one kept.
  bool small = false;
  bool keep_all = false;   // every candidate is above T and kept: no compaction
  u64 sb_lo = 0;
  uint32_t sb_need = 0;
  bool err = false;   // a level's counts disagreed with the previous level's
  if (hi >= klo && c > 0) {
    RangeLevel lv{klo, hi, k, 0};
    uint32_t above = 0;
    bool first = true;
    for (int it = 0; it <= RangeLevel::kMaxLevels; ++it) {
      if (it == RangeLevel::kMaxLevels) {   // no 32-bit range needs another level
        err = true;
        break;
      }
      const uint32_t shift = lv.shift();
      const uint32_t base = lv.base, top = lv.top;
      const uint32_t span = top - base;
      const uint32_t need = lv.need;
      for_groups<NT>(c, [&](auto gs, uint32_t e0) {
        constexpr int G = decltype(gs)::value;
        u64 v[G];
        read_group<G>(sm, e0, c, v);
        if (key_only) {   // every candidate in [base, top] is above T
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint32_t d = key_of(v[g]) - base;
            if (d <= span) atomicAdd(&sm.hist[d >> shift], 1u);
          }
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint32_t d = key_of(v[g]) - base;
            if ((d <= span) & (v[g] > T)) atomicAdd(&sm.hist[d >> shift], 1u);
          }
        }
      });
      __syncthreads();
      hist_find_top(sm, need, first ? need2 : 0u);
      if (first) {
        first = false;
        if (need2 != 0) {
          const uint32_t b2 = uniform(sm.res[4]);
          if (b2 < static_cast<uint32_t>(kBins)) xv = (static_cast<u64>(base + (b2 << shift)) << 32) - 1u;
        }
        const uint32_t above_T = uniform(sm.res[3]);
        if (above_T <= keep_max) {   // few enough above T: only drop those at or below T
          keep_all = above_T == c;
          kept = above_T;
          break;
        }
      }
      const uint32_t b = uniform(sm.res[0]), ab = uniform(sm.res[1]), bc = uniform(sm.res[2]);
      if (!lv.narrow(b, ab, bc)) {
        err = true;
        break;
      }
      above += ab;
      const u64 lo_edge = (static_cast<u64>(lv.base) << 32) - 1u;
      if (above + bc <= keep_max) {
        newT = lo_edge > T ? lo_edge : T;
        kept = above + bc;
        break;
      }
      if (bc <= kSmallBin) {
        // Keys of the bin are [base, ub]: the bin's width, capped at the top
        // of the range this level divides (keys above it were counted in
        // higher bins before).  ub + 1 fits in 32 bits for any non-NaN key.
        // Everything above the bin is kept outright.
        const uint32_t ub = lv.top;
        small = true;
        sb_lo = lo_edge > T ? lo_edge : T;
        sb_need = lv.need;
        kept = above + lv.need;
        newT = (static_cast<u64>(ub + 1u) << 32) - 1u;
        break;
      }
      if (lv.single()) {
        const uint32_t I = index_cut<NT, CAP>(sm, c, lv.base, lv.need, T, n_cols);
        if (uniform(sm.flags) & static_cast<uint32_t>(DS_ROW_INTERNAL)) {
          err = true;
          break;
        }
        const u64 cand = comp_of(lv.base, I) - 1u;
        newT = cand > T ? cand : T;
        kept = above + lv.need;
        break;
      }
    }
  }
  if (err) {
    // The row is flagged and its buffer emptied (the threshold stays), so no
    // later append can overflow it; the row's outputs become -1 / qNaN.
    if (t == 0) {
      atomicOr(&sm.flags, static_cast<uint32_t>(DS_ROW_INTERNAL));
      sm.thr = T;
      sm.xv = 0;
      sm.kept = 0;
    }
    __syncthreads();
    return cur ^ 1;   // sm.cnt[cur ^ 1] was set to zero above
  }

  int nxt = cur ^ 1;
  if (keep_all || find_only) {
    nxt = cur;
  } else if (small) {
    compact_buffer<NT, CAP, true>(sm, c, nxt, newT, sb_lo);
    newT = resolve_small_bin<NT, CAP>(sm, nxt, sb_need);
  } else {
    compact_buffer<NT, CAP, false>(sm, c, nxt, newT, 0ull);
  }
  if (t == 0) {
    sm.thr = newT;
    sm.xv = xv;
    sm.kept = kept;
  }
  __syncthreads();
  return nxt;
}

// The exact top-k of a buffer of at most G * NT candidates (k of those above
// sm.thr are kept, the rest dropped), in four barriers where cut_buffer needs
// about nine.  Every thread holds its G candidates in registers, so the
// compaction may overwrite the buffer in place.  One histogram of 256 bins
// over [lowest key above sm.thr, sm.hikey], which every wave scans for
// itself, finds the boundary bin; everything above it is kept, and the bin's
// members (at most kSmallBin) are ranked by one wave, which keeps the top
// ones.  A larger boundary bin, or no more than k candidates above sm.thr,
// falls back to cut_buffer.  sm.hikey must bound every candidate's key.
template <int G, int NT, int CAP>
__device__ __forceinline__ int small_cut(Smem<CAP, NT>& sm, int cur, uint32_t k, uint32_t n_cols,
                                         uint32_t hi_key) {
  static_assert(G * NT + static_cast<int>(kSmallBin) <= CAP, "small cut room");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nxt = cur ^ 1;
  if (t == 0) sm.n_cut += 1u;
  const uint32_t c = min(uniform(sm.cnt[cur]), static_cast<uint32_t>(CAP));
  const u64 T = uniform64(sm.thr);
  const uint32_t hi = uniform(sm.hikey);
  const uint32_t K = static_cast<uint32_t>(T >> 32);
  const uint32_t klo = static_cast<uint32_t>(T) == 0xFFFFFFFFu ? K + 1u : K;   // lowest key above T
  const uint32_t span = hi - klo;
  const uint32_t sh = bit_length(span) > 8u ? bit_length(span) - 8u : 0u;
  auto bin_of = [&](u64 v) -> uint32_t {
    const uint32_t d = key_of(v) - klo;
    return (d < span ? d : span) >> sh;
  };
  u64 v[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t i = static_cast<uint32_t>(t + g * NT);
    v[g] = i < c ? sm.comp[i] : 0ull;
    v[g] = v[g] > T ? v[g] : 0ull;   // 0 is never above T
  }
  const bool usable = (hi >= klo) & (c > k);
  if (usable) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (v[g] != 0ull) atomicAdd(&sm.hist[bin_of(v[g])], 1u);
  }
  if (t == 0) {
    sm.cnt[nxt] = 0u;
    sm.nside = 0u;
  }
  __syncthreads();
  // Bins 4 lane .. 4 lane + 3 per lane, suffix counts from the top: the bin b
  // with fewer than k candidates above it and at least k at or above it.
  uint32_t b = 0, ab = 0, bc = 0;
  bool found = false;
  if (usable) {
    const u32x4 hb = reinterpret_cast<const u32x4*>(sm.hist)[lane];
    const uint32_t h4[4] = {hb.x, hb.y, hb.z, hb.w};
    const uint32_t s4 = hb.x + hb.y + hb.z + hb.w;
    const uint32_t incl = wave_prefix_sum(s4);
    const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
    const uint32_t above = total - incl;
    const u64 hit = ballot((above < k) & (above + s4 >= k));
    if (hit) {
      const int hl = static_cast<int>(__ffsll(static_cast<long long>(hit))) - 1;
      uint32_t lb = 0, lab = 0, lbc = 0, acc = above;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if ((acc < k) & (acc + h4[i] >= k)) {
          lb = 4u * static_cast<uint32_t>(lane) + static_cast<uint32_t>(i);
          lab = acc;
          lbc = h4[i];
        }
        acc += h4[i];
      }
      b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lb), hl));
      ab = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lab), hl));
      bc = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lbc), hl));
      found = bc <= kSmallBin;
    }
  }
  if (!found) {   // nothing written yet: clear the bins and cut the general way
    __syncthreads();
    for (uint32_t j = t; j < 256u; j += NT) sm.hist[j] = 0u;
    return cut_buffer<NT, CAP>(sm, cur, k, k, n_cols, hi_key);
  }
  const uint32_t need = k - ab;   // 1 <= need <= bc
  const bool whole = need == bc;  // the boundary bin is kept whole
  u64* side = sm.comp + (CAP - static_cast<int>(kSmallBin));
  {
    u64 mk[G], ms[G];
    uint32_t nk = 0, ns = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t bn = bin_of(v[g]);
      const bool live = v[g] != 0ull;
      mk[g] = ballot(live & ((bn > b) | (whole & (bn == b))));
      ms[g] = ballot(live & !whole & (bn == b));
      nk += static_cast<uint32_t>(__popcll(mk[g]));
      ns += static_cast<uint32_t>(__popcll(ms[g]));
    }
    uint32_t kb = 0, sb = 0;
    if (lane == 0) {
      if (nk) kb = atomicAdd(&sm.cnt[nxt], nk);
      if (ns) sb = atomicAdd(&sm.nside, ns);
    }
    kb = uniform(kb);
    sb = uniform(sb);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if ((mk[g] >> lane) & 1ull) sm.comp[kb + mbcnt64(mk[g])] = v[g];
      if ((ms[g] >> lane) & 1ull) side[sb + mbcnt64(ms[g])] = v[g];
      kb += static_cast<uint32_t>(__popcll(mk[g]));
      sb += static_cast<uint32_t>(__popcll(ms[g]));
    }
  }
  if (whole && t == 0) {
    const u64 lo_edge = (static_cast<u64>(klo + (b << sh)) << 32) - 1u;
    sm.thr = lo_edge > T ? lo_edge : T;
  }
  __syncthreads();   // every wave has scanned the bins and appended
  for (uint32_t j = t; j < 256u; j += NT) sm.hist[j] = 0u;
  if (!whole && w == 0) {
    // Composites are distinct: the member with need - 1 larger members is the
    // last one kept.
    const uint32_t n = bc;
    const u64 mine = static_cast<uint32_t>(lane) < n ? side[lane] : 0ull;
    uint32_t r = 0;
    for (uint32_t j = 0; j < n; ++j) r += side[j] > mine ? 1u : 0u;
    const bool in = static_cast<uint32_t>(lane) < n;
    const u64 m = ballot(in & (r < need));
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&sm.cnt[nxt], static_cast<uint32_t>(__popcll(m)));
    base = uniform(base);
    if ((m >> lane) & 1ull) sm.comp[base + mbcnt64(m)] = mine;
    const u64 last = ballot(in & (r + 1u == need));
    const int ll = static_cast<int>(__ffsll(static_cast<long long>(last))) - 1;
    const u64 kth = static_cast<u64>(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                        static_cast<int>(static_cast<uint32_t>(mine >> 32)), ll)))
                        << 32 |
                    static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(mine)), ll));
    if (lane == 0) sm.thr = kth - 1u;
  }
  if (t == 0) {
    sm.kept = k;
    sm.xv = 0ull;
  }
  __syncthreads();
  return nxt;
}
// The same out of line.  The merge inlines the cut for k <= 1024, where
// nearly every shared row's buffer fits it; for larger k the inlined body
// would only add code to the kernel around a cut that rarely applies.
template <int G, int NT, int CAP>
__device__ __noinline__ int small_cut_call(Smem<CAP, NT>& sm, int cur, uint32_t k, uint32_t n_cols,
                                           uint32_t hi_key) {
  return small_cut<G, NT, CAP>(sm, cur, k, n_cols, hi_key);
}

// ---------------------------------------------------------------- the filter
// Filter one block held in registers and append its survivors.  Returns the
// append counter as this wave left it (0 if the wave appended nothing).
template <bool BF16, bool RAG, int V, int NT, int CAP>
__device__ __forceinline__ uint32_t filter_block(const u32x4 (&r)[V], uint32_t blk, uint32_t L,
                                                 const Filter& F, float& hi_lane, bool& nan_lane,
                                                 Smem<CAP, NT>& sm, int cur) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NS = V * EPV;
  const int t = threadIdx.x, lane = t & 63;
  float f[NS];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint32_t w[4] = {r[v].x, r[v].y, r[v].z, r[v].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (BF16) {
        f[v * 8 + 2 * q] = __uint_as_float(w[q] << 16);
        f[v * 8 + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      } else {
        f[v * 4 + q] = __uint_as_float(w[q]);
      }
    }
  }
  const uint32_t base_idx = blk * static_cast<uint32_t>(kBlockElems) + t * EPV;
  auto col = [&](int s) { return base_idx + static_cast<uint32_t>((s / EPV) * (NT * EPV) + (s % EPV)); };
  if (RAG) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bool valid = col(s) < L;
      nan_lane |= valid & (f[s] != f[s]);
      if (!valid) f[s] = __uint_as_float(kQNaN32);
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS; s += 2) nan_lane |= __builtin_isunordered(f[s], f[s + 1]);
  }
  // The threshold is the same in every lane; reading it into scalar registers
  // lets the compiler see that, so the per-element wave masks below stay
  // scalar and each store reuses its compare as the execution mask.
  const float ff = __uint_as_float(uniform(__float_as_uint(F.f)));
  const uint32_t lim = uniform(F.idx_lim);
  float mx = f[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) mx = fmaxf(mx, f[s]);
  hi_lane = fmaxf(hi_lane, mx);
  if (!ballot(mx >= ff)) return 0u;

  // Admission test: f >= ff when the threshold is a key bound (lim = ~0u, the
  // usual case), else branch-free f > ff or f == ff at a lower column.  A NaN
  // never passes.  The wave masks give the block's total and each store's
  // position; the test itself is repeated as each store's execution mask.
  const uint32_t ncol0 = ~base_idx;   // ~col(s) = ncol0 - (col(s) - base_idx)
  auto run = [&](auto key_only, auto positive) -> uint32_t {
    auto pass = [&](int s) -> bool {
      if (decltype(key_only)::value) return f[s] >= ff;
      return (f[s] > ff) | ((f[s] == ff) & (col(s) < lim));
    };
    u64 m[NS];
    uint32_t total = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      m[s] = ballot(pass(s));
      total += static_cast<uint32_t>(__popcll(m[s]));
    }
    if (total == 0) return 0u;
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&sm.cnt[cur], total);
    base = uniform(base);
    const uint32_t after = base + total;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (pass(s)) {
        const uint32_t bits = __float_as_uint(f[s]);
        // Above a positive threshold every admitted value is positive, and
        // the key of a positive value is its bit pattern with the top bit set.
        const uint32_t key = decltype(positive)::value ? (bits | kBias) : key_of_bits(bits);
        const uint32_t pos = __builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m[s] >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m[s]), base));
        const uint32_t off = static_cast<uint32_t>((s / EPV) * (NT * EPV) + (s % EPV));
        sm.comp[pos] = (static_cast<u64>(key) << 32) | (ncol0 - off);
      }
      base += static_cast<uint32_t>(__popcll(m[s]));
    }
    return after;
  };
  const bool positive = ff > 0.0f;
  if (lim == 0xFFFFFFFFu)
    return positive ? run(std::true_type{}, std::true_type{}) : run(std::true_type{}, std::false_type{});
  return positive ? run(std::false_type{}, std::true_type{}) : run(std::false_type{}, std::false_type{});
}

template <int V>
struct BlockRegs {
  u32x4 v[V];
};

struct RaggedResult {
  uint32_t after;
  float hi_lane;
  uint32_t nan_lane;
};

// The row's last, partial block: the same filter with every column checked
// against L.  Out of line (once per row); everything goes in and out by value,
// so the caller's running maximum and NaN flag stay in registers (an address
// taken would put them in scratch memory, whose loads share the counter of
// the block loads in flight).
template <bool BF16, int V, int NT, int CAP>
__device__ __noinline__ RaggedResult filter_ragged(BlockRegs<V> r, uint32_t blk, uint32_t L,
                                                   Filter F, float hi_lane, uint32_t nan_lane,
                                                   Smem<CAP, NT>& sm, int cur) {
  bool nl = nan_lane != 0;
  const uint32_t after = filter_block<BF16, true, V, NT, CAP>(r.v, blk, L, F, hi_lane, nl, sm, cur);
  return {after, hi_lane, nl ? 1u : 0u};
}

// Starting thresholds from whole blocks held in registers, before any of
// them is appended (used for the three-block start of k above half a
// block; one block uses the per-wave version below).  The values are binned
// linearly between their finite minimum and maximum (2048 bins; -inf and
// +inf clamp to the end bins, NaN is left out).  Linear bins spread the
// usual bell-shaped scores over many bins, so the LDS atomics rarely
// collide, where bins on the key bits would pile most of a binade into a
// few.  The suffix search finds the bin b* with at least k elements in bins
// >= b*; since the binning never decreases with the value, a value that
// bins below b* lies below all of those elements, and its key is a
// threshold with at least k of the blocks' elements above it -- a valid
// (monotone) starting point for the row (t0).  With need2 > 0 the same
// search for need2 gives t2, with at least need2 of the elements above it:
// only an estimate for the row, which the caller must verify.  Leaves hist
// zeroed.  Its reductions use bt[0..1], set at the kernel's start (it runs
// at most once per workgroup).
struct ThrPair {
  u64 t0, t2;
};
template <bool BF16, int V, int NT, int CAP>
__device__ __forceinline__ ThrPair block_threshold_body(const BlockRegs<V>& r, uint32_t k,
                                                        uint32_t need2, Smem<CAP, NT>& sm) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NS = V * EPV;
  const int t = threadIdx.x, lane = t & 63;
  float f[NS];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = r.v[v][q];
      if (BF16) {
        f[v * 8 + 2 * q] = __uint_as_float(w << 16);
        f[v * 8 + 2 * q + 1] = __uint_as_float(w & 0xFFFF0000u);
      } else {
        f[v * 4 + q] = __uint_as_float(w);
      }
    }
  }
  // finite range in floats, turned into the order-preserving keys once per
  // lane (a lane with no finite value gives +inf / -inf, which lose)
  float flo = __uint_as_float(0x7F800000u), fhi = __uint_as_float(kNegInf32);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool fin = __builtin_fabsf(f[s]) <= 3.402823466e38f;
    flo = fin ? __builtin_fminf(flo, f[s]) : flo;
    fhi = fin ? __builtin_fmaxf(fhi, f[s]) : fhi;
  }
  uint32_t klo = wave_min(key_of_bits(__float_as_uint(flo)));
  uint32_t khi = wave_max(key_of_bits(__float_as_uint(fhi)));
  if (lane == 0) {   // bt[] was set at the kernel's start
    atomicMin(&sm.bt[0], klo);
    atomicMax(&sm.bt[1], khi);
  }
  __syncthreads();
  klo = uniform(sm.bt[0]);
  khi = uniform(sm.bt[1]);
  if (khi < klo) {   // no finite value in the block
    __syncthreads();
    return {kThrInit, kThrInit};
  }
  const float lo = __uint_as_float(bits_of_key(klo));
  const float hi = __uint_as_float(bits_of_key(khi));
  const float span = hi - lo;   // may be +inf for extreme ranges: then scale 0, one bin
  const float scale = span > 0.0f ? static_cast<float>(kBins - 1) / span : 0.0f;
  auto bin_of = [&](float x) -> uint32_t {
    // fmaxf / fminf drop a NaN product (inf * 0) in favour of the bound
    const float y = __builtin_fminf(__builtin_fmaxf((x - lo) * scale, 0.0f),
                                    static_cast<float>(kBins - 1));
    return static_cast<uint32_t>(y);
  };
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (f[s] == f[s]) atomicAdd(&sm.hist[bin_of(f[s])], 1u);
  __syncthreads();
  hist_find_top(sm, k, need2);
  const uint32_t b = uniform(sm.res[0]);
  const uint32_t b2 = need2 ? uniform(sm.res[4]) : static_cast<uint32_t>(kBins);
  if (b >= static_cast<uint32_t>(kBins)) return {kThrInit, kThrInit};   // fewer than k non-NaN values
  // A key at or below every member of bins >= bb: the middle of bin bb - 1,
  // confirmed by binning it (bin_of never decreases as x grows, so every
  // value binned at bb or above is strictly greater).  Bin 0 holds every
  // non-NaN value (and -inf), as does a middle that does not bin below bb:
  // the lowest key.
  auto below_bin = [&](uint32_t bb) -> uint32_t {
    if (bb == 0u) return kNegInfKey;
    const float mid = lo + (static_cast<float>(bb) - 0.5f) * (span / static_cast<float>(kBins - 1));
    return bin_of(mid) < bb ? key_of_bits(__float_as_uint(mid)) : kNegInfKey;
  };
  const u64 t0 = (static_cast<u64>(below_bin(b)) << 32) - 1u;
  const u64 t2 = b2 < static_cast<uint32_t>(kBins) ? (static_cast<u64>(below_bin(b2)) << 32) - 1u : kThrInit;
  return {t0, t2};
}
// The same starting thresholds with one barrier, for one block: each of the
// NW waves bins
// its own values linearly between their finite minimum and maximum, into
// its own 256 bins (hist[256 w, 256 w + 256)), and finds with a wave scan
// the highest bin b with ceil(k / NW) of its values in bins >= b; its edge is
// a value that bins below b (so lies below all of them).  Every wave thus
// vouches for ceil(k / NW) values above its edge, so the smallest edge over
// the waves has NW ceil(k / NW) >= k values of the block(s) at or above it:
// t0, a valid start.  The waves' edges for ceil(need2 / NW) are combined by
// their lower median into the estimate t2 (the caller verifies it).  A wave
// with fewer than ceil(k / NW) finite values vouches for nothing, and then
// t0 = kThrInit.  Leaves hist zeroed.  Binning each wave's values on its
// own also keeps a rare outlier from stretching every bin: it widens one
// wave's bins, and the median passes over that wave's estimate.
template <bool BF16, int V, int NT, int CAP>
__device__ __forceinline__ ThrPair wave_threshold(const BlockRegs<V>& r, uint32_t k, uint32_t need2,
                                                  Smem<CAP, NT>& sm) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int NS = V * EPV;
  constexpr int NW = NT / 64;
  constexpr uint32_t kWaveBins = 256;
  static_assert(NW * kWaveBins <= kBins, "per-wave bins");
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t w = static_cast<uint32_t>(t) >> 6;
  const uint32_t kw = (k + NW - 1u) / NW;
  const uint32_t nw2 = need2 ? (need2 + NW - 1u) / NW : 0u;
  float f[NS];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x = r.v[v][q];
      if (BF16) {
        f[v * 8 + 2 * q] = __uint_as_float(x << 16);
        f[v * 8 + 2 * q + 1] = __uint_as_float(x & 0xFFFF0000u);
      } else {
        f[v * 4 + q] = __uint_as_float(x);
      }
    }
  }
  // The finite range in floats, turned into keys once per lane (keys order
  // like the values; both zeros share one key).
  float flo = __uint_as_float(0x7F800000u), fhi = __uint_as_float(kNegInf32);
  bool ninf = false;   // a -inf, which bin 0 holds below klo
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool fin = __builtin_fabsf(f[s]) <= 3.402823466e38f;
    flo = fin ? __builtin_fminf(flo, f[s]) : flo;
    fhi = fin ? __builtin_fmaxf(fhi, f[s]) : fhi;
    ninf |= f[s] == __uint_as_float(kNegInf32);
  }
  // No finite value in a lane: its +inf / -inf keys lose every min / max.
  uint32_t klo = wave_min(key_of_bits(__float_as_uint(flo)));
  uint32_t khi = wave_max(key_of_bits(__float_as_uint(fhi)));
  const bool any_ninf = ballot(ninf) != 0ull;
  uint32_t e0 = 0, e2 = 0xFFFFFFFFu;   // this wave's edges (keys); 0: vouches for nothing
  uint32_t* hw = sm.hist + w * kWaveBins;
  if (khi >= klo) {
    const float lo = __uint_as_float(bits_of_key(klo));
    const float hi = __uint_as_float(bits_of_key(khi));
    const float span = hi - lo;
    const float scale = span > 0.0f ? static_cast<float>(kWaveBins - 1) / span : 0.0f;
    auto bin_of = [&](float x) -> uint32_t {
      const float y = __builtin_fminf(__builtin_fmaxf((x - lo) * scale, 0.0f),
                                      static_cast<float>(kWaveBins - 1));
      return static_cast<uint32_t>(y);
    };
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (f[s] == f[s]) atomicAdd(&hw[bin_of(f[s])], 1u);
    // Bins 4 lane .. 4 lane + 3 of this wave; suffix counts from the top.
    // One wave's LDS accesses complete in the order issued, so its reads see
    // all of its atomics: no barrier, only no reordering by the compiler.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const u32x4 hb = reinterpret_cast<const u32x4*>(hw)[lane];
    reinterpret_cast<u32x4*>(hw)[lane] = u32x4{0u, 0u, 0u, 0u};
    const uint32_t h4[4] = {hb.x, hb.y, hb.z, hb.w};
    const uint32_t s4 = hb.x + hb.y + hb.z + hb.w;
    const uint32_t incl = wave_prefix_sum(s4);
    const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
    const uint32_t above = total - incl;   // in the bins of higher lanes
    auto edge_bin = [&](uint32_t need) -> uint32_t {   // highest b with >= need in bins >= b
      uint32_t b = 0xFFFFFFFFu, acc = above;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if ((acc < need) & (acc + h4[i] >= need)) b = 4u * static_cast<uint32_t>(lane) + static_cast<uint32_t>(i);
        acc += h4[i];
      }
      return wave_min(b);   // exactly one lane has it; 0xFFFFFFFF if total < need
    };
    const uint32_t b0 = edge_bin(kw);
    const uint32_t b2 = nw2 ? edge_bin(nw2) : 0xFFFFFFFFu;
    // A key at or below every member of bins >= b.  For b > 0: the middle
    // of bin b - 1, confirmed by binning it (bin_of never decreases as x
    // grows, so any x binned at b or above is strictly greater than a value
    // binned below b, and so is its key).  Bin 0 holds every non-NaN value:
    // the smallest finite key, or that of -inf if the wave holds one.  A
    // middle that does not bin below b gives the lowest key.
    auto below_bin = [&](uint32_t b) -> uint32_t {
      if (b == 0u) return any_ninf ? kNegInfKey : klo;
      const float mid = lo + (static_cast<float>(b) - 0.5f) * (span / static_cast<float>(kWaveBins - 1));
      return bin_of(mid) < b ? key_of_bits(__float_as_uint(mid)) : kNegInfKey;
    };
    if (b0 != 0xFFFFFFFFu) e0 = below_bin(b0);
    if (b2 != 0xFFFFFFFFu) e2 = below_bin(b2);
  }
  if (lane == 0) {
    sm.wsum[w] = e0;
    sm.snap[0][w] = e2;   // reused: no step has run yet
  }
  __syncthreads();
  // The same in every lane: combined in scalar registers.
  uint32_t lo0 = 0xFFFFFFFFu;
  uint32_t e2s[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t a0 = uniform(sm.wsum[i]);
    lo0 = a0 < lo0 ? a0 : lo0;
    e2s[i] = uniform(sm.snap[0][i]);
  }
  // lower median of the waves' estimates (a small sorting network)
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int j = 0; j + 1 < NW - i; ++j) {
      const uint32_t x = e2s[j], y = e2s[j + 1];
      e2s[j] = x < y ? x : y;
      e2s[j + 1] = x < y ? y : x;
    }
  const uint32_t med = e2s[(NW - 1) / 2];
  __syncthreads();   // wsum and snap are free again
  const u64 t0 = lo0 == 0u || lo0 == 0xFFFFFFFFu ? kThrInit : (static_cast<u64>(lo0) << 32) - 1u;
  const u64 t2 = (!nw2 || med == 0xFFFFFFFFu || med == 0u) ? kThrInit : (static_cast<u64>(med) << 32) - 1u;
  return {t0, t2};
}



// Loads of one block.  Always issued, whatever the block: a vector that would
// start at or past L reads the row's first vector instead (its lanes are
// discarded by the filter), so the compiler can count outstanding loads
// exactly.
template <bool BF16, int V, int NT>
__device__ __forceinline__ void load_block(u32x4 (&r)[V], const char* xrow, uint32_t blk,
                                           uint32_t L) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  const uint32_t e0 = blk * static_cast<uint32_t>(kBlockElems) + threadIdx.x * EPV;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    uint32_t e = e0 + v * NT * EPV;
    e = e < L ? e : 0u;
    r[v] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(xrow + static_cast<size_t>(e) * ESZ));
  }
}

// ---------------------------------------------------------------- epilogue
// Order the m results held in comp[0, m) (m <= MMAX).  The sort key
// (ascending = output order) is ~composite by value and the column by
// column; both are unique.  Every thread keeps the same elements in registers
// throughout and only their final positions are worked out, level by level:
//  * a level bins every still-unplaced element within its segment (a run of
//    final positions whose keys lie in [lo, lo + 2^bits)); the 2048 bins are
//    shared out among the segments in proportion to their sizes;
//  * a scan over the bins gives each bin its run of final positions, and the
//    elements are grouped there in a scratch region;
//  * an element in a bin of at most 32 is placed by its rank within the bin;
//    a larger bin becomes a segment of the next level, binned on the exact
//    minimum and maximum of its own keys (so a run of equal values, whose keys
//    differ only in the column, spreads out at once).
// Regions: R0 = comp[0, MMAX) receives the sorted output, R1 = comp[MMAX,
// 2 MMAX) holds the grouped elements, and after R1 come two segment tables
// (this level's and the next), 4 words of 64 bits per segment.
// Longest share (in blocks) of a shared row that may start from an estimate.
constexpr uint32_t kSpecSteps = 16;

constexpr int kSortSegs = 512;   // > 4096 / 9, the most segments a level can make
// A level ranks bins of up to 32 members directly, unless the ranking work of
// its bins of 9..32 members (the sum of their squared sizes) exceeds what
// another level costs: then those bins are split again too (runs of equal
// values make such bins, and the next level spreads them by column at once).
constexpr uint32_t kSplitWork = 6000;

template <int NT, int CAP, int MMAX>
__device__ __noinline__ void sort_results(Smem<CAP, NT>& sm, uint32_t m, bool by_value,
                                          u64 key_lo, uint32_t span_bits) {
  static_assert(2 * MMAX + 2 * 4 * kSortSegs <= CAP, "sort regions");
  constexpr int PER = MMAX / NT;          // elements per thread at most
  constexpr int RB = 4;                   // in-bin rank: members read per round
  constexpr uint32_t kDone = 0xFFFFu;
  const int t = threadIdx.x;
  u64* out = sm.comp;
  u64* grp = sm.comp + MMAX;
  // Two segment tables after R1, addressed by offset into comp: a pointer
  // picked at run time from an array would lose its LDS address space and
  // turn every table access into a flat one.  Entry: [0] lo, [1] start |
  // base << 13 | shift << 25, [2] min, [3] max.
  constexpr uint32_t kTab0 = 2 * MMAX, kTab1 = 2 * MMAX + 4 * kSortSegs;
  auto order_key = [&](u64 c) -> u64 { return by_value ? ~c : static_cast<u64>(col_of(c)); };

  u64 c[PER];
  uint32_t seg[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t p = t + j * NT;
    c[j] = out[p < m ? p : 0];
    seg[j] = p < m ? 0u : kDone;
  }
  if (t == 0) {
    sm.comp[kTab0] = key_lo;
    sm.comp[kTab0 + 1] = static_cast<u64>(span_bits > kRadixBits ? span_bits - kRadixBits : 0u) << 25;
  }
  __syncthreads();   // everything is in registers: R0 may be written
  int cur = 0;
  // Distinct keys need at most ~22 levels (each narrows a segment's range at
  // least 8-fold); the cap only guards against a corrupted buffer.
#pragma unroll 1
  for (int level = 0; level < 64; ++level) {
    const uint32_t tc = cur ? kTab1 : kTab0;   // this level's table
    const uint32_t tn = cur ? kTab0 : kTab1;   // the next level's
    uint32_t bin[PER], start[PER], base[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t sj = seg[j] == kDone ? 0u : seg[j];
      const u64 lo = sm.comp[tc + 4 * sj];
      const uint32_t pk = static_cast<uint32_t>(sm.comp[tc + 4 * sj + 1]);
      start[j] = pk & 0x1FFFu;
      base[j] = (pk >> 13) & 0xFFFu;
      bin[j] = base[j] + static_cast<uint32_t>((order_key(c[j]) - lo) >> (pk >> 25));
      if (seg[j] != kDone) atomicAdd(&sm.hist[bin[j]], 1u);
    }
    if (t == 0) {
      sm.nwork = 0u;
      sm.res[4] = 0u;
    }
    __syncthreads();
    uint32_t cnt[PER], first[PER], b0[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) cnt[j] = sm.hist[bin[j]];
    {
      constexpr int BPT = kBins / NT;
      uint32_t hb[BPT];
      own_bins_read<BPT>(sm, hb);
      uint32_t w2 = 0;
#pragma unroll
      for (int i = 0; i < BPT; ++i) w2 += ((hb[i] > 8u) & (hb[i] <= 32u)) ? hb[i] * hb[i] : 0u;
      w2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_prefix_sum(w2)), 63));
      if ((t & 63) == 0 && w2) atomicAdd(&sm.res[4], w2);
    }
    hist_exclusive_scan(sm);   // writes only after a barrier, so the reads above see counts
    const uint32_t H = uniform(sm.res[4]) > kSplitWork ? 8u : 32u;   // bins above H split again
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      b0[j] = sm.hist[base[j]];
      first[j] = start[j] + (sm.hist[bin[j]] - b0[j]);   // final position of the bin
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (seg[j] != kDone) {
        const uint32_t slot = atomicAdd(&sm.hist[bin[j]], 1u);
        grp[start[j] + (slot - b0[j])] = c[j];
      }
    }
    __syncthreads();
    // place the members of small bins; the first member of a large bin
    // registers it as a segment of the next level
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (seg[j] == kDone) continue;
      if (cnt[j] <= H) {
        uint32_t rank = 0;
        if (cnt[j] > 1) {
          const u64 q = order_key(c[j]);
          const uint32_t be = first[j] + cnt[j];
          for (uint32_t r0 = first[j]; r0 < be; r0 += RB) {
            u64 o[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) o[i] = grp[r0 + i < be ? r0 + i : first[j]];
#pragma unroll
            for (int i = 0; i < RB; ++i) rank += ((r0 + i < be) & (order_key(o[i]) < q)) ? 1u : 0u;
          }
        }
        out[first[j] + rank] = c[j];
        seg[j] = kDone;
      } else if (grp[first[j]] == c[j]) {
        const uint32_t id = atomicAdd(&sm.nwork, 1u);
        sm.comp[tn + 4 * id + 2] = ~0ull;
        sm.comp[tn + 4 * id + 3] = 0ull;
        sm.hist[bin[j]] = id;   // read back by the bin's members
      }
    }
    __syncthreads();
    const uint32_t nseg = uniform(sm.nwork);
    // Every element placed: done.  The histogram is left as it is (the sort
    // is its last user in the kernel).
    if (nseg == 0) break;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (seg[j] == kDone) continue;
      seg[j] = sm.hist[bin[j]];
      const u64 q = order_key(c[j]);
      atomicMin(&sm.comp[tn + 4 * seg[j] + 2], q);
      atomicMax(&sm.comp[tn + 4 * seg[j] + 3], q);
    }
    __syncthreads();
    hist_zero_own(sm);
    // the first member of each new segment fills in its entry
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (seg[j] == kDone || grp[first[j]] != c[j]) continue;
      const u64 mn = sm.comp[tn + 4 * seg[j] + 2], mx = sm.comp[tn + 4 * seg[j] + 3];
      const uint32_t s0 = first[j], s1 = first[j] + cnt[j];
      const uint32_t b_lo = static_cast<uint32_t>((static_cast<u64>(s0) * kBins) / m);
      const uint32_t b_hi = static_cast<uint32_t>((static_cast<u64>(s1) * kBins) / m);
      const uint32_t bits = bit_length64(mx - mn);
      const uint32_t nbits = 31u - static_cast<uint32_t>(__clz(b_hi - b_lo));
      const uint32_t sh = bits > nbits ? bits - nbits : 0u;
      sm.comp[tn + 4 * seg[j]] = mn;
      sm.comp[tn + 4 * seg[j] + 1] = static_cast<u64>(s0 | (b_lo << 13) | (sh << 25));
    }
    __syncthreads();   // the histogram and the next table are ready
    cur ^= 1;
  }
}

// The buffer holds m candidates: exactly the top min(k, L) after an exact
// cut, or (value order only) every candidate above the threshold, at most
// MMAX of them, of which the sort puts the top k first.
template <int NT, int CAP, int MMAX>
__device__ __forceinline__ void write_outputs(Smem<CAP, NT>& sm, const KArgs& a, bool bf16,
                                              int row, int cur, uint32_t status, uint32_t L) {
  const int t = threadIdx.x;
  const uint32_t k = a.k;
  const int64_t out0 = static_cast<int64_t>(row) * k;
  uint32_t m = min(uniform(sm.cnt[cur]), a.sorted == 1 ? static_cast<uint32_t>(MMAX) : k);
  if (status) m = 0;
  if (a.sorted != 0 && m > 1) {
    // Bounds of the sort keys: every result is above the threshold and has a
    // key no larger than hikey; columns are below L.
    if (a.sorted == 1) {
      const u64 lo = static_cast<u64>(~uniform(sm.hikey)) << 32;
      const u64 hi = ~uniform64(sm.thr) - 1u;
      sort_results<NT, CAP, MMAX>(sm, m, true, lo, bit_length64(hi - lo));
    } else {
      sort_results<NT, CAP, MMAX>(sm, m, false, 0ull, bit_length(L - 1u));
    }
  }
  m = min(m, k);
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * (bf16 ? 2 : 4);

  for (uint32_t j = t; j < k; j += NT) {
    uint32_t ix, v;
    if (j < m) {
      const u64 c = sm.comp[j];
      ix = col_of(c);
      const uint32_t key = key_of(c);
      if (key == kBias) {   // a zero: its sign is only in the input
        v = bf16 ? static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(xrow)[ix]) << 16
                 : reinterpret_cast<const uint32_t*>(xrow)[ix];
      } else {
        v = bits_of_key(key);
      }
    } else {
      ix = 0xFFFFFFFFu;
      v = status ? kQNaN32 : kNegInf32;
    }
    const int64_t o = out0 + j;
    if (a.idx64)
      static_cast<int64_t*>(a.indices)[o] = static_cast<int64_t>(static_cast<int32_t>(ix));
    else
      static_cast<int32_t*>(a.indices)[o] = static_cast<int32_t>(ix);
    if (a.return_values) {
      if (bf16)
        static_cast<uint16_t*>(a.values)[o] = static_cast<uint16_t>(v >> 16);
      else
        static_cast<uint32_t*>(a.values)[o] = v;
    }
  }
  if (t == 0) a.row_status[row] = static_cast<int32_t>(status);
}

// ---------------------------------------------------------------- the kernel
template <bool BF16, int CLS, bool MULTI>
__global__ __launch_bounds__(kernel_threads(CLS, BF16 ? 1 : 0, MULTI), kWavesPerSimd) void topk_kernel(
    KArgs a) {
  constexpr int NT = kernel_threads(CLS, BF16 ? 1 : 0, MULTI);
  constexpr int CAP = class_cap(CLS);
  constexpr int KMAX = class_kmax(CLS);
  // A value sort takes up to SORT_CAP candidates, so for value order the
  // exact cut is skipped whenever all candidates above the threshold fit:
  // the sort puts the top k first.
  constexpr int SORT_CAP = CLS <= 1 ? 2 * KMAX : KMAX;
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int V = kBlockElems / (NT * EPV);
  constexpr int NBUF = 4;   // ring of blocks: 3 loading while 1 is filtered
  static_assert(V >= 1 && V * NT * EPV == kBlockElems, "block geometry");
  __shared__ Smem<CAP, NT> sm;

  const int t = threadIdx.x, lane = t & 63;
  const uint32_t wid = uniform(static_cast<uint32_t>(t) >> 6);   // wave index, in a scalar register
  const int S = MULTI ? a.segments : 1;
  const int seg = MULTI ? static_cast<int>(blockIdx.x) % S : 0;
  int row = MULTI ? static_cast<int>(blockIdx.x) / S : static_cast<int>(blockIdx.x);
  // Variable-length rows: schedule from the last row down (for causal
  // prefill the longest rows are last), so long rows do not trail the grid.
  if (a.end) row = a.batch - 1 - row;

  uint32_t status = 0;
  uint32_t L = static_cast<uint32_t>(a.n_cols);
  if (a.end) {
    const int32_t e = a.end[row];
    if (e < 0 || e > a.n_cols) {
      status = DS_ROW_BAD_END;
      L = 0;
    } else {
      L = static_cast<uint32_t>(e);
    }
  }
  hist_zero_own(sm);
  if (t == 0) {
    sm.cnt[0] = 0u;
    sm.cnt[1] = 0u;
    sm.hikey = 0u;
    sm.flags = 0u;
    sm.n_cut = 0u;
    sm.n_reread = 0u;
    sm.thr = kThrInit;
    sm.bt[0] = 0xFFFFFFFFu;   // the start's reductions, used once, start here
    sm.bt[1] = 0u;
    sm.bt[2] = 0xFFFFFFFFu;
    sm.bt[3] = 0xFFFFFFFFu;
    sm.bt[4] = 0u;
  }
  __syncthreads();

  u64* thr_g = MULTI ? reinterpret_cast<u64*>(a.ws_thr) + row : nullptr;
  u64* spec_g = MULTI ? reinterpret_cast<u64*>(a.ws_spec) + row : nullptr;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t trigger = static_cast<uint32_t>(a.trigger);
  const uint32_t slack = (trigger - k) / 4u;
  int cur = 0;
  u64 thr = kThrInit;
  Filter F = filter_of(thr);
  float hi_lane = __uint_as_float(kNegInf32);
  bool nan_lane = false;
  auto hi_key = [&]() { return key_of_bits(__float_as_uint(hi_lane)); };

  const uint32_t nb = (L + kBlockElems - 1) / kBlockElems;
  const uint32_t ntl = nb > static_cast<uint32_t>(seg) ? (nb - seg + S - 1) / S : 0u;
  const BlockOrder order(nb, a.perm_seed, static_cast<uint32_t>(row), a.in_order != 0);
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * ESZ;
  const bool ragged_row = (L % kBlockElems) != 0;
  const uint32_t last_blk = nb - 1u;
  // Block of this workgroup's j-th step; steps past the end re-read the last
  // one (from L2) so that every step issues the same loads.
  auto blk_at = [&](uint32_t j) -> uint32_t {
    return ntl == 0 ? 0u : order(seg + (j < ntl ? j : ntl - 1u) * S);
  };

  // The decision to cut must be the same in every wave, but a fast wave may
  // append for the next block before a slow wave has looked at the counter.
  // So each wave records the count its own append produced, in a slot chosen
  // by step parity; the maximum over the waves is the count after the block.
  int par = 0;
  bool spec_used = false;   // this workgroup started from an estimate
  auto count_after_step = [&](uint32_t after) -> uint32_t {
    if (lane == 0) sm.snap[par][wid] = after;
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) c = max(c, sm.snap[par][w2]);
    par ^= 1;
    return uniform(c);
  };

  // The ring: block j goes to r[j % 4], and the shared threshold is read into
  // g0 just before the loads of every fourth block are issued, so waiting
  // for a block never waits for a later load.  Steps past the workgroup's last block
  // still issue loads (the compiler then counts outstanding loads exactly),
  // but every lane reads the row's first vector, one cache line per wave.
  u32x4 r0[V], r1[V], r2[V], r3[V];
  u64 g0 = 0, g1 = 0, g2 = 0, g3 = 0;
  // The shared threshold is read once per turn of the ring (with the blocks
  // that go to r0): every workgroup of a shared row reads the same word, up
  // to 256 of them on one row, and a bound read late only admits more.
  auto issue = [&](u32x4 (&r)[V], u64& g, uint32_t j) {
    if (MULTI && (j & 3u) == 0u) g = load_thr(thr_g);
    load_block<BF16, V, NT>(r, xrow, blk_at(j), j < ntl ? L : 0u);
  };

  auto step = [&](u32x4 (&cur_r)[V], u64& g, u32x4 (&nxt_r)[V], u64& g_nxt, uint32_t u) {
    const u64 g_cur = g;
    if (ntl > 0) issue(nxt_r, g_nxt, u + NBUF - 1);
    if (u < ntl) {
      const uint32_t blk = blk_at(u);
      // The whole blocks among the first three (bit j: block j).
      uint32_t whole = 0;
      if (u == 0) {
#pragma unroll
        for (uint32_t j = 0; j < 3; ++j)
          if (j < ntl && blk_at(j) * static_cast<uint32_t>(kBlockElems) + kBlockElems <= L)
            whole |= 1u << j;
      }
      if (u == 0 && (whole & 3u) != 0u && 2 * k <= kBlockElems) {
        // The start comes from the first whole block in the ring, where at
        // least half of a block can be dropped: block 0, or block 1 when
        // block 0 is the row's partial last block (then filtered from it).
        BlockRegs<V> br;
        if (whole & 1u) {
#pragma unroll
          for (int v = 0; v < V; ++v) br.v[v] = cur_r[v];
        } else {
          // The empty asm keeps this a branch: as a select between the two
          // copies, every workgroup would wait for block 1 first.
#pragma unroll
          for (int v = 0; v < V; ++v) {
            br.v[v] = r1[v];
            asm volatile("" : "+v"(br.v[v].x), "+v"(br.v[v].y), "+v"(br.v[v].z), "+v"(br.v[v].w));
          }
        }
        // The whole blocks already in the ring (up to three) can vouch for a
        // tighter start, which saves appends and cuts later.  t2 estimates,
        // from that block alone and with 10% to spare, the edge with k
        // of those blocks' elements at or above it; a plain count over them
        // confirms it before it is used.  They are elements of the row, so
        // the edge is valid for the whole row, shared or not.
        //
        // A workgroup with a short share (a whole row or part of one) goes
        // further: t2 is then an estimate of the edge with fk of the row's L
        // elements at or above it (the fkB/L-th largest of that block).  It
        // is used if the ring's count scales to at least 0.75 min(f, 2) k for
        // the row, and checked at the end: by the merge for a shared row (the
        // estimate is recorded for the row), by the final count for a whole
        // row.  A failed check means one of the top k may lie at or below
        // it, and the row is read again from a valid bound.  f is 3 on a
        // shared row whose results need no sort, 2 on other shared rows: the
        // wider margin makes a refused estimate (whose workgroup then lags
        // the row) rarer, and costs more survivors at the end, which the
        // sort pays for per candidate and the merge's exact cut hardly at
        // all.  A whole row has no other workgroup to lag behind, and its
        // exact cut pays for every extra candidate: f is 1.5 there.
        const uint32_t nw = static_cast<uint32_t>(__popc(whole));
        const uint32_t fold4 = MULTI ? (a.sorted != 1 ? 12u : 8u) : 6u;   // f in quarters
        const uint32_t nspec =
            (ntl <= kSpecSteps && nw >= 2u)
                ? static_cast<uint32_t>((static_cast<u64>(fold4) * k * kBlockElems + 4ull * L - 1u) /
                                        (4ull * L))
                : k;
        const bool spec = nspec < k;
        const uint32_t need2 =
            spec ? nspec : (nw >= 2u ? (11u * k + 10u * nw - 1u) / (10u * nw) : 0u);
        const ThrPair tp = wave_threshold<BF16, V, NT, CAP>(br, k, need2, sm);
        u64 t0 = uniform64(tp.t0);   // the same in every lane: keep it scalar
        const u64 t2 = uniform64(tp.t2);
        u64 tloc = t0;               // this workgroup's start
        if (need2 != 0u && t0 != kThrInit && t2 > t0) {
          // Elements with key >= tk2 are the values >= the value of key tk2
          // (keys order like the values, both zeros share one key, and a NaN
          // compares false): one float compare per element.
          const uint32_t tk2 = static_cast<uint32_t>(t2 >> 32) + 1u;
          const float tf = __uint_as_float(uniform(bits_of_key(tk2)));
          uint32_t n = 0;
          auto count_in = [&](const u32x4 (&rr)[V]) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
              const uint32_t w[4] = {rr[v].x, rr[v].y, rr[v].z, rr[v].w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int h = 0; h < (BF16 ? 2 : 1); ++h) {
                  const uint32_t bits = BF16 ? (h ? (w[q] & 0xFFFF0000u) : (w[q] << 16)) : w[q];
                  n += __uint_as_float(bits) >= tf ? 1u : 0u;
                }
              }
            }
          };
          if (whole & 1u) count_in(cur_r);
          if (whole & 2u) count_in(r1);
          if (whole & 4u) count_in(r2);
          const uint32_t wt = static_cast<uint32_t>(
              __builtin_amdgcn_readlane(static_cast<int>(wave_prefix_sum(n)), 63));
          if (lane == 0) atomicAdd(&sm.bt[4], wt);
          __syncthreads();
          const uint32_t ring = uniform(sm.bt[4]);
          if (ring >= k) {
            t0 = t2;   // k of the row's elements at or above it: valid
            tloc = t2;
          } else if (spec && 16ull * ring * nb >= 3ull * (fold4 < 8u ? fold4 : 8u) * k * nw) {
            tloc = t2;   // an estimate, checked by the merge
          }
        }
        spec_used = tloc != t0;
        if (!MULTI && t == 0) sm.tvalid = t0;   // where a re-read starts
        if (tloc > thr) {
          thr = tloc;
          F = filter_of(thr);
          if (t == 0) {
            atomicMax(&sm.thr, tloc);
            if (MULTI) {
              publish_thr(thr_g, t0);   // only a valid bound is shared
              if (tloc != t0)
                __hip_atomic_fetch_max(spec_g, tloc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
      if constexpr (2 * KMAX > kBlockElems) {
        // k above half a block: one block cannot drop enough, but three whole
        // ring blocks (3 B >= 2 k) can.  Their k-th largest value is a valid
        // start (k elements of the row at or above it).
        if (u == 0 && whole == 7u && 2u * k <= 3u * static_cast<uint32_t>(kBlockElems)) {
          BlockRegs<3 * V> b3;
#pragma unroll
          for (int v = 0; v < V; ++v) {
            b3.v[v] = cur_r[v];
            b3.v[V + v] = r1[v];
            b3.v[2 * V + v] = r2[v];
          }
          // (the block-wide histogram: its k-th value is tighter than the
          // smallest of the waves' edges, and no estimate is needed here)
          const u64 t3 = uniform64(block_threshold_body<BF16, 3 * V, NT, CAP>(b3, k, 0u, sm).t0);
          if (t == 0) sm.tvalid = t3;
          if (t3 > thr) {
            thr = t3;
            F = filter_of(thr);
            if (t == 0) {
              atomicMax(&sm.thr, t3);
              if (MULTI) publish_thr(thr_g, t3);
            }
          }
        }
      }
      uint32_t after;
      if (ragged_row && blk == last_blk) {
        BlockRegs<V> br;
#pragma unroll
        for (int v = 0; v < V; ++v) br.v[v] = cur_r[v];
        const RaggedResult rr =
            filter_ragged<BF16, V, NT, CAP>(br, blk, L, F, hi_lane, nan_lane ? 1u : 0u, sm, cur);
        after = rr.after;
        hi_lane = rr.hi_lane;
        nan_lane = rr.nan_lane != 0;
      } else {
        after = filter_block<BF16, false, V, NT, CAP>(cur_r, blk, L, F, hi_lane, nan_lane, sm, cur);
      }
      if (MULTI && g_cur > thr && lane == 0) atomicMax(&sm.thr, g_cur);
      const uint32_t c = count_after_step(after);
      // No cut after the last block: the exact cut that follows the stream
      // takes the buffer as it is (a block never overfills it).
      if (c > trigger && u + 1 < ntl) {
        const u64 before = uniform64(sm.thr);
        cur = cut_buffer<NT, CAP>(sm, cur, k, k + slack, L, hi_key());
        thr = uniform64(sm.thr);
        if (MULTI && t == 0 && thr > before) publish_thr(thr_g, thr);
      } else if (MULTI) {
        const u64 seen = uniform64(sm.thr);   // may include a later wave's raise: still a valid bound
        thr = seen > thr ? seen : thr;
      }
      F = filter_of(thr);
    }
  };

  if (ntl > 0) {
    issue(r0, g0, 0);
    issue(r1, g1, 1);
    issue(r2, g2, 2);
  }
  for (uint32_t u = 0; u < ntl; u += NBUF) {
    step(r0, g0, r3, g3, u);
    step(r1, g1, r0, g0, u + 1);
    step(r2, g2, r1, g1, u + 2);
    step(r3, g3, r2, g2, u + 3);
  }

  // The whole row read again, in order, from the largest valid bound
  // (sm.tvalid), with the usual filter and cuts: for an estimated start that
  // may have dropped one of the top k.
  auto reread_row = [&]() {
    if (t == 0) {
      sm.cnt[cur] = 0u;
      sm.thr = sm.tvalid;
      sm.n_reread += 1u;
    }
    __syncthreads();
    thr = uniform64(sm.thr);
    F = filter_of(thr);
    for (uint32_t b = 0; b < nb; ++b) {
      u32x4 rb[V];
      load_block<BF16, V, NT>(rb, xrow, b, L);
      uint32_t after;
      if (ragged_row && b == last_blk) {
        BlockRegs<V> br;
#pragma unroll
        for (int v = 0; v < V; ++v) br.v[v] = rb[v];
        const RaggedResult rr =
            filter_ragged<BF16, V, NT, CAP>(br, b, L, F, hi_lane, nan_lane ? 1u : 0u, sm, cur);
        after = rr.after;
        hi_lane = rr.hi_lane;
        nan_lane = rr.nan_lane != 0;
      } else {
        after = filter_block<BF16, false, V, NT, CAP>(rb, b, L, F, hi_lane, nan_lane, sm, cur);
      }
      const uint32_t c2 = count_after_step(after);
      if (c2 > trigger && b + 1 < nb) {
        cur = cut_buffer<NT, CAP>(sm, cur, k, k + slack, L, hi_key());
        thr = uniform64(sm.thr);
        F = filter_of(thr);
      }
    }
    const uint32_t hk = wave_max(hi_key());   // every candidate key, for the sort
    if (lane == 0) atomicMax(&sm.hikey, hk);
    __syncthreads();
  };

  // NaN anywhere in this workgroup's share of [0, L).
  if (ballot(nan_lane) && lane == 0) atomicOr(&sm.flags, static_cast<uint32_t>(DS_ROW_NAN));
  // A workgroup that owns its row and started from an estimate holds every
  // element above the estimate; with at least k of them (or after a cut,
  // which keeps k) none of the top k was dropped.  Otherwise it reads the row
  // again from t0.
  if (!MULTI && spec_used) {
    __syncthreads();   // the NaN flags are in
    if (uniform(sm.cnt[cur]) < k && uniform(sm.flags) == 0u) reread_row();
  }
  // A shared row's small buffer needs no cut, only the bound x_w and, when
  // it holds more than the hand-over's k + kSmallBin slots, a bin edge with
  // between k and k + kSmallBin candidates above it.  Both come from a
  // 256-bin histogram that every wave scans for itself (two barriers instead
  // of a cut's five); a boundary bin too large for the slots falls back to
  // the cut.
  const uint32_t c_end = min(uniform(sm.cnt[cur]), static_cast<uint32_t>(CAP));
  const bool x_only = MULTI && c_end <= static_cast<uint32_t>(small_cut_g(CAP, NT) * NT);
  if (MULTI && !x_only && t == 0) {
    const u64 gl = load_thr(thr_g);
    if (gl > sm.thr) sm.thr = gl;   // survivors at or below the shared bound are not needed
  }
  // One workgroup on the row: the exact top-k.  Several: only the threshold
  // that leaves between k and k + kSmallBin candidates (the merge makes the
  // row's one exact cut), and the bound x_seg with at least ceil(k / S) of
  // this workgroup's candidates above it: the smallest x_seg over the row has
  // at least k candidates above it, so the merge drops everything at or
  // below it.  The buffer is not compacted: the hand-over below reads it
  // filtered by the threshold.
  if (!MULTI) {   // hikey bounds every candidate's key, cut or no cut
    const uint32_t hk = wave_max(hi_key());
    if (lane == 0) atomicMax(&sm.hikey, hk);
    __syncthreads();
  }
  uint32_t mine = 0;   // shared rows: candidates above the threshold
  u64 x_w = 0;         // and the bound they vouch for
  u64 t_keep = 0;      // small buffer: the threshold the hand-over filters by
  bool cut = !x_only && (MULTI || a.sorted != 1 || uniform(sm.cnt[cur]) > static_cast<uint32_t>(SORT_CAP));
  if (x_only) {
    const uint32_t need_w = (k + static_cast<uint32_t>(S) - 1u) / static_cast<uint32_t>(S);
    const u64 T = uniform64(sm.thr);
    const uint32_t K = static_cast<uint32_t>(T >> 32);
    const uint32_t klo = static_cast<uint32_t>(T) == 0xFFFFFFFFu ? K + 1u : K;
    const uint32_t hk = wave_max(hi_key());
    uint32_t n = 0;
    for (uint32_t i = t; i < c_end; i += NT) n += sm.comp[i] > T ? 1u : 0u;
    n = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_prefix_sum(n)), 63));
    if (lane == 0) {
      sm.snap[par][wid] = n;
      atomicMax(&sm.hikey, hk);
    }
    __syncthreads();   // also: every wave's NaN flag is in
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) mine += sm.snap[par][w2];
    par ^= 1;
    mine = uniform(mine);
    t_keep = T;
    const uint32_t hi = uniform(sm.hikey);
    if (mine >= need_w && hi >= klo) {
      const uint32_t sh = bit_length(hi - klo) > 8u ? bit_length(hi - klo) - 8u : 0u;
      for (uint32_t i = t; i < c_end; i += NT) {
        const u64 v = sm.comp[i];
        if (v > T) atomicAdd(&sm.hist[(key_of(v) - klo) >> sh], 1u);
      }
      __syncthreads();
      // Bins 4 lane .. 4 lane + 3 per lane; the suffix count from the top
      // finds the bin b with >= need_w candidates in bins >= b.
      const u32x4 hb = reinterpret_cast<const u32x4*>(sm.hist)[lane];
      const uint32_t s4 = hb.x + hb.y + hb.z + hb.w;
      const uint32_t incl = wave_prefix_sum(s4);
      const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
      const uint32_t above = total - incl;   // bins of the lanes above this one
      const u64 hit = ballot((above < need_w) & (above + s4 >= need_w));
      const int hl = static_cast<int>(__ffsll(static_cast<long long>(hit))) - 1;   // one lane
      uint32_t b = 4u * static_cast<uint32_t>(lane) + 3u, acc = above;
      const uint32_t h4[4] = {hb.x, hb.y, hb.z, hb.w};
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (acc < need_w) b = 4u * static_cast<uint32_t>(lane) + static_cast<uint32_t>(i);
        acc += h4[i];
      }
      b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), hl));
      x_w = (static_cast<u64>(klo + (b << sh)) << 32) - 1u;
      if (mine > k + static_cast<uint32_t>(kSmallBin)) {
        // The bin bk with fewer than k candidates above it and at least k
        // at or above it; its lower edge keeps the candidates of bins >= bk.
        const u64 kh = ballot((above < k) & (above + s4 >= k));
        const int kl = static_cast<int>(__ffsll(static_cast<long long>(kh))) - 1;   // one lane
        uint32_t bk = 0, in_k = 0;
        acc = above;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if ((acc < k) & (acc + h4[i] >= k)) {
            bk = 4u * static_cast<uint32_t>(lane) + static_cast<uint32_t>(i);
            in_k = acc + h4[i];
          }
          acc += h4[i];
        }
        bk = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bk), kl));
        in_k = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(in_k), kl));
        if (in_k <= k + static_cast<uint32_t>(kSmallBin)) {
          const u64 edge = (static_cast<u64>(klo + (bk << sh)) << 32) - 1u;
          t_keep = edge > T ? edge : T;
          mine = in_k;
        } else {
          cut = true;
        }
      }
    }
    if (cut) {   // every wave has scanned the bins: clear them for the cut
      __syncthreads();
      for (uint32_t j = t; j < 256u; j += NT) sm.hist[j] = 0u;
    }
  }
  if (cut) {
    cur = cut_buffer<NT, CAP>(sm, cur, k, MULTI ? k + kSmallBin : k, L, hi_key(),
                              MULTI ? (k + static_cast<uint32_t>(S) - 1u) / static_cast<uint32_t>(S) : 0u,
                              MULTI);
    if (MULTI) {
      mine = uniform(sm.kept);   // at most k + kSmallBin
      x_w = uniform64(sm.xv);
    }
  }

  if (MULTI) {
    // Hand the survivors to the row's last workgroup.  Each workgroup
    // reserves a range of the row's contiguous array with one atomic on the
    // row's fill cursor and fills all of it, and the merge reads up to the
    // row's fill, so the array needs no clearing between calls (slots past
    // the fill hold whatever an earlier call left).  Every shared word is
    // written and read with agent-scope atomic accesses, and the stores are
    // complete before the arrival counter moves, so no L2 write-back or
    // invalidate is needed.
    constexpr int PER_FIT = (8 * (KMAX + static_cast<int>(kSmallBin)) + 2 * NT - 1) / (2 * NT);
    constexpr int PER_ROOM = (CAP - (3 * KMAX + class_trigger(CLS)) / 4) / NT;
    constexpr int PER_A = PER_FIT > 9 ? 9 : PER_FIT;
    constexpr int PER_B = PER_A > PER_ROOM ? PER_ROOM : PER_A;
    constexpr int PER = PER_B < 4 ? 4 : PER_B;
    static_assert(PER * NT + (3 * KMAX + class_trigger(CLS)) / 4 <= CAP, "merge chunk room");
    constexpr uint32_t CHUNK = PER * NT;
    const uint32_t area = static_cast<uint32_t>(S) * (k + kSmallBin);
    constexpr bool fixed_slots = false;
    const uint32_t c = uniform(sm.cnt[cur]);
    const u64 Tk = (x_only && !cut) ? t_keep : uniform64(sm.thr);
    u64* wsc = reinterpret_cast<u64*>(a.ws_comp) + static_cast<int64_t>(row) * S * (k + kSmallBin);
    if (t == 0) {
      if (!fixed_slots)
        sm.res[0] = mine ? __hip_atomic_fetch_add(&a.ws_fill[row], mine, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                         : 0u;
      sm.cnt[cur ^ 1] = 0u;
      sm.thr = Tk;   // read again only after the barrier below
      if (mine >= k) publish_thr(thr_g, Tk);
      st_agent(&a.ws_x[static_cast<int64_t>(row) * S + seg], x_w);
      if (sm.flags)
        __hip_atomic_fetch_or(&a.ws_flags[row], sm.flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (x_only)   // the 256 bins x_w used go back to zero (every wave has read them)
      for (uint32_t i = t; i < 256u; i += NT) sm.hist[i] = 0u;
    const uint32_t own0 = fixed_slots ? static_cast<uint32_t>(seg) * (k + static_cast<uint32_t>(kSmallBin))
                                      : uniform(sm.res[0]);
    // Every candidate above the threshold goes to the workgroup's range, at
    // an offset taken with one LDS atomic per wave and group (never past the
    // range, whatever the count).
    for_groups<NT>(c, [&](auto gs, uint32_t e0) {
      constexpr int G = decltype(gs)::value;
      u64 v[G];
      read_group<G>(sm, e0, c, v);
      u64 mk[G];
      uint32_t tot = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        mk[g] = ballot(v[g] > Tk);
        tot += static_cast<uint32_t>(__popcll(mk[g]));
      }
      if (tot) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&sm.cnt[cur ^ 1], tot);
        base = uniform(base);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t pos = base + mbcnt64(mk[g]);
          if (((mk[g] >> lane) & 1ull) & (pos < mine)) st_agent(&wsc[own0 + pos], v[g]);
          base += static_cast<uint32_t>(__popcll(mk[g]));
        }
      }
    });
    // Every reserved slot is written: should fewer than `mine` candidates
    // pass (never expected), the rest of the range gets zero, which no
    // threshold admits.
    __syncthreads();
    for (uint32_t j = uniform(sm.cnt[cur ^ 1]) + t; j < mine; j += NT) st_agent(&wsc[own0 + j], 0ull);
    wait_all_memory();
    __syncthreads();
    if (t == 0) {
      sm.rng[0] = ~0ull;   // the merge's minimum over the bounds x_seg
      const uint32_t prev =
          __hip_atomic_fetch_add(&a.ws_done[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.is_last = prev == static_cast<uint32_t>(S - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!uniform(sm.is_last)) {
      if (a.stats && t == 0 && sm.n_cut) atomicAdd(&a.stats[4 * static_cast<int64_t>(row) + DS_STAT_CUTS], sm.n_cut);
      return;
    }

    // Last arrival: merge every workgroup's survivors.  Start from the largest
    // of the shared threshold and min_seg x_seg (0 if any workgroup had fewer
    // than ceil(k / S) survivors).
    // Every load goes out at once: the row's counters and bounds first (so
    // that using them waits for nothing else), then the first two chunks of
    // survivor slots, before the row's fill is known: positions at or past
    // the fill (whatever an earlier call left there) are dropped once it
    // is.  A chunk is at most 9 slots per
    // thread: two chunks hold the slots of up to 4 workgroups at k near the
    // class's largest (all of them, for the sampler and indexer shapes) in
    // one round trip, and the registers stay clear of the spills whose
    // reloads would wait for every load and store in flight.  A chunk must
    // also fit in the buffer after a cut (at most k + slack candidates
    // remain).
    // Loads of one chunk; positions past the array read position 0 (a valid
    // address) and are dropped.
    auto load_chunk = [&](uint32_t c0, u64 (&mv)[PER]) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const uint32_t p = c0 + t + q * NT;
        mv[q] = ld_agent(&wsc[p < area ? p : 0u]);
      }
    };
    u64 gfin = 0, spm = 0;
    uint32_t fl = 0, fill = 0;
    if (t == 0) {
      gfin = load_thr(thr_g);
      spm = ld_agent(spec_g);
      fl = ld_agent(&a.ws_flags[row]);
      if (!fixed_slots) fill = ld_agent(&a.ws_fill[row]);
    }
    u64 xs = ~0ull;
    u64* xp = &a.ws_x[static_cast<int64_t>(row) * S + (t < S ? t : 0)];
    if (t < S) xs = ld_agent(xp);
    u64 va[PER], vb[PER];
    load_chunk(0, va);
    load_chunk(CHUNK, vb);
    xs = wave_extreme64<false>(xs);
    if (lane == 0 && t < S) atomicMin(&sm.rng[0], xs);   // rng[0] was set before the arrival count
    if (t == 0) {
      if (gfin > sm.thr) sm.thr = gfin;
      sm.tvalid = gfin;
      sm.specmax = spm;
      sm.flags |= fl;
      sm.res[1] = fill;
      // Its own candidates come back from the array with everyone else's,
      // filtered by the same bound, so the LDS buffer starts empty.
      sm.cnt[cur] = 0u;
    }
    __syncthreads();
    const uint32_t total = fixed_slots ? area : min(uniform(sm.res[1]), area);
    const u64 xmin = uniform64(sm.rng[0]);
    u64 T0 = uniform64(sm.thr);
    T0 = xmin > T0 ? xmin : T0;
    if (t == 0) {   // read again only after the next barrier
      sm.thr = T0;
      if (xmin > sm.tvalid) sm.tvalid = xmin;
    }
    u64 Tm = T0;
    // Appended candidates above the row's largest estimated start (checked
    // after the merge).  A cut inside the merge can only drop candidates at
    // or below its new bound, and keeps k above it: if that bound is below
    // the estimate the count stays exact, else the check passes either way.
    const u64 specmax = uniform64(sm.specmax);
    uint32_t n_above = 0;
    auto merge_chunk = [&](uint32_t c0, const u64 (&mv)[PER]) {
      auto pass = [&](int q) -> bool {
        const uint32_t p = c0 + t + q * NT;
        return (p < total) & (mv[q] > Tm);
      };
      u64 mm[PER];
      uint32_t tot = 0, kmax = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const bool p = pass(q);
        const uint32_t kq = p ? key_of(mv[q]) : 0u;
        kmax = kq > kmax ? kq : kmax;
        mm[q] = ballot(p);
        tot += static_cast<uint32_t>(__popcll(mm[q]));
      }
      // The chunk's total is known before anything is appended: if it would
      // not fit, cut first and filter the chunk again with the raised bound.
      const uint32_t wk = wave_max(kmax);
      if (lane == 0) {
        sm.snap[par][wid] = tot;
        atomicMax(&sm.hikey, wk);
      }
      __syncthreads();
      uint32_t sum = 0;
#pragma unroll
      for (int w2 = 0; w2 < NT / 64; ++w2) sum += sm.snap[par][w2];
      par ^= 1;
      if (uniform(sm.cnt[cur]) + uniform(sum) > static_cast<uint32_t>(CAP)) {
        cur = cut_buffer<NT, CAP>(sm, cur, k, k + slack, L, hi_key());
        Tm = uniform64(sm.thr);
        tot = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          mm[q] = ballot(pass(q));
          tot += static_cast<uint32_t>(__popcll(mm[q]));
        }
      }
      if (tot) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&sm.cnt[cur], tot);
        base = uniform(base);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          const uint32_t pos = base + mbcnt64(mm[q]);
          const bool mine = (mm[q] >> lane) & 1ull;
          if (mine & (pos < static_cast<uint32_t>(CAP))) sm.comp[pos] = mv[q];
          n_above += (mine & (mv[q] > specmax)) ? 1u : 0u;
          base += static_cast<uint32_t>(__popcll(mm[q]));
        }
      }
    };
    for (uint32_t c0 = 0; c0 < total; c0 += 2 * CHUNK) {
      merge_chunk(c0, va);
      if (c0 + 2 * CHUNK < total) load_chunk(c0 + 2 * CHUNK, va);
      if (c0 + CHUNK < total) merge_chunk(c0 + CHUNK, vb);
      if (c0 + 3 * CHUNK < total) load_chunk(c0 + 3 * CHUNK, vb);
    }
    n_above = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(wave_prefix_sum(n_above)), 63));
    if (lane == 0) sm.snap[par][wid] = n_above;
    __syncthreads();   // every append is counted
    uint32_t above = 0;
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) above += sm.snap[par][w2];
    par ^= 1;

    // An estimated start dropped, unseen, whatever lay at or below it.  That
    // lost nothing iff at least k merged candidates lie above the row's
    // largest estimate (then so does the row's k-th largest).  Otherwise the
    // row is read again, whole and in order, from the largest valid bound.
    if (specmax != 0ull) {
      if (uniform(above) < k && uniform(sm.flags) == 0u) reread_row();
    }
    if (a.sorted != 1 || uniform(sm.cnt[cur]) > static_cast<uint32_t>(SORT_CAP)) {
      if (uniform(sm.cnt[cur]) <= static_cast<uint32_t>(small_cut_g(CAP, NT) * NT)) {
        if constexpr (CLS <= 1)
          cur = small_cut<small_cut_g(CAP, NT), NT, CAP>(sm, cur, k, L, hi_key());
        else
          cur = small_cut_call<small_cut_g(CAP, NT), NT, CAP>(sm, cur, k, L, hi_key());
      } else {
        cur = cut_buffer<NT, CAP>(sm, cur, k, k, L, hi_key());
      }
    }
    if (t == 0) {
      st_agent(spec_g, 0ull);
      st_agent(&a.ws_done[row], 0u);
      st_agent(&a.ws_flags[row], 0u);
      st_agent(&a.ws_fill[row], 0u);
      st_agent(thr_g, 0ull);
    }
  }

  status |= sm.flags;
  if (a.stats && t == 0) {
    uint32_t* st = a.stats + 4 * static_cast<int64_t>(row);
    if (sm.n_reread) atomicAdd(&st[DS_STAT_ROW_REREADS], sm.n_reread);
    atomicAdd(&st[DS_STAT_FINAL_CANDIDATES], uniform(sm.cnt[cur]));
  }
  write_outputs<NT, CAP, SORT_CAP>(sm, a, BF16, row, cur, status, L);
  if (a.stats && t == 0 && sm.n_cut) atomicAdd(&a.stats[4 * static_cast<int64_t>(row) + DS_STAT_CUTS], sm.n_cut);
}

// ---------------------------------------------------------------- read ceiling
// A measurement aid, not part of the selection: the TopK stream's grid, block
// order and 16-byte loads (a ring of four blocks, three in flight), with the
// data only folded into one word per lane.  The word is stored only if it
// equals a constant, so no load can be dropped.  Its time is the read ceiling
// of this access pattern on the same input.
template <bool BF16, int NT>
__global__ __launch_bounds__(NT, 2) void read_kernel(KArgs a, uint32_t* sink) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int V = kBlockElems / (NT * EPV);
  const int S = a.segments;
  const int seg = static_cast<int>(blockIdx.x) % S;
  const int row = static_cast<int>(blockIdx.x) / S;
  uint32_t L = static_cast<uint32_t>(a.n_cols);
  if (a.end) {
    const int32_t e = a.end[row];
    L = (e < 0 || e > a.n_cols) ? 0u : static_cast<uint32_t>(e);
  }
  const uint32_t nb = (L + kBlockElems - 1) / kBlockElems;
  const uint32_t ntl = nb > static_cast<uint32_t>(seg) ? (nb - seg + S - 1) / S : 0u;
  const BlockOrder order(nb, a.perm_seed, static_cast<uint32_t>(row), a.in_order != 0);
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * ESZ;
  auto ld = [&](u32x4 (&r)[V], uint32_t j) {
    const uint32_t blk = ntl == 0 ? 0u : order(seg + (j < ntl ? j : ntl - 1u) * S);
    load_block<BF16, V, NT>(r, xrow, blk, j < ntl ? L : 0u);
  };
  uint32_t acc = 0;
  auto use = [&](const u32x4 (&r)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v) acc += (r[v].x ^ r[v].y) + (r[v].z ^ r[v].w);
  };
  u32x4 r0[V], r1[V], r2[V], r3[V];
  if (ntl > 0) {
    ld(r0, 0);
    ld(r1, 1);
    ld(r2, 2);
  }
  for (uint32_t u = 0; u < ntl; u += 4) {
    ld(r3, u + 3);
    use(r0);
    ld(r0, u + 4);
    use(r1);
    ld(r1, u + 5);
    use(r2);
    ld(r2, u + 6);
    use(r3);
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

// The launch's own error code: hipLaunchKernel returns it, and an earlier,
// unrelated error left in the runtime is neither returned nor cleared.
static int launch_fn(const void* fn, unsigned grid, unsigned block, void** args, hipStream_t stream) {
  return static_cast<int>(hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, stream));
}

template <bool BF16, int CLS>
static int launch_one(const KArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.segments);
  KArgs arg = a;
  void* args[] = {&arg};
  if (a.segments > 1)
    return launch_fn(reinterpret_cast<const void*>(&topk_kernel<BF16, CLS, true>), grid,
                     kernel_threads(CLS, BF16 ? 1 : 0, true), args, stream);
  return launch_fn(reinterpret_cast<const void*>(&topk_kernel<BF16, CLS, false>), grid,
                   kernel_threads(CLS, BF16 ? 1 : 0, false), args, stream);
}

int launch_read(const KArgs& a, int dtype, int cls, uint32_t* sink, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.segments);
  const int nt = kernel_threads(cls, dtype, a.segments > 1);
  KArgs arg = a;
  void* args[] = {&arg, &sink};
  const void* fn;
  if (dtype == 0) fn = nt == 512 ? reinterpret_cast<const void*>(&read_kernel<false, 512>)
                                 : reinterpret_cast<const void*>(&read_kernel<false, 256>);
  else fn = nt == 512 ? reinterpret_cast<const void*>(&read_kernel<true, 512>)
                      : reinterpret_cast<const void*>(&read_kernel<true, 256>);
  return launch_fn(fn, grid, static_cast<unsigned>(nt), args, stream);
}

int launch_topk(const KArgs& a, int dtype, int cls, hipStream_t stream) {
  if (dtype == 0) {
    switch (cls) {
      case 0: return launch_one<false, 0>(a, stream);
      case 1: return launch_one<false, 1>(a, stream);
      case 2: return launch_one<false, 2>(a, stream);
      default: return launch_one<false, 3>(a, stream);
    }
  }
  switch (cls) {
    case 0: return launch_one<true, 0>(a, stream);
    case 1: return launch_one<true, 1>(a, stream);
    case 2: return launch_one<true, 2>(a, stream);
    default: return launch_one<true, 3>(a, stream);
  }
}

}  // namespace dstk
