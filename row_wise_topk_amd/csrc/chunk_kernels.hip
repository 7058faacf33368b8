// Row-wise TopK for MI355X (gfx950, wave64): the chunk kernels.
//
// Method (narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for
// sparse attention and sampling", method paragraph): a threshold T that never
// falls, the row read once in contiguous blocks, the values that pass T
// appended to a candidate buffer, and a radix select that cuts the buffer back
// to k and raises T when it fills.  These kernels serve rows of up to a few
// hundred thousand elements (the sampler and Lightning Indexer shapes), where
// the cost is not the stream but the serial chain of a workgroup's steps; they
// are laid out to keep that chain short on CDNA4:
//
//  * a chunk is 8 16-byte loads per lane of a 512-lane workgroup (16384 fp32
//    or 32768 bf16 values, 64 KiB), all issued at once and held in
//    registers; a workgroup takes either one chunk of a row (a row split
//    into one workgroup per chunk, when the batch alone cannot fill the
//    chip) or a whole row, chunk by chunk, two workgroups per CU keeping
//    each other's loads in flight;
//  * the first chunk sets T before anything is appended.  A workgroup that
//    holds a whole row sets the row's exact start (at least min(k, L) of its
//    values pass); otherwise T is an estimate, at least m values of the chunk
//    pass it, with m the chunk's expected share of the top k plus a margin of
//    six standard deviations.  An estimate is checked once the row is
//    complete: if fewer than min(k, L) candidates passed, the row is read
//    again from a valid bound;
//  * T comes from a 256-bin histogram anchored at the chunk's largest value,
//    one bin per bf16 value (1/128 octave for fp32) and coarser windows after
//    it, over each lane's largest value when m is small, else (whole rows)
//    one representative per group of values: a member of each group, so the
//    m-th largest representative has m values at or above it;
//  * a split row's chunk is filtered in one pass over the registers into a
//    region of LDS per wave; a whole row's chunk tests each 16-byte vector
//    once and compacts only the vectors holding a candidate, staged in LDS;
//  * a candidate is the 64-bit composite (key(v) << 32) | ~column, so one
//    unsigned compare orders candidates exactly as the output (larger value
//    first, then lower column: xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！",
//    Q&A on stable results).  key() maps fp32 sign-magnitude onto offset
//    binary, so -0.0 and +0.0 share a key; a zero's sign is read back from the
//    input when it is written out.  A threshold is a composite too: a
//    candidate passes iff its composite is >= T;
//  * the cut is an MSD radix select over the composites' live range (11-bit
//    LDS histograms, at most six levels), which ranks a boundary bin of at
//    most 64 members directly; it keeps exactly the requested count;
//  * a split row hands its candidates over through the workspace, with the
//    chunk's threshold (agent-scope stores, all waited for before the row's
//    arrival counter moves), and the last workgroup of the row to arrive
//    merges them;
//  * value order comes from every candidate's rank (a 2048-bin histogram,
//    a scatter into bin order, the bin-mates above it); any order from the
//    boundary bin ranked by one wave; a bitonic sort in registers
//    (cross-lane steps on the VALU, cross-wave steps through LDS) serves
//    the rows these cannot (long runs of equal values).
//
// NaN (narracomm.com, NaN paragraph): always checked over [0, end); a NaN sets
// a status bit for the row instead of trapping.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_topk.h"
#include "topk_internal.h"

namespace dstk {
namespace {

typedef unsigned long long u64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

#ifndef CHUNK_SPLIT
#error "built with CHUNK_SPLIT = 1 (split rows) or 0 (whole rows)"
#endif
constexpr bool kSplit = CHUNK_SPLIT != 0;
constexpr int NT = kSplit ? kChunkThreadsSplit : kChunkThreadsRow;   // lanes per workgroup
constexpr int NW = NT / 64;
// Waves per SIMD for `blocks` workgroups per CU (the second launch bound).
constexpr int waves_per_simd(int blocks) { return blocks * NT / 256 > 0 ? blocks * NT / 256 : 1; }
constexpr int V = kChunkLoads;      // 16-byte loads per lane per chunk
constexpr uint32_t kBias = 0x80000000u;
constexpr uint32_t kNegInfKey = 0x00800000u;   // key of -inf, the lowest non-NaN key
constexpr uint32_t kQNaN32 = 0x7FC00000u;
constexpr uint32_t kNegInf32 = 0xFF800000u;
constexpr int kWinBins = 256;                  // the start histogram: one bin per lane
constexpr int kCutBits = 11;
constexpr int kCutBins = 1 << kCutBits;        // the cut's histogram
constexpr int kCutBPT = kCutBins / NT;         // bins per lane
constexpr uint32_t kRankMax = 64;              // boundary bins ranked directly
constexpr uint32_t kNone = 0xFFFFFFFFu;
constexpr u64 kTAll = static_cast<u64>(kNegInfKey) << 32;   // every non-NaN value passes

// The start histogram is scanned one bin per lane; lanes past its bins read
// bins that are zero at rest.
static_assert(kWinBins <= NT && NT <= kCutBins, "one start bin per lane");
static_assert(kCutBins % NT == 0, "cut bins per lane");

// ---------------------------------------------------------------- keys
__device__ __forceinline__ uint32_t key_of_bits(uint32_t b) {
  const uint32_t mag = b & 0x7FFFFFFFu;
  return (b & 0x80000000u) ? kBias - mag : kBias + mag;
}
// Inverse for keys of non-NaN values; the key of both zeros gives +0.0.
__device__ __forceinline__ uint32_t bits_of_key(uint32_t key) {
  return key >= kBias ? key - kBias : ((kBias - key) | 0x80000000u);
}
__device__ __forceinline__ u64 comp_of(uint32_t key, uint32_t col) {
  return (static_cast<u64>(key) << 32) | static_cast<uint32_t>(~col);
}
__device__ __forceinline__ uint32_t key_of(u64 c) { return static_cast<uint32_t>(c >> 32); }
__device__ __forceinline__ uint32_t col_of(u64 c) { return ~static_cast<uint32_t>(c); }

// "composite >= T" as float compares on the value:  x > f, or x == f and
// column <= cmax.  For T = (K << 32) | ~C this is key > K or (key == K and
// column <= C); keys order like values and both zeros share a key, so the
// float compares agree with the key compares for every non-NaN x, and a NaN
// passes nothing.
struct Pass {
  float f;
  uint32_t cmax;
};
__device__ __forceinline__ Pass pass_of(u64 T) {
  return {__uint_as_float(bits_of_key(key_of(T))), ~static_cast<uint32_t>(T)};
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}
__device__ __forceinline__ u64 uniform64(u64 v) {
  return (static_cast<u64>(uniform(static_cast<uint32_t>(v >> 32))) << 32) |
         uniform(static_cast<uint32_t>(v));
}
__device__ __forceinline__ u64 ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ uint32_t mbcnt64(u64 m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}
__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

template <int CTRL, int ROW_MASK, uint32_t IDENT>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(IDENT), static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}
// Inclusive scans over the 64 lanes (all lanes active): row_shr 1/2/4/8 in
// each 16-lane row, then row_bcast 15 and 31 across rows.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += dpp<0x111, 0xF, 0u>(x);
  x += dpp<0x112, 0xF, 0u>(x);
  x += dpp<0x114, 0xF, 0u>(x);
  x += dpp<0x118, 0xF, 0u>(x);
  x += dpp<0x142, 0xA, 0u>(x);
  x += dpp<0x143, 0xC, 0u>(x);
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp<0x111, 0xF, 0u>(x));
  x = max(x, dpp<0x112, 0xF, 0u>(x));
  x = max(x, dpp<0x114, 0xF, 0u>(x));
  x = max(x, dpp<0x118, 0xF, 0u>(x));
  x = max(x, dpp<0x142, 0xA, 0u>(x));
  x = max(x, dpp<0x143, 0xC, 0u>(x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp<0x111, 0xF, 0xFFFFFFFFu>(x));
  x = min(x, dpp<0x112, 0xF, 0xFFFFFFFFu>(x));
  x = min(x, dpp<0x114, 0xF, 0xFFFFFFFFu>(x));
  x = min(x, dpp<0x118, 0xF, 0xFFFFFFFFu>(x));
  x = min(x, dpp<0x142, 0xA, 0xFFFFFFFFu>(x));
  x = min(x, dpp<0x143, 0xC, 0xFFFFFFFFu>(x));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
__device__ __forceinline__ uint32_t bit_length64(u64 v) { return v ? 64u - __clzll(v) : 0u; }

// Relaxed agent-scope accesses to the workspace: coherent across the XCDs'
// L2 caches; the ordering comes from the release / acquire on the row's
// arrival counter.
template <typename W>
__device__ __forceinline__ void st_agent(W* p, W v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename W>
__device__ __forceinline__ W ld_agent(const W* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory access this wave has issued is complete.
__device__ __forceinline__ void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- LDS
template <int CAP>
struct Smem {
  alignas(16) u64 buf[CAP + 8];       // candidate composites (also the sort's exchange area);
                                      // the last 8 are zero padding for the rank epilogue
  alignas(16) uint32_t hist[kCutBins];  // zero whenever not in use
  u64 side[kRankMax];                 // members of a small boundary bin
  uint32_t wtot[2][NW];               // per-wave counts, alternating by use
  uint32_t wmax[NW];
  uint32_t wscan[2][NW];
  u64 wred[NW];
  u64 wred2[NW];
  uint32_t res[4];
  uint32_t side_n;
  uint32_t cnt_out;
  uint32_t err;
  uint32_t n_cut;                     // cuts back to k made by this workgroup (statistics)
  uint32_t is_last;
  uint32_t zeros;                     // a zero was stored as an output value
  uint32_t rowmax;                    // whole rows: largest key of the chunks after the first
  uint32_t acnt;                      // append_fast: candidates reserved so far
  uint32_t aovf;                      // append_fast: a reservation ran past its limit
  u64 res64;
};

// ---------------------------------------------------------------- block scans
// Exclusive prefix over the lanes of the workgroup and the total.  `par`
// alternates between consecutive calls so that a fast wave never overwrites
// a total a slow wave has yet to read (a barrier separates any two calls with
// the same parity).
template <int CAP>
__device__ __forceinline__ uint32_t block_excl(Smem<CAP>& sm, uint32_t v, int par,
                                               uint32_t* total, uint32_t* wave_base = nullptr) {
  const uint32_t incl = wave_incl_sum(v);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 63) sm.wscan[par][w] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = sm.wscan[par][i];
    before += i < w ? s : 0u;
    tot += s;
  }
  *total = tot;
  if (wave_base) *wave_base = uniform(before);
  return before + incl - v;
}

// Bins in rank order (bin 0 ranks first), BPT of them per lane, lane t owning
// bins [t*BPT, (t+1)*BPT).  Returns the bin b where the running count reaches
// `need`: sum(bins < b) < need <= sum(bins <= b), or kNone when the total is
// below need; then res = {b, sum below b, count of b}.  The total goes to
// *total_out when given.
template <int BPT, int CAP>
__device__ __forceinline__ uint32_t find_rank(Smem<CAP>& sm, const uint32_t (&h)[BPT], uint32_t need,
                                              int par, uint32_t* total_out = nullptr) {
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) s += h[i];
  uint32_t total;
  const uint32_t before = block_excl(sm, s, par, &total);
  if (total_out) *total_out = total;
  // Exactly one lane holds the crossing when total >= need; every reader of
  // an earlier result has passed block_excl's barrier.
  if (before < need && need <= before + s) {
    uint32_t acc = before;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (acc < need && need <= acc + h[i]) {
        sm.res[0] = threadIdx.x * BPT + i;
        sm.res[1] = acc;
        sm.res[2] = h[i];
      }
      acc += h[i];
    }
  }
  __syncthreads();
  return total < need ? kNone : uniform(sm.res[0]);
}


// ---------------------------------------------------------------- chunks
template <bool BF16>
struct Geo {
  static constexpr int EPV = BF16 ? 8 : 4;      // values per 16-byte vector
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int EPL = V * EPV;           // values per lane per chunk
  static constexpr uint32_t CE = NT * EPL;      // values per chunk
};

// Vectors per lane of chunk c that hold a column below L (uniform): vector
// i of every lane lies at or past L for i >= chunk_nv.
template <bool BF16>
__device__ __forceinline__ uint32_t chunk_nv(uint32_t c, uint32_t L) {
  using G = Geo<BF16>;
  constexpr uint32_t VW = NT * G::EPV;   // columns of vector i over the workgroup
  const uint32_t c0 = c * G::CE;
  return L > c0 ? min(static_cast<uint32_t>(V), (L - c0 + VW - 1) / VW) : 0u;
}

// Vectors per lane that load_chunk loads: every vector for split rows (their
// chunks are full but for a row's last), only those below chunk_nv for whole
// rows (a short row's chunk is mostly past L).
template <bool BF16>
__device__ __forceinline__ uint32_t loaded_nv(uint32_t c, uint32_t L) {
  return kSplit ? static_cast<uint32_t>(V) : chunk_nv<BF16>(c, L);
}

// Chunk c of a row: lane t's vector i covers columns c*CE + (i*NT + t)*EPV ...
// Vectors past loaded_nv are not loaded: they hold negative NaNs (the ragged
// padding, see sanitize_ragged).  A vector below it that starts at or past L
// is loaded from column 0 instead (a valid address); its values are replaced
// before use (sanitize_ragged).
template <bool BF16>
__device__ __forceinline__ void load_chunk(u32x4 (&r)[V], const char* xrow, uint32_t c,
                                           uint32_t L) {
  using G = Geo<BF16>;
  const uint32_t e0 = c * G::CE + threadIdx.x * G::EPV;
  const uint32_t nv = loaded_nv<BF16>(c, L);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (static_cast<uint32_t>(i) < nv) {
      uint32_t e = e0 + static_cast<uint32_t>(i * NT * G::EPV);
      e = e < L ? e : 0u;
      r[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(xrow + static_cast<size_t>(e) * G::ESZ));
    } else {
      r[i] = u32x4{~0u, ~0u, ~0u, ~0u};
    }
  }
}

template <bool BF16>
__device__ __forceinline__ uint32_t col_at(uint32_t c, int i, int q) {
  using G = Geo<BF16>;
  // The lane's first column plus a constant, added where it is used (an
  // opaque add the compiler cannot hoist), so the 32-64 column numbers of a
  // chunk are never held in registers at once.
  const uint32_t base = c * G::CE + threadIdx.x * G::EPV;
  const uint32_t off = static_cast<uint32_t>(i * NT * G::EPV + q);
  uint32_t r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(off), "v"(base));
  return r;
}

// Apply f(bits as fp32, value index q) to every value of vector r.
// The low bf16 of a word as an fp32 bit pattern.  Computed where it is used
// (an opaque shift the compiler cannot hoist), so a chunk's 32 shifted words
// are never held in registers across passes.
__device__ __forceinline__ uint32_t lo_half(uint32_t d) {
  uint32_t r;
  asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(d));
  return r;
}

template <bool BF16, typename F>
__device__ __forceinline__ void for_values(const u32x4& r, F&& f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t d = r[w];
    if constexpr (BF16) {
      f(lo_half(d), 2 * w);
      f(d & 0xFFFF0000u, 2 * w + 1);
    } else {
      f(d, w);
    }
  }
}

// The chunk that holds column L-1: returns whether a NaN is among the valid
// values, then replaces every value at or past L by a negative NaN (all bits
// set), which no float compare admits, no histogram counts, and which sits
// below every positive pattern as a signed integer.
template <bool BF16>
__device__ __forceinline__ bool sanitize_ragged(u32x4 (&r)[V], uint32_t c, uint32_t L) {
  bool nan = false;
  const uint32_t nv = loaded_nv<BF16>(c, L);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (static_cast<uint32_t>(i) >= nv) continue;   // padding already (not loaded)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t d = r[i][w];
      if constexpr (BF16) {
        const bool ok0 = col_at<true>(c, i, 2 * w) < L, ok1 = col_at<true>(c, i, 2 * w + 1) < L;
        nan |= ok0 & ((d & 0x7FFFu) > 0x7F80u);
        nan |= ok1 & (((d >> 16) & 0x7FFFu) > 0x7F80u);
        r[i][w] = (ok0 ? (d & 0xFFFFu) : 0xFFFFu) | (ok1 ? (d & 0xFFFF0000u) : 0xFFFF0000u);
      } else {
        const bool ok = col_at<false>(c, i, w) < L;
        nan |= ok & ((d & 0x7FFFFFFFu) > 0x7F800000u);
        r[i][w] = ok ? d : 0xFFFFFFFFu;
      }
    }
  }
  return nan;
}

// Per lane: the key of its largest value (0 if that is a NaN or the lane
// has none) and, with CHECK, whether any value is a NaN.  Integer maxima of
// the raw patterns, two bf16 per instruction: as signed integers the
// non-negative values order like their floats, above every negative one,
// with positive NaNs above +inf; as unsigned integers negative NaNs lie
// above -inf.  A lane whose values are all negative takes its largest as
// the smallest unsigned pattern, on a branch that typical data never takes.
template <bool BF16, bool CHECK>
__device__ __forceinline__ void chunk_max_nan(const u32x4 (&r)[V], uint32_t* maxkey, bool* nan,
                                              uint32_t nv = V) {
  uint32_t top;   // the lane's largest value as an fp32 pattern
  bool bad;
  if constexpr (BF16) {
    // One accumulator per word of a vector: four independent chains.
    i16x2 smax[4];
    u16x2 umax[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      smax[w] = i16x2{-32768, -32768};
      umax[w] = u16x2{0, 0};
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (static_cast<uint32_t>(i) >= nv) continue;   // padding: below every value
        // (a copy first: a bit cast of a vector element in place reads the
        // vector's first element with this compiler)
        const uint32_t d = r[i][w];
        smax[w] = __builtin_elementwise_max(smax[w], __builtin_bit_cast(i16x2, d));
        if (CHECK) umax[w] = __builtin_elementwise_max(umax[w], __builtin_bit_cast(u16x2, d));
      }
    const i16x2 s2 = __builtin_elementwise_max(__builtin_elementwise_max(smax[0], smax[1]),
                                               __builtin_elementwise_max(smax[2], smax[3]));
    const u16x2 u2 = __builtin_elementwise_max(__builtin_elementwise_max(umax[0], umax[1]),
                                               __builtin_elementwise_max(umax[2], umax[3]));
    const int sm = max(static_cast<int>(s2.x), static_cast<int>(s2.y));
    bad = sm > 0x7F80 || max(static_cast<uint32_t>(u2.x), static_cast<uint32_t>(u2.y)) > 0xFF80u;
    top = static_cast<uint32_t>(sm) << 16;
    if (sm < 0) {
      u16x2 umin = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (static_cast<uint32_t>(i) >= nv) continue;
          const uint32_t d = r[i][w];
          umin = __builtin_elementwise_min(umin, __builtin_bit_cast(u16x2, d));
        }
      top = min(static_cast<uint32_t>(umin.x), static_cast<uint32_t>(umin.y)) << 16;
    }
  } else {
    int32_t sa = INT32_MIN, sb = INT32_MIN;
    uint32_t ua = 0, ub = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (static_cast<uint32_t>(i) >= nv) continue;
      sa = max(sa, max(static_cast<int32_t>(r[i][0]), static_cast<int32_t>(r[i][1])));
      sb = max(sb, max(static_cast<int32_t>(r[i][2]), static_cast<int32_t>(r[i][3])));
      if (CHECK) {
        ua = max(ua, max(r[i][0], r[i][1]));
        ub = max(ub, max(r[i][2], r[i][3]));
      }
    }
    const int32_t smax = max(sa, sb);
    bad = smax > 0x7F800000 || max(ua, ub) > 0xFF800000u;
    top = static_cast<uint32_t>(smax);
    if (smax < 0) {
      uint32_t umin = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) if (static_cast<uint32_t>(i) < nv) umin = min(umin, r[i][w]);
      top = umin;
    }
  }
  *nan = CHECK && bad;
  *maxkey = (top & 0x7FFFFFFFu) > 0x7F800000u ? 0u : key_of_bits(top);
}

// Values of the lane >= f (NaN never).
template <bool BF16>
__device__ __forceinline__ uint32_t vec_count(const u32x4& r, float f) {
  uint32_t n = 0;
  for_values<BF16>(r, [&](uint32_t b, int) { n += __uint_as_float(b) >= f ? 1u : 0u; });
  return n;
}

// Write the wave's values of vector i that are >= f to buf[pos ...] in
// slot-major order; a slot that no lane keeps costs one compare.
template <bool BF16, int CAP>
__device__ __forceinline__ uint32_t vec_write(Smem<CAP>& sm, const u32x4& r, int i, uint32_t c,
                                              float f, uint32_t pos) {
  for_values<BF16>(r, [&](uint32_t b, int q) {
    const bool ok = __uint_as_float(b) >= f;
    const u64 m = ballot(ok);
    if (m) {
      if (ok) sm.buf[pos + mbcnt64(m)] = comp_of(key_of_bits(b), col_at<BF16>(c, i, q));
      pos += static_cast<uint32_t>(__popcll(m));
    }
  });
  return pos;
}

// ---------------------------------------------------------------- the start
// Per-group representatives of a vector: for GS > 0, one value of each run
// of GS consecutive values, the group's largest as a signed integer pattern
// (its largest value when it holds a non-negative one, else some member:
// always a member, which is all the start needs).  f(bits as fp32) is called
// once per representative.
template <bool BF16, int GS, typename F>
__device__ __forceinline__ void for_reps(const u32x4& v, F&& f) {
  if constexpr (BF16) {
    const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
    const i16x2 a0 = __builtin_bit_cast(i16x2, w0), a1 = __builtin_bit_cast(i16x2, w1);
    const i16x2 a2 = __builtin_bit_cast(i16x2, w2), a3 = __builtin_bit_cast(i16x2, w3);
    auto bits = [](int x) { return static_cast<uint32_t>(static_cast<uint16_t>(x)) << 16; };
    if constexpr (GS == 8) {
      const i16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                __builtin_elementwise_max(a2, a3));
      f(bits(max(static_cast<int>(m.x), static_cast<int>(m.y))));
    } else if constexpr (GS == 4) {
      const i16x2 m0 = __builtin_elementwise_max(a0, a1), m1 = __builtin_elementwise_max(a2, a3);
      f(bits(max(static_cast<int>(m0.x), static_cast<int>(m0.y))));
      f(bits(max(static_cast<int>(m1.x), static_cast<int>(m1.y))));
    } else if constexpr (GS == 2) {
      f(bits(max(static_cast<int>(a0.x), static_cast<int>(a0.y))));
      f(bits(max(static_cast<int>(a1.x), static_cast<int>(a1.y))));
      f(bits(max(static_cast<int>(a2.x), static_cast<int>(a2.y))));
      f(bits(max(static_cast<int>(a3.x), static_cast<int>(a3.y))));
    } else {
      for_values<true>(v, [&](uint32_t b, int) { f(b); });
    }
  } else {
    const int32_t w0 = static_cast<int32_t>(v[0]), w1 = static_cast<int32_t>(v[1]);
    const int32_t w2 = static_cast<int32_t>(v[2]), w3 = static_cast<int32_t>(v[3]);
    if constexpr (GS >= 4) {
      f(static_cast<uint32_t>(max(max(w0, w1), max(w2, w3))));
    } else if constexpr (GS == 2) {
      f(static_cast<uint32_t>(max(w0, w1)));
      f(static_cast<uint32_t>(max(w2, w3)));
    } else {
      f(v[0]);
      f(v[1]);
      f(v[2]);
      f(v[3]);
    }
  }
}

// The start threshold from a 256-bin histogram over the window of keys just
// below `maxkey` (the chunk's largest key): bin j holds keys
// maxkey - (j+1)*2^s < key <= maxkey - j*2^s.  GS == 0 bins each lane's
// largest value (lane_max), with s = 16 (one bin per bf16 value, 1/128
// octave for fp32), then s = 24 (the window spans every key) when the first
// window holds fewer than m.  GS > 0 bins one representative per group of GS
// values (for_reps), with s = 16, then 20 (16 bf16 values per bin, 32 octaves
// in all), then 24 (split rows: 16, then 24); with `wide`, when the m-th
// value is expected far below the maximum, from 20.  Returns T = (edge key << 32): at least m values of the
// chunk are at or above it (m binned members are, each a distinct value of
// the chunk).  Leaves the histogram zeroed.  Every binned key is at most
// maxkey: a lane maximum is, and a chunk holding a NaN (whose maxkey may lie
// below other lanes' values) does not come here with GS > 0.
template <bool BF16, int GS, int CAP>
__device__ __forceinline__ u64 start_threshold(Smem<CAP>& sm, const u32x4 (&r)[V],
                                               uint32_t maxkey, uint32_t lane_max, uint32_t m,
                                               uint32_t nv, bool wide = false) {
  // (Split rows keep two scales: their start bins lane maxima or small shares.)
  constexpr int NP = (GS == 0 || kSplit) ? 2 : 3;
  for (int pass = (NP == 3 && wide) ? 1 : 0; pass < NP; ++pass) {
    const uint32_t s = pass == 0 ? 16u : (pass == NP - 1 ? 24u : 20u);
    const u64 span = static_cast<u64>(kWinBins) << s;   // keys the window covers
    const uint32_t lo_key = static_cast<u64>(maxkey) - kNegInfKey >= span
                                ? static_cast<uint32_t>(maxkey - span + 1u)
                                : kNegInfKey;
    if constexpr (GS == 0) {
      if (lane_max >= lo_key) atomicAdd(&sm.hist[(maxkey - lane_max) >> s], 1u);
    } else {
      const float flo = __uint_as_float(bits_of_key(lo_key));
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if (static_cast<uint32_t>(i) >= nv) continue;   // padding: binned nowhere
        for_reps<BF16, GS>(r[i], [&](uint32_t b) {
          if (__uint_as_float(b) >= flo) atomicAdd(&sm.hist[(maxkey - key_of_bits(b)) >> s], 1u);
        });
      }
    }
    __syncthreads();
    uint32_t h[1];
    h[0] = sm.hist[threadIdx.x];
    sm.hist[threadIdx.x] = 0u;   // own bin: no other lane touches it until the next barrier
    const uint32_t b = find_rank<1>(sm, h, m, pass & 1);   // parity 0 / 1 (wscan has two rows)
    if (b != kNone) {
      const int64_t e = static_cast<int64_t>(maxkey) - (static_cast<int64_t>(b + 1) << s) + 1;
      const uint32_t edge = e > static_cast<int64_t>(lo_key) ? static_cast<uint32_t>(e) : lo_key;
      return static_cast<u64>(edge) << 32;
    }
    if (lo_key == kNegInfKey) return kTAll;
  }
  return kTAll;   // not reached: the last window spans every key
}

// ---------------------------------------------------------------- the cut
// f(value, valid) over buf[0, n): each lane reads its G slots of a group
// (slot q of lane t is j0 + q*NT + t) back to back before using any.
template <int G, int CAP, typename F>
__device__ __forceinline__ void for_buf(const Smem<CAP>& sm, uint32_t n, F&& f) {
  const uint32_t t = threadIdx.x;
  for (uint32_t j0 = 0; j0 < n; j0 += G * NT) {
    u64 v[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const uint32_t j = j0 + q * NT + t;
      v[q] = sm.buf[j < n ? j : 0u];
    }
#pragma unroll
    for (int q = 0; q < G; ++q) f(v[q], j0 + q * NT + t < n);
  }
}

// Keep exactly the `keep` largest of the n composites in buf (keep < n),
// compacting them to buf[0, keep).  Returns the new threshold, the keep-th
// largest composite.  An MSD radix select over the live composite range:
// each level bins the range in 2048 bins (at most six levels for 64 bits),
// and a boundary bin of at most 64 members is ranked directly.  If a level's
// counts ever disagree with the previous level's (which a correct buffer
// cannot produce) it sets sm.err and leaves the buffer as it is.  Enter and
// leave with the histogram zeroed and after a barrier.
template <int CAP>
__device__ __noinline__ u64 cut_exact(Smem<CAP>& sm, uint32_t n, uint32_t keep) {
  const int t = threadIdx.x;
  if (t == 0) sm.n_cut += 1u;
  // Live range of the composites.
  u64 lo = ~0ull, hi = 0;
  for_buf<8>(sm, n, [&](u64 v, bool ok) {
    if (ok) {
      lo = v < lo ? v : lo;
      hi = v > hi ? v : hi;
    }
  });
  {
    const uint32_t a = wave_min_u32(static_cast<uint32_t>(lo >> 32));
    const uint32_t b = wave_max_u32(static_cast<uint32_t>(hi >> 32));
    // Exact 64-bit extremes: the low words among the lanes that hold the
    // extreme high word.
    const uint32_t al = wave_min_u32(static_cast<uint32_t>(lo >> 32) == a ? static_cast<uint32_t>(lo) : 0xFFFFFFFFu);
    const uint32_t bl = wave_max_u32(static_cast<uint32_t>(hi >> 32) == b ? static_cast<uint32_t>(hi) : 0u);
    if (lane_id() == 0) {
      sm.wred[t >> 6] = (static_cast<u64>(a) << 32) | al;
      sm.wred2[t >> 6] = (static_cast<u64>(b) << 32) | bl;
    }
    __syncthreads();
    u64 l2 = ~0ull, h2 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      l2 = sm.wred[w] < l2 ? sm.wred[w] : l2;
      h2 = sm.wred2[w] > h2 ? sm.wred2[w] : h2;
    }
    lo = uniform64(l2);
    hi = uniform64(h2);
  }

  uint32_t need = keep;
  u64 T = 0;
  bool done = false;
  int par = 0;
  for (int level = 0; level < 6 && !done; ++level) {
    const u64 span = hi - lo;
    const uint32_t bl = bit_length64(span);
    const uint32_t shift = bl > kCutBits ? bl - kCutBits : 0u;
    // Bin 0 holds the largest composites.
    for_buf<8>(sm, n, [&](u64 v, bool ok) {
      if (ok && v >= lo && v <= hi)
        atomicAdd(&sm.hist[(kCutBins - 1) - static_cast<uint32_t>((v - lo) >> shift)], 1u);
    });
    __syncthreads();
    uint32_t h[kCutBPT];
#pragma unroll
    for (int i = 0; i < kCutBPT; ++i) {
      h[i] = sm.hist[t * kCutBPT + i];
      sm.hist[t * kCutBPT + i] = 0u;
    }
    const uint32_t b = find_rank<kCutBPT>(sm, h, need, par);
    par ^= 1;
    if (b == kNone) {   // fewer than `need` in range: inconsistent counts
      if (t == 0) sm.err = 1u;
      return 0;
    }
    const uint32_t below = uniform(sm.res[1]), hb = uniform(sm.res[2]);
    need -= below;
    // Composites of bin b: [blo, bhi].
    const u64 blo = lo + (static_cast<u64>((kCutBins - 1) - b) << shift);
    const u64 bhi_full = blo + ((1ull << shift) - 1ull);
    const u64 bhi = bhi_full < hi ? bhi_full : hi;
    if (hb == need) {   // the whole bin is kept
      T = blo;
      done = true;
    } else if (hb <= kRankMax) {
      // Rank the bin's members directly.
      if (t == 0) sm.side_n = 0u;
      __syncthreads();
      for (uint32_t j0 = 0; j0 < n; j0 += NT) {
        const uint32_t j = j0 + t;
        const u64 v = j < n ? sm.buf[j] : 0ull;
        const bool in = (j < n) & (v >= blo) & (v <= bhi);
        const u64 mk = ballot(in);
        if (mk) {
          uint32_t base = 0;
          if (lane_id() == 0) base = atomicAdd(&sm.side_n, static_cast<uint32_t>(__popcll(mk)));
          base = uniform(base);
          if (in && base + mbcnt64(mk) < kRankMax) sm.side[base + mbcnt64(mk)] = v;
        }
      }
      __syncthreads();
      const uint32_t ns = uniform(sm.side_n);
      if (ns != hb) {
        if (t == 0) sm.err = 1u;
        return 0;
      }
      if (t < 64) {   // wave 0: one member per lane, the others read by readlane
        const u64 mine = static_cast<uint32_t>(t) < ns ? sm.side[t] : 0ull;
        const uint32_t mlo = static_cast<uint32_t>(mine), mhi = static_cast<uint32_t>(mine >> 32);
        uint32_t above = 0;
        for (uint32_t j = 0; j < ns; ++j) {
          const uint32_t olo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mlo), static_cast<int>(j)));
          const uint32_t ohi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mhi), static_cast<int>(j)));
          above += ((static_cast<u64>(ohi) << 32) | olo) > mine ? 1u : 0u;
        }
        if (static_cast<uint32_t>(t) < ns && above + 1u == need) sm.res64 = mine;
      }
      __syncthreads();
      T = uniform64(sm.res64);
      done = true;
    } else if (shift == 0) {   // cannot happen: a bin of width 1 holds one composite
      if (t == 0) sm.err = 1u;
      return 0;
    } else {
      lo = blo;
      hi = bhi;
    }
  }
  if (!done) {
    if (t == 0) sm.err = 1u;
    return 0;
  }
  // Compaction in groups: every lane reads its slots of a group before any
  // write of that group, and a write position never exceeds the number of
  // slots read so far, so no unread slot is overwritten.
  uint32_t out = 0;
  for (uint32_t g0 = 0; g0 < n; g0 += 8 * NT) {
    u64 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t j = g0 + q * NT + t;
      v[q] = j < n ? sm.buf[j] : 0ull;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) cnt += (v[q] >= T) ? 1u : 0u;   // empty slots read 0 < T
    uint32_t total;
    const uint32_t pre = block_excl(sm, cnt, par, &total);   // its barrier orders the reads
    par ^= 1;
    uint32_t pos = out + pre;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (v[q] >= T) sm.buf[pos++] = v[q];
    out += total;
    __syncthreads();
  }
  return T;
}

// ---------------------------------------------------------------- appending a chunk
// Shared state of one workgroup's candidate buffer (all fields uniform).
struct Buf {
  uint32_t count;   // candidates in buf
  u64 T;            // every value of the row (or chunk) with composite >= T is in buf
  int par;          // parity of the next block scan
};

// Append the values of vector i with key >= key(B.T), cutting first when they
// might not fit.  Used when a whole chunk does not fit at once.
template <bool BF16, int CAP>
__device__ __forceinline__ void append_vec(Smem<CAP>& sm, Buf& B, const u32x4& r, int i,
                                           uint32_t c, uint32_t k, uint32_t cap) {
  using G = Geo<BF16>;
  constexpr uint32_t PIECE = NT * G::EPV;
  if (B.count + PIECE > cap && B.count > k) {
    __syncthreads();
    const u64 Tn = cut_exact(sm, B.count, k);
    if (uniform(sm.err)) return;
    B.T = Tn;
    B.count = k;
  }
  const float f = __uint_as_float(bits_of_key(key_of(B.T)));
  const uint32_t n = vec_count<BF16>(r, f);
  uint32_t total, wb;
  block_excl(sm, n, B.par, &total, &wb);
  B.par ^= 1;
  vec_write<BF16>(sm, r, i, c, f, B.count + wb);
  B.count += total;
}

// Append every value of chunk c with key >= key(B.T).  Values at a key equal
// to T's whose column lies past T's are admitted too: harmless, since every
// later step keeps the buffer a superset of the values >= T.
template <bool BF16, int CAP>
__device__ __forceinline__ void append_chunk(Smem<CAP>& sm, Buf& B, const u32x4 (&r)[V], uint32_t c,
                                             uint32_t k, uint32_t cap, uint32_t nv = V) {
  const float f = __uint_as_float(bits_of_key(key_of(B.T)));
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) if (static_cast<uint32_t>(i) < nv) n += vec_count<BF16>(r[i], f);
  uint32_t total, wb;
  block_excl(sm, n, B.par, &total, &wb);
  B.par ^= 1;
  if (B.count + total <= cap) {
    uint32_t pos = B.count + wb;
#pragma unroll
    for (int i = 0; i < V; ++i) if (static_cast<uint32_t>(i) < nv) pos = vec_write<BF16>(sm, r[i], i, c, f, pos);
    B.count += total;
    return;
  }
  // Piecewise: one vector per lane at a time (a cut leaves room for one).
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (static_cast<uint32_t>(i) >= nv) break;
    append_vec<BF16>(sm, B, r[i], i, c, k, cap);
    if (uniform(sm.err)) return;
  }
}

// The first chunk of a workgroup: NaN check and start threshold (into B.T).
// With `exact`, the chunk is a whole row and T is a valid start (at least
// min(k, L) values pass); otherwise T is an estimate of the row's k-th value
// for this chunk's share.  Returns whether a NaN was found.
template <bool BF16, int CAP>
__device__ __forceinline__ bool start_chunk(Smem<CAP>& sm, Buf& B, u32x4 (&r)[V], uint32_t c,
                                            uint32_t L, uint32_t k, bool exact, bool* spec,
                                            uint32_t* top = nullptr) {
  using G = Geo<BF16>;
  const int t = threadIdx.x;
  bool nan = false;
  const bool rag = (c + 1) * G::CE > L;
  if (rag) nan = sanitize_ragged<BF16>(r, c, L);
  const uint32_t nv = loaded_nv<BF16>(c, L);
  uint32_t mk;
  bool nn;
  if (rag) chunk_max_nan<BF16, false>(r, &mk, &nn, nv);
  else chunk_max_nan<BF16, true>(r, &mk, &nn);
  nan |= nn;
  const uint32_t wm = wave_max_u32(mk);
  if (lane_id() == 0) sm.wmax[t >> 6] = wm;
  __syncthreads();
  uint32_t maxkey = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) maxkey = max(maxkey, sm.wmax[w]);
  maxkey = uniform(maxkey);
  if (top) *top = maxkey;
  const uint32_t nvalid = min(G::CE, L - c * G::CE);
  uint32_t m;
  if (exact) {
    m = min(k, L);
  } else {
    // The chunk's expected share of the row's top k plus six standard
    // deviations (its count is hypergeometric, variance below the mean).
    const float E = static_cast<float>(k) * static_cast<float>(nvalid) / static_cast<float>(L);
    const float mf = E + 6.0f * __builtin_sqrtf(E) + 8.0f;
    m = mf >= static_cast<float>(k) ? k : static_cast<uint32_t>(mf) + 1u;
  }
  u64 T = kTAll;
  if (maxkey != 0 && m < nvalid) {
    if (m <= static_cast<uint32_t>(NT / 2)) {
      T = start_threshold<BF16, 0>(sm, r, maxkey, mk, m, nv);
    } else if (!nan) {
      // One representative per group of g values, g the largest power of
      // two (at most one 16-byte vector) that leaves about 3m groups: the
      // m-th largest representative then has about 1.1m values at or above
      // it, at an eighth of the histogram work of binning every value.
      // (Split rows, whose shares are small, bin every value: one variant.)
      const uint32_t q = kSplit ? 0u : nvalid / (3u * m);
      const uint32_t g = q >= 8u && BF16 ? 8u : q >= 4u ? 4u : q >= 2u ? 2u : 1u;
      // More than an eighth of the chunk above the start: the first window
      // (two octaves below the maximum) would rarely hold it.
      const bool wide = 8u * m > nvalid;
      if (!kSplit && g == 8u) T = start_threshold<BF16, 8>(sm, r, maxkey, mk, m, nv, wide);
      else if (!kSplit && g == 4u) T = start_threshold<BF16, 4>(sm, r, maxkey, mk, m, nv, wide);
      else if (!kSplit && g == 2u) T = start_threshold<BF16, 2>(sm, r, maxkey, mk, m, nv, wide);
      else T = start_threshold<BF16, 1>(sm, r, maxkey, mk, m, nv, wide);
    }
  }
  *spec = !exact && m < k && T != kTAll;
  B.T = T;
  return nan;
}

// Write the wave's values that pass `ok` (a test on the raw word d and the
// half h of it) to the region reg of R slots as raw pairs (d << 32) | column;
// `hit` tells whether a 16-byte vector holds a value that passes.  For bf16
// the column's parity tells which half of d is the value.  Returns the
// wave's count (uniform), which exceeds R when the region overflowed (then
// it holds only the first R).
//
// Few vectors hold a candidate (about one lane in sixteen per vector on a
// split row), so the vectors that do are first copied, with their first
// column, to the top of the region, one lane each; the wave then compacts
// their values slot by slot: EPV ballots over the copies instead of EPV
// ballots per vector of every lane.  With more than SM such vectors in the
// wave, or a region too small, the compaction runs over the registers.
template <bool BF16, typename OK, typename HIT>
__device__ __forceinline__ uint32_t region_pass(u64* buf, uint32_t rb, const u32x4 (&r)[V],
                                                uint32_t c, uint32_t R, OK&& ok, HIT&& hit) {
  using G = Geo<BF16>;
  constexpr uint32_t SM = 64;   // copies per wave
  u64* reg = buf + rb;
  bool hl[V];
  u64 hv[V];
  uint32_t nh = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    hl[i] = hit(r[i]);
    hv[i] = ballot(hl[i]);
    nh += static_cast<uint32_t>(__popcll(hv[i]));
  }
  uint32_t pos = 0;
  if (nh <= SM && nh * G::EPV <= R && R >= 3 * SM) {
    // Copies at the top of the region: SM vectors (16-byte aligned), below
    // them SM first columns.  Every copy is read back by one instruction
    // before any candidate is written, so the candidates, written from the
    // region's start, may overwrite them.
    u32x4* st = reinterpret_cast<u32x4*>(buf + ((rb + R - 2 * SM) & ~1u));
    uint32_t* stc = reinterpret_cast<uint32_t*>(st) - SM;
    const uint32_t col0 = c * G::CE + threadIdx.x * G::EPV;
    uint32_t sp = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (hv[i]) {
        if (hl[i]) {
          const uint32_t j = sp + mbcnt64(hv[i]);
          st[j] = r[i];
          stc[j] = col0 + static_cast<uint32_t>(i * NT * G::EPV);
        }
        sp += static_cast<uint32_t>(__popcll(hv[i]));
      }
    }
    // Lanes past the copies hold negative NaNs, which pass no test.
    u32x4 v = {~0u, ~0u, ~0u, ~0u};
    uint32_t cb = 0;
    if (lane_id() < sp) {
      v = st[lane_id()];
      cb = stc[lane_id()];
    }
#pragma unroll
    for (int q = 0; q < G::EPV; ++q) {
      const uint32_t d = v[BF16 ? q >> 1 : q];
      const bool p = ok(d, q & 1);
      const u64 m = ballot(p);
      if (m) {
        if (p) reg[pos + mbcnt64(m)] = (static_cast<u64>(d) << 32) | (cb + static_cast<uint32_t>(q));
        pos += static_cast<uint32_t>(__popcll(m));
      }
    }
    return pos;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (!hv[i]) continue;
    if (pos + 64u * G::EPV <= R) {   // the whole vector fits whatever passes
#pragma unroll
      for (int q = 0; q < G::EPV; ++q) {
        const uint32_t d = r[i][BF16 ? q >> 1 : q];
        const bool p = ok(d, q & 1);
        const u64 m = ballot(p);
        if (m) {
          if (p) reg[pos + mbcnt64(m)] = (static_cast<u64>(d) << 32) | col_at<BF16>(c, i, q);
          pos += static_cast<uint32_t>(__popcll(m));
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < G::EPV; ++q) {
        const uint32_t d = r[i][BF16 ? q >> 1 : q];
        const bool p = ok(d, q & 1);
        const u64 m = ballot(p);
        if (m) {
          const uint32_t at = pos + mbcnt64(m);
          if (p && at < R) reg[at] = (static_cast<u64>(d) << 32) | col_at<BF16>(c, i, q);
          pos += static_cast<uint32_t>(__popcll(m));
        }
      }
    }
  }
  return pos;
}

// A raw pair of region_pass as a composite.
template <bool BF16>
__device__ __forceinline__ u64 comp_of_raw(u64 pr) {
  const uint32_t d = static_cast<uint32_t>(pr >> 32), col = static_cast<uint32_t>(pr);
  uint32_t b = d;
  if constexpr (BF16) b = (col & 1u) ? (d & 0xFFFF0000u) : (d << 16);
  return comp_of(key_of_bits(b), col);
}

// Write the wave's values >= f of a chunk to its own region of buf (R slots
// from w*R) as raw pairs.  Returns the wave's count (uniform), which exceeds
// R when the region overflowed (then it holds only the first R).  For bf16
// and f > 0 the test is an integer compare of each half's pattern with the
// smallest bf16 pattern >= f (positive floats order like their patterns,
// every negative one and the ragged padding lie below); else a float compare.
template <bool BF16, int CAP>
__device__ __forceinline__ uint32_t region_write(Smem<CAP>& sm, const u32x4 (&r)[V], uint32_t c,
                                                 float f, uint32_t R) {
  const uint32_t rb = uniform(threadIdx.x >> 6) * R;   // the wave's region: buf[rb, rb + R)
  const uint32_t fb = __float_as_uint(f);
  if constexpr (BF16) {
    if (static_cast<int32_t>(fb) > 0) {
      const uint32_t tb = (fb + 0xFFFFu) >> 16;
      const int16_t tlo = static_cast<int16_t>(tb);
      const int32_t thi = static_cast<int32_t>(tb << 16);
      return region_pass<true>(
          sm.buf, rb, r, c, R,
          [&](uint32_t d, int h) { return h ? static_cast<int32_t>(d) >= thi : static_cast<int16_t>(d) >= tlo; },
          [&](const u32x4& v) {
            const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
            const i16x2 a = __builtin_elementwise_max(__builtin_bit_cast(i16x2, w0), __builtin_bit_cast(i16x2, w1));
            const i16x2 b = __builtin_elementwise_max(__builtin_bit_cast(i16x2, w2), __builtin_bit_cast(i16x2, w3));
            const i16x2 m = __builtin_elementwise_max(a, b);
            return max(m.x, m.y) >= tlo;
          });
    }
    const auto ok = [&](uint32_t d, int h) { return __uint_as_float(h ? (d & 0xFFFF0000u) : lo_half(d)) >= f; };
    return region_pass<true>(sm.buf, rb, r, c, R, ok, [&](const u32x4& v) {
      bool any = false;
#pragma unroll
      for (int q = 0; q < 8; ++q) any |= ok(v[q >> 1], q & 1);
      return any;
    });
  } else {
    return region_pass<false>(
        sm.buf, rb, r, c, R, [&](uint32_t d, int) { return __uint_as_float(d) >= f; },
        [&](const u32x4& v) {
          return fmaxf(fmaxf(__uint_as_float(v[0]), __uint_as_float(v[1])),
                       fmaxf(__uint_as_float(v[2]), __uint_as_float(v[3]))) >= f;
        });
  }
}

// Append every value of chunk c with key >= key(B.T), without a count pass:
// each wave tests each 16-byte vector once (its largest value against T),
// copies the vectors that hold a candidate, with their first column, to a
// staging area of its own at the top of buf (64 at a time), and compacts
// their values slot by slot, reserving room for each batch with one LDS
// atomic.  Candidates go to buf[B.count, lim), lim leaving the staging areas
// free.  Returns false, with B unchanged and buf past B.count undefined,
// when they would not fit there (or the buffer already reaches lim): the
// caller then appends the chunk the counted way (append_chunk), which cuts
// as it goes.
template <bool BF16, int CAP>
__device__ __forceinline__ bool append_fast(Smem<CAP>& sm, Buf& B, const u32x4 (&r)[V], uint32_t c,
                                            uint32_t cap, uint32_t nv) {
  using G = Geo<BF16>;
  constexpr uint32_t SM = 64;                  // staged vectors per wave
  constexpr uint32_t STG = SM * 2 + SM / 2;    // u64 slots per wave: vectors, then columns
  constexpr uint32_t TOP = (CAP - NW * STG) & ~1u;
  static_assert(CAP > NW * STG, "staging fits in the buffer");
  const uint32_t lim = min(cap, TOP);
  // The staging areas lie above lim: a buffer already past it (filled by
  // append_chunk) holds candidates there.
  if (B.count >= lim) return false;
  const int t = threadIdx.x;
  if (t == 0) {
    sm.acnt = B.count;
    sm.aovf = 0u;
  }
  __syncthreads();
  const uint32_t w = static_cast<uint32_t>(t) >> 6;
  u32x4* sv = reinterpret_cast<u32x4*>(sm.buf + TOP + w * STG);
  uint32_t* sc = reinterpret_cast<uint32_t*>(sm.buf + TOP + w * STG + 2 * SM);
  const float f = __uint_as_float(bits_of_key(key_of(B.T)));
  const uint32_t fb = __float_as_uint(f);
  // bf16 above zero: integer compares of each half's pattern with the
  // smallest bf16 pattern >= f (positive floats order like their patterns;
  // negative values and the ragged padding lie below).  Else float compares.
  const bool ipath = BF16 && static_cast<int32_t>(fb) > 0;
  const uint32_t tb = (fb + 0xFFFFu) >> 16;
  const int16_t tlo = static_cast<int16_t>(tb);
  const int32_t thi = static_cast<int32_t>(tb << 16);
  auto val_bits = [&](uint32_t d, int h) -> uint32_t {
    if constexpr (BF16) return h ? (d & 0xFFFF0000u) : lo_half(d);
    else return d;
  };
  auto ok = [&](uint32_t d, int h) -> bool {
    if (BF16 && ipath) return h ? static_cast<int32_t>(d) >= thi : static_cast<int16_t>(d) >= tlo;
    return __uint_as_float(val_bits(d, h)) >= f;
  };
  auto hit = [&](const u32x4& v) -> bool {
    if constexpr (BF16) {
      if (ipath) {
        const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
        const i16x2 a = __builtin_elementwise_max(__builtin_bit_cast(i16x2, w0), __builtin_bit_cast(i16x2, w1));
        const i16x2 b = __builtin_elementwise_max(__builtin_bit_cast(i16x2, w2), __builtin_bit_cast(i16x2, w3));
        const i16x2 mx = __builtin_elementwise_max(a, b);
        return max(mx.x, mx.y) >= tlo;
      }
      bool any = false;
#pragma unroll
      for (int q = 0; q < 8; ++q) any |= ok(v[q >> 1], q & 1);
      return any;
    } else {
      return fmaxf(fmaxf(__uint_as_float(v[0]), __uint_as_float(v[1])),
                   fmaxf(__uint_as_float(v[2]), __uint_as_float(v[3]))) >= f;
    }
  };
  // The key of a passing value: above zero on the integer path, where the
  // offset-binary key is the pattern with the sign bit set.
  auto key_at = [&](uint32_t d, int h) -> uint32_t {
    if (BF16 && ipath) return (h ? (d & 0xFFFF0000u) : (d << 16)) | kBias;
    return key_of_bits(val_bits(d, h));
  };
  // Compact the wave's nh staged vectors (one per lane; lanes past them hold
  // negative NaNs, which pass no test): each lane writes its own passing
  // values one after another from its place in the wave's prefix sum.
  auto flush = [&](uint32_t nh) {
    u32x4 v = {~0u, ~0u, ~0u, ~0u};
    uint32_t cb = 0;
    if (lane_id() < nh) {
      v = sv[lane_id()];
      cb = sc[lane_id()];
    }
    uint32_t pbits = 0;
#pragma unroll
    for (int q = 0; q < G::EPV; ++q) pbits |= ok(v[BF16 ? q >> 1 : q], q & 1) ? (1u << q) : 0u;
    const uint32_t cnt = static_cast<uint32_t>(__builtin_popcount(pbits));
    const uint32_t incl = wave_incl_sum(cnt);
    const uint32_t tot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
    uint32_t base = 0;
    if (lane_id() == 0) base = atomicAdd(&sm.acnt, tot);
    base = uniform(base);
    if (base + tot > lim) {
      if (lane_id() == 0) sm.aovf = 1u;
      return;
    }
    uint32_t pos = base + incl - cnt;
#pragma unroll
    for (int q = 0; q < G::EPV; ++q) {
      if ((pbits >> q) & 1u) {
        sm.buf[pos] = comp_of(key_at(v[BF16 ? q >> 1 : q], q & 1), cb + static_cast<uint32_t>(q));
        ++pos;
      }
    }
  };
  const uint32_t col0 = c * G::CE + static_cast<uint32_t>(t) * G::EPV;
  uint32_t nh = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (static_cast<uint32_t>(i) >= nv) continue;   // padding: no candidate
    const bool hl = hit(r[i]);
    const u64 hv = ballot(hl);
    if (hv) {
      const uint32_t nv = static_cast<uint32_t>(__popcll(hv));
      if (nh + nv > SM) {
        flush(nh);
        nh = 0;
      }
      if (hl) {
        const uint32_t j = nh + mbcnt64(hv);
        sv[j] = r[i];
        sc[j] = col0 + static_cast<uint32_t>(i * NT * G::EPV);
      }
      nh += nv;
    }
  }
  if (nh) flush(nh);
  __syncthreads();
  const uint32_t n = uniform(sm.acnt), bad = uniform(sm.aovf);
  if (bad) return false;
  B.count = n;
  return true;
}

// A later chunk of a whole row.
template <bool BF16, int CAP>
__device__ __forceinline__ bool next_chunk(Smem<CAP>& sm, Buf& B, u32x4 (&r)[V], uint32_t c,
                                           uint32_t L, uint32_t k, uint32_t cap) {
  using G = Geo<BF16>;
  bool nan = false;
  uint32_t mk;
  bool nn;
  if ((c + 1) * G::CE > L) {
    nan = sanitize_ragged<BF16>(r, c, L);
    chunk_max_nan<BF16, false>(r, &mk, &nn, chunk_nv<BF16>(c, L));
  } else {
    chunk_max_nan<BF16, true>(r, &mk, &nn);
    nan = nn;
  }
  // The row's largest key, for the epilogue's range (read after a barrier).
  const uint32_t wm = wave_max_u32(mk);
  if (lane_id() == 0) atomicMax(&sm.rowmax, wm);
  const uint32_t nv = chunk_nv<BF16>(c, L);
  if (!append_fast<BF16>(sm, B, r, c, cap, nv)) append_chunk<BF16>(sm, B, r, c, k, cap, nv);
  return nan;
}

// The row read again, in order, from T = every value (a start estimate that
// turned out too high).  The NaN check was done on the first read.
template <bool BF16, int CAP>
__device__ __noinline__ Buf restream(Smem<CAP>& sm, int par, const char* xrow, uint32_t L,
                                     uint32_t k, uint32_t cap) {
  using G = Geo<BF16>;
  const uint32_t nch = (L + G::CE - 1) / G::CE;
  Buf B{0u, kTAll, par};
  __syncthreads();
  for (uint32_t j = 0; j < nch; ++j) {
    u32x4 r[V];
    load_chunk<BF16>(r, xrow, j, L);
    if ((j + 1) * G::CE > L) sanitize_ragged<BF16>(r, j, L);
    append_chunk<BF16>(sm, B, r, j, k, cap, chunk_nv<BF16>(j, L));
    if (uniform(sm.err)) break;
  }
  return B;
}

// Chunk c appended again, contiguously, from its bytes in memory, starting
// from B (its threshold kept): the rare path of a split row's chunk whose
// candidates overflowed their per-wave regions.  Out of line, so that no
// register of the first pass has to live across it.
template <bool BF16, int CAP>
__device__ __noinline__ Buf reappend_chunk(Smem<CAP>& sm, Buf B, const char* xrow, uint32_t c,
                                           uint32_t L, uint32_t k, uint32_t cap) {
  using G = Geo<BF16>;
  u32x4 r[V];
  load_chunk<BF16>(r, xrow, c, L);
  if ((c + 1) * G::CE > L) sanitize_ragged<BF16>(r, c, L);
  __syncthreads();
  B.count = 0;
  append_chunk<BF16>(sm, B, r, c, k, cap, chunk_nv<BF16>(c, L));
  return B;
}

// ---------------------------------------------------------------- the sort
// Value of lane (lane ^ X), on the VALU: DPP quad permutes for 1 and 2, row
// shifts for 4 and 8 (each half of a 8- or 16-lane group reads the other
// half), and the gfx950 permlane swaps for 16 and 32 (which pair up rows and
// halves of the wave).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int X>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const uint32_t lane = lane_id();
  if constexpr (X == 1) {
    return dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  } else if constexpr (X == 2) {
    return dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  } else if constexpr (X == 4) {
    const uint32_t up = dpp_mov<0x104>(v), down = dpp_mov<0x114>(v);   // row_shl:4, row_shr:4
    return (lane & 4u) ? down : up;
  } else if constexpr (X == 8) {
    const uint32_t up = dpp_mov<0x108>(v), down = dpp_mov<0x118>(v);   // row_shl:8, row_shr:8
    return (lane & 8u) ? down : up;
  } else if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16u) ? r[0] : r[1];
  } else {
    static_assert(X == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32u) ? r[0] : r[1];
  }
}
template <int X>
__device__ __forceinline__ u64 xor_lane(u64 v) {
  return (static_cast<u64>(xor_lane<X>(static_cast<uint32_t>(v >> 32))) << 32) |
         xor_lane<X>(static_cast<uint32_t>(v));
}

// Bitonic sort, descending, of PER*NT keys (32- or 64-bit); lane t holds
// elements t*PER .. t*PER+PER-1.  Before the merge of blocks of `size`, the
// keys of every block that must come out ascending are complemented, so each
// compare-exchange of the merge puts the larger key at the lower position;
// the next merge's complement pattern replaces this one, and the last merge
// (one block) complements nothing.  Strides below PER stay in registers,
// strides up to 32*PER cross lanes on the VALU, larger strides cross waves
// through `xch` (PER*NT keys of LDS).
// The larger (keep_max) or the smaller of v and o.  For 64-bit keys one
// compare serves both choices.
__device__ __forceinline__ uint32_t pick(uint32_t v, uint32_t o, bool keep_max) {
  return keep_max ? max(v, o) : min(v, o);
}
__device__ __forceinline__ u64 pick(u64 v, u64 o, bool keep_max) {
  return ((v > o) == keep_max) ? v : o;
}

template <int PER, int S, typename K>
__device__ __forceinline__ void bitonic_in_lane(K (&v)[PER]) {
  K a[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) a[i] = v[i];
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if ((i | S) < PER) v[i] = pick(a[i], a[i ^ S], (i & S) == 0);
}
// The stage's exchanges first, then its compares: the PER independent chains
// interleave instead of waiting on one another.
template <int PER, int X, typename K>
__device__ __forceinline__ void bitonic_cross_lane(K (&v)[PER]) {
  const bool lower = (lane_id() & X) == 0;
  K o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = xor_lane<X>(v[i]);
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = pick(v[i], o[i], lower);
}
// One stage of the merge of blocks of SIZE: compare-exchange at distance
// STRIDE, then the next stage down to distance 1 (all resolved at compile
// time, so every stage is straight-line code).
template <typename K, int PER, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stage(K (&v)[PER], K* xch) {
  if constexpr (STRIDE < PER) {
    bitonic_in_lane<PER, STRIDE>(v);
  } else if constexpr (STRIDE < 64 * PER) {
    bitonic_cross_lane<PER, STRIDE / PER>(v);
  } else {
    const uint32_t t = threadIdx.x;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) xch[t * PER + i] = v[i];
    __syncthreads();
    K o[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = xch[(t * PER + i) ^ STRIDE];
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = pick(v[i], o[i], ((t * PER + i) & STRIDE) == 0);
  }
  if constexpr (STRIDE > 1) bitonic_stage<K, PER, SIZE, STRIDE / 2>(v, xch);
}

// The merges of blocks of SIZE, 2*SIZE, ... N.  Before the merge of blocks of
// SIZE, the keys of every block that must come out ascending (element e with
// e & SIZE set) are complemented, so each compare-exchange of the merge puts
// the larger key at the lower position; the pattern of the previous merge
// (e & SIZE/2) is undone in the same step.  The last merge (one block)
// complements nothing.
template <typename K, int PER, int SIZE>
__device__ __forceinline__ void bitonic_merges(K (&v)[PER], K* xch) {
  constexpr int N = PER * NT;
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t e = t * PER + i;
    const bool was = SIZE > 2 && (e & (SIZE / 2)) != 0;
    const bool now = SIZE < N && (e & SIZE) != 0;
    if (was != now) v[i] = ~v[i];
  }
  bitonic_stage<K, PER, SIZE, SIZE / 2>(v, xch);
  if constexpr (SIZE < N) bitonic_merges<K, PER, SIZE * 2>(v, xch);
}

// Bitonic sort, descending, of PER*NT keys (32- or 64-bit); lane t holds
// elements t*PER .. t*PER+PER-1.  Strides below PER stay in registers,
// strides up to 32*PER cross lanes on the VALU, larger strides cross waves
// through `xch` (PER*NT keys of LDS).
template <typename K, int PER>
__device__ __forceinline__ void sort_desc(K (&v)[PER], K* xch) {
  bitonic_merges<K, PER, 2>(v, xch);
  __syncthreads();
}

// ---------------------------------------------------------------- outputs
__device__ __forceinline__ bool store_one(const CArgs& a, bool bf16, const char* xrow, int64_t o,
                                          u64 c, bool valid, uint32_t status) {
  (void)xrow;
  uint32_t ix, v;
  bool zero = false;
  if (valid) {
    ix = col_of(c);
    const uint32_t key = key_of(c);
    // Both zeros share a key; +0 is stored and fix_zero_signs restores a -0
    // from the input afterwards (no load here, so the stores never wait).
    zero = key == kBias;
    v = zero ? 0u : bits_of_key(key);
  } else {
    ix = 0xFFFFFFFFu;
    v = status ? kQNaN32 : kNegInf32;
  }
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
  return zero && a.return_values;
}

// After a barrier that follows a row's stores: every output value stored as
// +0 takes the zero's sign from the input (its index was stored beside it).
__device__ __forceinline__ void fix_zero_signs(const CArgs& a, bool bf16, const char* xrow,
                                            int64_t out0, uint32_t m) {
  for (uint32_t e = threadIdx.x; e < m; e += NT) {
    const int64_t o = out0 + e;
    const uint32_t vb = bf16 ? static_cast<uint32_t>(static_cast<const uint16_t*>(a.values)[o])
                             : static_cast<const uint32_t*>(a.values)[o];
    if (vb != 0u) continue;
    const uint32_t ix = a.idx64 ? static_cast<uint32_t>(static_cast<const int64_t*>(a.indices)[o])
                                : static_cast<uint32_t>(static_cast<const int32_t*>(a.indices)[o]);
    if (bf16) {
      const uint16_t xb = reinterpret_cast<const uint16_t*>(xrow)[ix];
      if (xb != 0u) static_cast<uint16_t*>(a.values)[o] = xb;
    } else {
      const uint32_t xb = reinterpret_cast<const uint32_t*>(xrow)[ix];
      if (xb != 0u) static_cast<uint32_t*>(a.values)[o] = xb;
    }
  }
}

// Sort keys of a composite: by value the composite itself, by column
// (~column << 32) | key; with 32-bit keys (bf16 values, columns below 2^16)
// the top 16 bits of the key and the low 16 of ~column.
template <typename K>
__device__ __forceinline__ K sort_key(u64 c, bool by_col) {
  if constexpr (sizeof(K) == 8) {
    return by_col ? ((static_cast<u64>(static_cast<uint32_t>(c)) << 32) | key_of(c)) : c;
  } else {
    const uint32_t hi = key_of(c) >> 16, lo = static_cast<uint32_t>(c) & 0xFFFFu;
    return by_col ? ((lo << 16) | hi) : ((hi << 16) | lo);
  }
}
template <typename K>
__device__ __forceinline__ u64 comp_of_sort_key(K s, bool by_col) {
  if constexpr (sizeof(K) == 8) {
    return by_col ? ((static_cast<u64>(static_cast<uint32_t>(s)) << 32) | static_cast<uint32_t>(s >> 32)) : s;
  } else {
    const uint32_t hi = by_col ? (s & 0xFFFFu) : (s >> 16);
    const uint32_t lo = by_col ? (s >> 16) : (s & 0xFFFFu);
    return (static_cast<u64>(hi << 16) << 32) | (0xFFFF0000u | lo);
  }
}

template <typename K, int PER, int CAP>
__device__ __forceinline__ void sort_and_store(Smem<CAP>& sm, const CArgs& a, bool bf16,
                                               const char* xrow, int64_t out0, uint32_t m,
                                               uint32_t status) {
  const uint32_t t = threadIdx.x;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const bool by_col = a.sorted == 2;
  K v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t e = t * PER + i;
    v[i] = e < m ? sort_key<K>(sm.buf[e], by_col) : K(0);
  }
  sort_desc<K, PER>(v, reinterpret_cast<K*>(sm.buf));
  bool z = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t e = t * PER + i;
    if (e < k) z |= store_one(a, bf16, xrow, out0 + e, comp_of_sort_key<K>(v[i], by_col), e < m, status);
  }
  if (z) sm.zeros = 1u;
}

// Rank selection: the exact output position of every candidate, without a
// cut or a sort.  One 2048-bin histogram over the candidates' composite range
// [lo, hi] (bin 0 the largest) gives each bin its first position; the
// candidates are scattered into their bins, and each one's rank is its bin's
// first position plus the number of its bin-mates above it.  A candidate of
// rank below m is stored at output position `rank` (value order), the rest are
// dropped.  Returns false, having stored nothing, when there are fewer than m
// candidates or a bin holds more than kBinRankMax of them (long runs of equal
// values; the caller then cuts and sorts).  The count goes to *n_out when
// given.  Needs a count <= RPT * NT.
constexpr uint32_t kBinRankMax = 128;
constexpr int kRankPerLane = 4096 / NT;

template <int CAP>
__device__ __forceinline__ bool rank_core(Smem<CAP>& sm, const CArgs& a, bool bf16,
                                          const char* xrow, int64_t out0, u64 (&v)[kRankPerLane],
                                          uint32_t nit, uint32_t m, uint32_t status,
                                          u64 lo_in = 0, u64 hi_in = 0, uint32_t* n_out = nullptr) {
  constexpr int RPT = kRankPerLane;
  const uint32_t t = threadIdx.x;
  u64 lo = hi_in != 0 ? lo_in : ~0ull, hi = hi_in;
  if (hi_in == 0) {   // else a known range holding every candidate
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit) {
    if (v[i] != 0ull) {
      lo = v[i] < lo ? v[i] : lo;
      hi = v[i] > hi ? v[i] : hi;
    }
  }
  {
    const uint32_t a0 = wave_min_u32(static_cast<uint32_t>(lo >> 32));
    const uint32_t b0 = wave_max_u32(static_cast<uint32_t>(hi >> 32));
    const uint32_t al = wave_min_u32(static_cast<uint32_t>(lo >> 32) == a0 ? static_cast<uint32_t>(lo) : 0xFFFFFFFFu);
    const uint32_t bl = wave_max_u32(static_cast<uint32_t>(hi >> 32) == b0 ? static_cast<uint32_t>(hi) : 0u);
    if (lane_id() == 0) {
      sm.wred[t >> 6] = (static_cast<u64>(a0) << 32) | al;
      sm.wred2[t >> 6] = (static_cast<u64>(b0) << 32) | bl;
    }
    __syncthreads();
    u64 l2 = ~0ull, h2 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      l2 = sm.wred[w] < l2 ? sm.wred[w] : l2;
      h2 = sm.wred2[w] > h2 ? sm.wred2[w] : h2;
    }
    lo = uniform64(l2);
    hi = uniform64(h2);
  }
  }
  // Bins over the composites' range.  bf16 values of rows of at most 2^16
  // columns repeat often; their composites are binned in a 32-bit form
  // (the value's 16 key bits, then the low 16 bits of ~column), which orders
  // them the same way but spreads a run of equal values over the column bits.
  const bool narrow = bf16 && a.n_cols <= 65536;
  auto red = [&](u64 x) -> u64 {
    return narrow ? ((static_cast<u64>(key_of(x) >> 16) << 16) | (static_cast<uint32_t>(x) & 0xFFFFu)) : x;
  };
  const u64 rlo = red(lo);
  const uint32_t bl = bit_length64(red(hi) - rlo);
  const uint32_t shift = bl > kCutBits ? bl - kCutBits : 0u;
  auto bin_of = [&](u64 x) { return (kCutBins - 1) - static_cast<uint32_t>((red(x) - rlo) >> shift); };
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit)
    if (v[i] != 0ull) atomicAdd(&sm.hist[bin_of(v[i])], 1u);
  __syncthreads();
  // Own bins: the largest, then each bin's first position.
  uint32_t h[kCutBPT], sum = 0, big = 0;
#pragma unroll
  for (int i = 0; i < kCutBPT; ++i) {
    h[i] = sm.hist[t * kCutBPT + i];
    sum += h[i];
    big = max(big, h[i]);
  }
  big = wave_max_u32(big);
  if (lane_id() == 0) sm.wmax[t >> 6] = big;
  uint32_t total;
  uint32_t run = block_excl(sm, sum, 0, &total);   // its barrier also publishes wmax
  const uint32_t n = total;
  if (n_out) *n_out = n;
#pragma unroll
  for (int w = 0; w < NW; ++w) big = max(big, sm.wmax[w]);
  if (n < m || uniform(big) > kBinRankMax) {
#pragma unroll
    for (int i = 0; i < kCutBPT; ++i) sm.hist[t * kCutBPT + i] = 0u;
    __syncthreads();
    return false;
  }
#pragma unroll
  for (int i = 0; i < kCutBPT; ++i) {
    sm.hist[t * kCutBPT + i] = run;
    run += h[i];
  }
  __syncthreads();
  bool z = false;
  if (narrow) {
    // The same scatter and ranking on the 32-bit form, which is exact for
    // these rows (16 key bits, then 16 column bits): half the LDS words read
    // per bin-mate and one compare each.  A kept candidate's composite is
    // rebuilt from it: a bf16 value's key (offset binary of its fp32
    // pattern) has zero low 16 bits, whatever the sign, and the column is
    // 0xFFFF minus the low 16 bits.
    uint32_t* b32 = reinterpret_cast<uint32_t*>(sm.buf);
    const uint32_t rlo32 = static_cast<uint32_t>(rlo);
    auto bin32 = [&](uint32_t x) { return (kCutBins - 1) - ((x - rlo32) >> shift); };
#pragma unroll
    for (int i = 0; i < RPT; ++i) if (i < nit)
      if (v[i] != 0ull) {
        const uint32_t x = static_cast<uint32_t>(red(v[i]));
        b32[atomicAdd(&sm.hist[bin32(x)], 1u)] = x;
      }
    if (t < 8) b32[n + t] = 0u;   // below every 32-bit form (keys of values are >= 0x0080 << 16)
    __syncthreads();
    const uint32_t npos = uniform((n + NT - 1) / NT);
#pragma unroll
    for (int g = 0; g < RPT; g += 8) if (static_cast<uint32_t>(g) < npos) {
      constexpr int RB = 8;
      uint32_t x[RB], st[RB], en[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint32_t p = (g + i) * NT + t;
        x[i] = b32[p < n ? p : 0u];
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint32_t b = bin32(x[i]);
        st[i] = b ? sm.hist[b - 1] : 0u;
        en[i] = sm.hist[b];
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint32_t p = (g + i) * NT + t;
        if (p >= n) continue;
        uint32_t r = st[i];
        if (en[i] - st[i] > 1u) {
          for (uint32_t q0 = st[i]; q0 < en[i]; q0 += 8) {
            uint32_t y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = b32[q0 + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) r += y[j] > x[i] ? 1u : 0u;
          }
        }
        if (r < m) {
          const uint32_t key = x[i] & 0xFFFF0000u;
          z |= store_one(a, bf16, xrow, out0 + r, comp_of(key, 0xFFFFu - (x[i] & 0xFFFFu)), true, status);
        }
      }
    }
    if (z) sm.zeros = 1u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCutBPT; ++i) sm.hist[t * kCutBPT + i] = 0u;
    return true;
  }
  // Scatter: afterwards hist[b] is the end of bin b, and bin b starts where
  // bin b-1 ends (bin 0 at 0).
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit)
    if (v[i] != 0ull) sm.buf[atomicAdd(&sm.hist[bin_of(v[i])], 1u)] = v[i];
  if (t < 8) sm.buf[n + t] = 0ull;
  __syncthreads();
  // Rank within the bin: the number of members above, read eight positions
  // at a time from the bin's start.  Positions past the bin's end hold lower
  // bins, whose members are all smaller, and past n the zero padding, so the
  // reads need no bound.  Positions are taken eight per lane at a time, each
  // batch's values and bin bounds read together.
  const uint32_t npos = uniform((n + NT - 1) / NT);
#pragma unroll
  for (int g = 0; g < RPT; g += 8) if (static_cast<uint32_t>(g) < npos) {
    constexpr int RB = 8;
    u64 x[RB];
    uint32_t st[RB], en[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t p = (g + i) * NT + t;
      x[i] = sm.buf[p < n ? p : 0u];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t b = bin_of(x[i]);
      st[i] = b ? sm.hist[b - 1] : 0u;
      en[i] = sm.hist[b];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t p = (g + i) * NT + t;
      if (p >= n) continue;
      uint32_t r = st[i];
      if (en[i] - st[i] > 1u) {
        for (uint32_t q0 = st[i]; q0 < en[i]; q0 += 8) {   // eight reads in flight
          u64 y[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = sm.buf[q0 + j];
#pragma unroll
          for (int j = 0; j < 8; ++j) r += y[j] > x[i] ? 1u : 0u;
        }
      }
      if (r < m) z |= store_one(a, bf16, xrow, out0 + r, x[i], true, status);
    }
  }
  if (z) sm.zeros = 1u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCutBPT; ++i) sm.hist[t * kCutBPT + i] = 0u;
  return true;
}

// rank_core over buf[0, n).
template <int CAP>
__device__ __forceinline__ bool rank_store(Smem<CAP>& sm, const CArgs& a, bool bf16,
                                           const char* xrow, int64_t out0, uint32_t n, uint32_t m,
                                           uint32_t status, u64 lo_in = 0, u64 hi_in = 0) {
  const uint32_t t = threadIdx.x;
  // Iterations past the last candidate are skipped as a whole (n is uniform).
  const uint32_t nit = uniform((n + NT - 1) / NT);
  u64 v[kRankPerLane];
#pragma unroll
  for (int i = 0; i < kRankPerLane; ++i) if (i < nit) {
    const uint32_t j = i * NT + t;
    v[i] = j < n ? sm.buf[j] : 0ull;
  }
  return rank_core(sm, a, bf16, xrow, out0, v, nit, m, status, lo_in, hi_in);
}

// Selection without order (unsorted output): the m largest of buf[0, n)
// stored in any order.  The candidates stay in registers; one 2048-bin
// histogram over their composite range finds the boundary bin, whose members
// (at most kRankMax, else false is returned with nothing stored) are ranked
// by one wave; every candidate at or above the m-th is stored at a position
// taken from a per-wave counter.  Needs n <= kRankPerLane * NT.
template <int CAP>
__device__ __forceinline__ bool select_core(Smem<CAP>& sm, const CArgs& a, bool bf16,
                                            const char* xrow, int64_t out0, u64 (&v)[kRankPerLane],
                                            uint32_t nit, uint32_t m, uint32_t status,
                                            u64 lo_in = 0, u64 hi_in = 0, uint32_t* n_out = nullptr) {
  constexpr int RPT = kRankPerLane;
  const uint32_t t = threadIdx.x;
  u64 lo = hi_in != 0 ? lo_in : ~0ull, hi = hi_in;
  if (hi_in != 0) {   // a known range holding every candidate
    if (t == 0) {
      sm.side_n = 0u;
      sm.cnt_out = 0u;
    }
  } else {
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit) {
    if (v[i] != 0ull) {
      lo = v[i] < lo ? v[i] : lo;
      hi = v[i] > hi ? v[i] : hi;
    }
  }
    const uint32_t a0 = wave_min_u32(static_cast<uint32_t>(lo >> 32));
    const uint32_t b0 = wave_max_u32(static_cast<uint32_t>(hi >> 32));
    const uint32_t al = wave_min_u32(static_cast<uint32_t>(lo >> 32) == a0 ? static_cast<uint32_t>(lo) : 0xFFFFFFFFu);
    const uint32_t bl = wave_max_u32(static_cast<uint32_t>(hi >> 32) == b0 ? static_cast<uint32_t>(hi) : 0u);
    if (lane_id() == 0) {
      sm.wred[t >> 6] = (static_cast<u64>(a0) << 32) | al;
      sm.wred2[t >> 6] = (static_cast<u64>(b0) << 32) | bl;
    }
    if (t == 0) {
      sm.side_n = 0u;
      sm.cnt_out = 0u;
    }
    __syncthreads();
    u64 l2 = ~0ull, h2 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      l2 = sm.wred[w] < l2 ? sm.wred[w] : l2;
      h2 = sm.wred2[w] > h2 ? sm.wred2[w] : h2;
    }
    lo = uniform64(l2);
    hi = uniform64(h2);
  }
  const uint32_t bl = bit_length64(hi - lo);
  const uint32_t shift = bl > kCutBits ? bl - kCutBits : 0u;
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit)
    if (v[i] != 0ull)
      atomicAdd(&sm.hist[(kCutBins - 1) - static_cast<uint32_t>((v[i] - lo) >> shift)], 1u);
  __syncthreads();
  uint32_t h[kCutBPT];
#pragma unroll
  for (int i = 0; i < kCutBPT; ++i) {
    h[i] = sm.hist[t * kCutBPT + i];
    sm.hist[t * kCutBPT + i] = 0u;
  }
  const uint32_t b = find_rank<kCutBPT>(sm, h, m, 0, n_out);
  if (b == kNone) return false;   // fewer than m candidates
  const uint32_t need = m - uniform(sm.res[1]), hb = uniform(sm.res[2]);
  const u64 blo = lo + (static_cast<u64>((kCutBins - 1) - b) << shift);
  const u64 bhi_full = blo + ((1ull << shift) - 1ull);
  const u64 bhi = bhi_full < hi ? bhi_full : hi;
  u64 T = blo;
  if (hb != need) {
    if (hb > kRankMax) return false;
    // The boundary bin's members, ranked by one wave.  Each wave takes its
    // span of the side buffer with one atomic.
    {
      u64 mk[RPT];
      uint32_t wn = 0;
#pragma unroll
      for (int i = 0; i < RPT; ++i) if (i < nit) {
        mk[i] = ballot((v[i] != 0ull) & (v[i] >= blo) & (v[i] <= bhi));
        wn += static_cast<uint32_t>(__popcll(mk[i]));
      }
      if (wn) {
        uint32_t base = 0;
        if (lane_id() == 0) base = atomicAdd(&sm.side_n, wn);
        base = uniform(base);
#pragma unroll
        for (int i = 0; i < RPT; ++i) if (i < nit) {
          if ((mk[i] >> lane_id()) & 1ull) sm.side[base + mbcnt64(mk[i])] = v[i];
          base += static_cast<uint32_t>(__popcll(mk[i]));
        }
      }
    }
    __syncthreads();
    if (t < 64) {
      const uint32_t ns = uniform(sm.side_n);
      const u64 mine = static_cast<uint32_t>(t) < ns ? sm.side[t] : 0ull;
      const uint32_t mlo = static_cast<uint32_t>(mine), mhi = static_cast<uint32_t>(mine >> 32);
      uint32_t above = 0;
      for (uint32_t j = 0; j < ns; ++j) {
        const uint32_t olo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mlo), static_cast<int>(j)));
        const uint32_t ohi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mhi), static_cast<int>(j)));
        above += ((static_cast<u64>(ohi) << 32) | olo) > mine ? 1u : 0u;
      }
      if (static_cast<uint32_t>(t) < ns && above + 1u == need) sm.res64 = mine;
    }
    __syncthreads();
    T = uniform64(sm.res64);
  }
  // Each wave takes its span of the output with one atomic, then stores its
  // kept candidates in lane order.
  u64 mk[RPT];
  uint32_t wn = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit) {
    mk[i] = ballot((v[i] != 0ull) & (v[i] >= T));
    wn += static_cast<uint32_t>(__popcll(mk[i]));
  }
  uint32_t base = 0;
  if (lane_id() == 0 && wn) base = atomicAdd(&sm.cnt_out, wn);
  base = uniform(base);
  bool z = false;
#pragma unroll
  for (int i = 0; i < RPT; ++i) if (i < nit) {
    if ((mk[i] >> lane_id()) & 1ull) z |= store_one(a, bf16, xrow, out0 + base + mbcnt64(mk[i]), v[i], true, status);
    base += static_cast<uint32_t>(__popcll(mk[i]));
  }
  if (z) sm.zeros = 1u;
  return true;
}

// select_core over buf[0, n).
template <int CAP>
__device__ __forceinline__ bool select_store(Smem<CAP>& sm, const CArgs& a, bool bf16,
                                             const char* xrow, int64_t out0, uint32_t n, uint32_t m,
                                             uint32_t status) {
  const uint32_t t = threadIdx.x;
  const uint32_t nit = uniform((n + NT - 1) / NT);
  u64 v[kRankPerLane];
#pragma unroll
  for (int i = 0; i < kRankPerLane; ++i) if (i < nit) {
    const uint32_t j = i * NT + t;
    v[i] = j < n ? sm.buf[j] : 0ull;   // 0: no candidate (every composite is above 0)
  }
  return select_core(sm, a, bf16, xrow, out0, v, nit, m, status);
}

// Per-row statistics, when the caller asked for them (a.stats non-null):
// counts added with device-scope atomics by lane 0 of the workgroup.
__device__ __forceinline__ void stat_add(const CArgs& a, int row, int field, uint32_t v) {
  if (a.stats && threadIdx.x == 0 && v) atomicAdd(&a.stats[4 * static_cast<int64_t>(row) + field], v);
}

// The epilogue of a row: the buffer holds `count` candidates, a superset of
// the top m = min(k, L) (m = 0 for a flagged row).  Cut to exactly m, order,
// write.
template <int KMAX, int CAP>
__device__ __forceinline__ void finish_row(Smem<CAP>& sm, const CArgs& a, bool bf16, int row,
                                           uint32_t count, uint32_t L, uint32_t status,
                                           bool direct = true, u64 lo_in = 0, u64 hi_in = 0) {
  constexpr int PER = KMAX > NT ? KMAX / NT : 1;
  const int t = threadIdx.x;
  const uint32_t k = static_cast<uint32_t>(a.k);
  uint32_t m = status ? 0u : min(k, L);
  if (direct) stat_add(a, row, DS_STAT_FINAL_CANDIDATES, count);
  if (t == 0) sm.zeros = 0u;
  __syncthreads();
  const int64_t out0 = static_cast<int64_t>(row) * k;
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * (bf16 ? 2 : 4);
  // Any order: the boundary found, every candidate above it stored.  Value
  // order: every candidate's rank, stored directly.
  if (direct && m > 0 && count >= m && count <= static_cast<uint32_t>(kRankPerLane * NT) &&
      ((a.sorted == 0 && select_store(sm, a, bf16, xrow, out0, count, m, status)) ||
       (a.sorted == 1 && rank_store(sm, a, bf16, xrow, out0, count, m, status, lo_in, hi_in)))) {
    for (uint32_t e = m + t; e < k; e += NT) store_one(a, bf16, xrow, out0 + e, 0ull, false, status);
    if (t == 0) a.row_status[row] = static_cast<int32_t>(status);
    stat_add(a, row, DS_STAT_CUTS, sm.n_cut);
    __syncthreads();
    if (uniform(sm.zeros)) fix_zero_signs(a, bf16, xrow, out0, m);
    return;
  }
  if (m > 0 && count > m) {
    cut_exact(sm, count, m);
    if (uniform(sm.err)) {
      status |= DS_ROW_INTERNAL;
      m = 0;
    }
  } else if (m > count) {   // cannot happen: every path leaves at least m candidates
    status |= DS_ROW_INTERNAL;
    m = 0;
  }
  __syncthreads();
  if (a.sorted != 0 && m > 1) {
    if (bf16 && a.n_cols <= 65536) sort_and_store<uint32_t, PER>(sm, a, bf16, xrow, out0, m, status);
    else sort_and_store<u64, PER>(sm, a, bf16, xrow, out0, m, status);
  } else {
    bool z = false;
    for (uint32_t e = t; e < k; e += NT)
      z |= store_one(a, bf16, xrow, out0 + e, e < m ? sm.buf[e] : 0ull, e < m, status);
    if (z) sm.zeros = 1u;
  }
  if (t == 0) a.row_status[row] = static_cast<int32_t>(status);
  stat_add(a, row, DS_STAT_CUTS, sm.n_cut);
  __syncthreads();
  if (uniform(sm.zeros)) fix_zero_signs(a, bf16, xrow, out0, m);
}

// finish_row for candidates held in registers: v[i] for i < nit, 0 where
// there is none.  The direct selections work on the registers and count the
// candidates on the way; their fallback (long runs of equal values, sorted by
// column) first packs the candidates into buf.  Returns false, having stored
// nothing, when there are fewer than min(k, L) candidates.
template <int KMAX, int CAP>
__device__ __forceinline__ bool finish_row_regs(Smem<CAP>& sm, const CArgs& a, bool bf16, int row,
                                                u64 (&v)[kRankPerLane], uint32_t nit, uint32_t L,
                                                uint32_t status, int par, u64 lo, u64 hi) {
  const int t = threadIdx.x;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t m = status ? 0u : min(k, L);
  if (t == 0) sm.zeros = 0u;   // ordered before any store by the selections' first barrier
  const int64_t out0 = static_cast<int64_t>(row) * k;
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * (bf16 ? 2 : 4);
  if (m > 0 && a.sorted != 2) {
    uint32_t n = 0;
    if ((a.sorted == 0 && select_core(sm, a, bf16, xrow, out0, v, nit, m, status, lo, hi, &n)) ||
        (a.sorted == 1 && rank_core(sm, a, bf16, xrow, out0, v, nit, m, status, lo, hi, &n))) {
      stat_add(a, row, DS_STAT_FINAL_CANDIDATES, n);
      for (uint32_t e = m + t; e < k; e += NT) store_one(a, bf16, xrow, out0 + e, 0ull, false, status);
      if (t == 0) a.row_status[row] = static_cast<int32_t>(status);
      stat_add(a, row, DS_STAT_CUTS, sm.n_cut);
      __syncthreads();
      if (uniform(sm.zeros)) fix_zero_signs(a, bf16, xrow, out0, m);
      return true;
    }
    if (n < m) return false;
  }
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < kRankPerLane; ++i) if (i < nit) c += v[i] != 0ull ? 1u : 0u;
  uint32_t total;
  uint32_t pos = block_excl(sm, c, par, &total);
  if (total < m) return false;
  stat_add(a, row, DS_STAT_FINAL_CANDIDATES, total);
#pragma unroll
  for (int i = 0; i < kRankPerLane; ++i) if (i < nit) {
    if (v[i] != 0ull) sm.buf[pos++] = v[i];
  }
  finish_row<KMAX>(sm, a, bf16, row, total, L, status, false);
  return true;
}

// OR of a per-lane flag over the workgroup (flag bits are small).
template <int CAP>
__device__ __forceinline__ uint32_t block_or(Smem<CAP>& sm, uint32_t f, int par) {
  const u64 b1 = ballot(f & 1u), b2 = ballot(f & 2u), b4 = ballot(f & 4u);
  if (lane_id() == 0) sm.wtot[par][threadIdx.x >> 6] = (b1 ? 1u : 0u) | (b2 ? 2u : 0u) | (b4 ? 4u : 0u);
  __syncthreads();
  uint32_t o = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) o |= sm.wtot[par][w];
  return uniform(o);
}

// ---------------------------------------------------------------- the kernels
// Row length and status of a row.
__device__ __forceinline__ uint32_t row_len(const CArgs& a, int row, uint32_t* status) {
  int64_t Ls = a.end ? static_cast<int64_t>(a.end[row]) : static_cast<int64_t>(a.n_cols);
  if (Ls < 0 || Ls > a.n_cols) {
    *status = DS_ROW_BAD_END;
    return 0;
  }
  return static_cast<uint32_t>(Ls);
}

// A whole row per workgroup, chunk by chunk.
template <bool BF16, int KC>
__global__ __launch_bounds__(NT, waves_per_simd(NT == 256 ? (KC >= 2 ? 3 : 4) : 2)) void chunk_row_kernel(CArgs a) {
  using G = Geo<BF16>;
  constexpr int KMAX = class_kmax(KC);
  constexpr int CAP = chunk_cap(KC, NT);
  static_assert(CAP >= KMAX + NT * G::EPV, "a cut leaves room for one vector per lane");
  __shared__ Smem<CAP> sm;
  const int t = threadIdx.x;
  const int row = a.reverse_rows ? a.batch - 1 - static_cast<int>(blockIdx.x) : static_cast<int>(blockIdx.x);
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t cap = a.cap_eff;
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * G::ESZ;
  uint32_t status = 0;
  const uint32_t L = row_len(a, row, &status);
  const uint32_t nch = (L + G::CE - 1) / G::CE;

  // Visiting order: an affine bijection j -> (p*j + q) mod nch, p coprime to
  // nch (the pages visit blocks in a random order).
  uint32_t pm = 1, pq = 0;
  if (!a.in_order && nch > 2) {
    uint32_t h = a.perm_seed * 0x9E3779B9u ^ (static_cast<uint32_t>(row) + 0x7F4A7C15u) * 0x85EBCA6Bu;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    pq = h % nch;
    pm = 1u + (h >> 8) % (nch - 1u);
    for (uint32_t guard = 0; guard < nch; ++guard) {   // the next value coprime to nch
      uint32_t x = pm, y = nch;
      while (y) {
        const uint32_t r2 = x % y;
        x = y;
        y = r2;
      }
      if (x == 1u) break;
      pm = pm + 1u < nch ? pm + 1u : 1u;
    }
  }
  auto chunk_at = [&](uint32_t j) -> uint32_t {
    return static_cast<uint32_t>((static_cast<u64>(pm) * j + pq) % nch);
  };

  for (int i = t; i < kCutBins / 4; i += NT) reinterpret_cast<u32x4*>(sm.hist)[i] = u32x4{0u, 0u, 0u, 0u};
  if (t == 0) {
    sm.err = 0u;
    sm.n_cut = 0u;
  }

  if (t == 0) sm.rowmax = 0u;
  Buf B{0u, kTAll, 0};
  bool spec = false, nan = false;
  uint32_t top0 = 0;   // the first chunk's largest key
  if (status == 0 && nch > 0) {
    // One chunk in registers at a time: the workgroups sharing a CU (many
    // rows) keep the loads in flight while this one filters.
    u32x4 ra[V];
    load_chunk<BF16>(ra, xrow, chunk_at(0), L);
    nan = start_chunk<BF16>(sm, B, ra, chunk_at(0), L, k, nch == 1, &spec, &top0);
    const uint32_t nv0 = chunk_nv<BF16>(chunk_at(0), L);
    if (!append_fast<BF16>(sm, B, ra, chunk_at(0), cap, nv0)) append_chunk<BF16>(sm, B, ra, chunk_at(0), k, cap, nv0);
    for (uint32_t j = 1; j < nch && !uniform(sm.err); ++j) {
      load_chunk<BF16>(ra, xrow, chunk_at(j), L);
      nan |= next_chunk<BF16>(sm, B, ra, chunk_at(j), L, k, cap);
    }
  }
  status |= block_or(sm, nan ? static_cast<uint32_t>(DS_ROW_NAN) : 0u, B.par);
  B.par ^= 1;
  if (uniform(sm.err)) status |= DS_ROW_INTERNAL;
  // An estimated start is checked: with fewer than min(k, L) candidates at or
  // above it, a value of the top k may lie below it.
  if (status == 0 && spec && B.count < min(k, L)) {
    B = restream<BF16>(sm, B.par, xrow, L, k, cap);
    stat_add(a, row, DS_STAT_ROW_REREADS, 1u);
    if (uniform(sm.err)) status |= DS_ROW_INTERNAL;
  }
  // Every candidate lies in [key(T), the row's largest key]: the value-order
  // epilogue bins that range without measuring it (unless T admits all).
  const uint32_t rmax = max(top0, uniform(sm.rowmax));
  const uint32_t tkey = key_of(B.T);
  const bool known = B.T != kTAll && rmax != 0u && tkey <= rmax;
  finish_row<KMAX>(sm, a, BF16, row, B.count, L, status, true,
                   known ? static_cast<u64>(tkey) << 32 : 0ull,
                   known ? (static_cast<u64>(rmax) << 32) | 0xFFFFFFFFull : 0ull);
}

// One chunk of a row per workgroup; the last workgroup of the row to finish
// merges the others' candidates.
template <bool BF16, int KC>
__global__ __launch_bounds__(NT, waves_per_simd(1024 / NT)) void chunk_split_kernel(CArgs a) {
  using G = Geo<BF16>;
  constexpr int KMAX = class_kmax(KC);
  constexpr int CAP = chunk_cap(KC, NT);
  constexpr int G8 = kRankPerLane / 2;   // slots per lane per merge round
  static_assert(CAP >= KMAX + NT * G::EPV, "a cut leaves room for one vector per lane");
  static_assert(G8 * NT <= CAP - KMAX, "a merge round fits after a cut");
  __shared__ Smem<CAP> sm;
  const int t = threadIdx.x;
  const int S = a.segments;
  const int row = static_cast<int>(blockIdx.x) / S;
  const int seg = static_cast<int>(blockIdx.x) - row * S;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t cap = a.cap_eff;
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * G::ESZ;
  uint32_t status = 0;
  const uint32_t L = row_len(a, row, &status);
  const uint32_t nch = (L + G::CE - 1) / G::CE;
  const bool mine = static_cast<uint32_t>(seg) < nch;

  for (int i = t; i < kCutBins / 4; i += NT) reinterpret_cast<u32x4*>(sm.hist)[i] = u32x4{0u, 0u, 0u, 0u};
  if (t == 0) {
    sm.err = 0u;
    sm.n_cut = 0u;
  }

  Buf B{0u, kTAll, 0};
  bool nan = false, spec = false;
  uint32_t top_key = 0;   // the chunk's largest key (0: no values)
  // The chunk's candidates go to one region of buf per wave, as raw pairs,
  // in one pass over the registers (regions == true); should a region
  // overflow, the chunk is appended again contiguously, cutting as needed.
  const uint32_t R = cap / NW;
  bool regions = false;
  uint32_t cnt[NW] = {};
  if (status == 0 && mine) {
    u32x4 ra[V];
    load_chunk<BF16>(ra, xrow, static_cast<uint32_t>(seg), L);
    nan = start_chunk<BF16>(sm, B, ra, static_cast<uint32_t>(seg), L, k, false, &spec, &top_key);
    const float f = __uint_as_float(bits_of_key(key_of(B.T)));
    const uint32_t wc = region_write<BF16>(sm, ra, static_cast<uint32_t>(seg), f, R);
    if (lane_id() == 0) sm.wtot[B.par][t >> 6] = wc;
    __syncthreads();
    uint32_t total = 0;
    bool over = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      cnt[w] = uniform(sm.wtot[B.par][w]);
      total += cnt[w];
      over |= cnt[w] > R;
    }
    B.par ^= 1;
    if (over) {
      B = reappend_chunk<BF16>(sm, B, xrow, static_cast<uint32_t>(seg), L, k, cap);
      stat_add(a, row, DS_STAT_CHUNK_REREADS, 1u);
    } else {
      regions = true;
      B.count = total;
    }
  }
  status |= block_or(sm, nan ? static_cast<uint32_t>(DS_ROW_NAN) : 0u, B.par);
  B.par ^= 1;
  // At most k candidates are handed over: the chunk's own top k, exactly.
  if (status == 0 && regions && B.count > k) {
    // Make the regions one run of composites: each wave converts its own,
    // then waves 1..3 in turn move theirs down (a move never overwrites a
    // slot it has still to read).
    const uint32_t w = t >> 6;
    u64* reg = sm.buf + w * R;
    for (uint32_t j = lane_id(); j < cnt[w]; j += 64) {
      reg[j] = comp_of_raw<BF16>(reg[j]);
    }
    uint32_t dst = cnt[0];
    for (uint32_t ww = 1; ww < static_cast<uint32_t>(NW); ++ww) {
      __syncthreads();
      if (w == ww)
        for (uint32_t j = lane_id(); j < cnt[ww]; j += 64) sm.buf[dst + j] = reg[j];
      dst += cnt[ww];
    }
    regions = false;
  }
  if (status == 0 && !uniform(sm.err) && !regions && B.count > k) {
    __syncthreads();
    const u64 Tn = cut_exact(sm, B.count, k);
    if (!uniform(sm.err)) {
      B.T = Tn;
      B.count = k;
    }
  }
  if (uniform(sm.err)) status |= DS_ROW_INTERNAL;

  // ---- hand-over: the chunk's candidates, its threshold and its flags.
  const int64_t rs = static_cast<int64_t>(row) * S + seg;
  u64* slot = a.ws_slot + rs * static_cast<int64_t>(k);
  const uint32_t hand = status ? 0u : B.count;
  if (regions) {
    const uint32_t w = t >> 6;
    uint32_t base = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) base += static_cast<uint32_t>(ww) < w ? cnt[ww] : 0u;
    const u64* reg = sm.buf + w * R;
    const uint32_t mc = status ? 0u : cnt[w];
    for (uint32_t j = lane_id(); j < mc; j += 64) {
      st_agent(&slot[base + j], comp_of_raw<BF16>(reg[j]));
    }
  } else {
    for (uint32_t j = t; j < hand; j += NT) st_agent(&slot[j], sm.buf[j]);
  }
  if (t == 0) {
    st_agent(&a.ws_rec[2 * rs], mine ? B.T : kTAll);
    st_agent(&a.ws_rec[2 * rs + 1],
             (static_cast<u64>(status) << 56) | (static_cast<u64>(top_key) << 24) | hand);
  }
  // Ordering of the hand-over.  Every store above is an agent-scope atomic
  // store: on gfx950 it is written through to the device-coherent level
  // (sc1), past the per-XCD L2 caches.  Each wave waits until all of its
  // stores are complete (vmcnt 0) before the barrier, so they are visible
  // device-wide before lane 0 moves the row's counter.  The last workgroup
  // reads the counter's old value, then (after a barrier on that value)
  // loads with agent-scope atomic loads, which also read the coherent level,
  // so it sees every hand-over.  A release / acquire pair on the counter
  // would order the same accesses but costs an L2 write-back and invalidate
  // in every workgroup (about 14 us per call on a 128-row split).
  wait_all_memory();
  __syncthreads();
  if (t == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.ws_arrive[row], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sm.is_last = prev == static_cast<uint32_t>(S - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!uniform(sm.is_last)) {
    stat_add(a, row, DS_STAT_CUTS, sm.n_cut);
    return;
  }

  // ---- merge: every chunk's candidates at or above the largest chunk threshold.
  // Chunk s's slots are read by lanes [s*PL, (s+1)*PL), PL = NT / S lanes per
  // chunk, G8 slots per lane per round.  The first round goes out together
  // with the records, before the counts are known; what it read past a
  // chunk's count (whatever an earlier call left there) is then replaced by
  // zero, which is below every threshold.
  const u64* rec = a.ws_rec + static_cast<int64_t>(row) * S * 2;
  const uint32_t PL = static_cast<uint32_t>(NT / S);
  const uint32_t my_s = static_cast<uint32_t>(t) / PL;
  const uint32_t my_l = static_cast<uint32_t>(t) - my_s * PL;
  const bool has_s = my_s < static_cast<uint32_t>(S);
  u64* my_slot = a.ws_slot + (static_cast<int64_t>(row) * S + my_s) * static_cast<int64_t>(k);
  const uint32_t per_round = PL * G8;
  // A second round goes out with the first when a chunk's expected
  // hand-over (its share estimate, plus the spread of a lane-maximum start)
  // exceeds one round.
  const float Es = static_cast<float>(k) * static_cast<float>(G::CE) / static_cast<float>(L > 0 ? L : 1u);
  const bool two = per_round < k && 1.5f * (Es + 6.0f * __builtin_sqrtf(Es) + 8.0f) > static_cast<float>(per_round);
  // The first two rounds' slots: [0, G8) the first, [G8, 2 G8) the second.
  static_assert(2 * G8 == kRankPerLane, "two merge rounds fill the epilogue's registers");
  u64 vr[kRankPerLane];
#pragma unroll
  for (int q = 0; q < G8; ++q) {
    const uint32_t j = q * PL + my_l;
    vr[q] = (has_s && j < k) ? ld_agent(&my_slot[j]) : 0ull;
  }
  if (two) {
#pragma unroll
    for (int q = 0; q < G8; ++q) {
      const uint32_t j = per_round + q * PL + my_l;
      vr[G8 + q] = (has_s && j < k) ? ld_agent(&my_slot[j]) : 0ull;
    }
  } else {
#pragma unroll
    for (int q = 0; q < G8; ++q) vr[G8 + q] = 0ull;
  }
  const uint32_t my_c = has_s ? static_cast<uint32_t>(ld_agent(&rec[2 * my_s + 1]) & 0xFFFFFFu) : 0u;
#pragma unroll
  for (int q = 0; q < G8; ++q) {
    if (q * PL + my_l >= my_c) vr[q] = 0ull;
    if (per_round + q * PL + my_l >= my_c) vr[G8 + q] = 0ull;
  }
  u64 Tm = 0;
  uint32_t fl = 0, cm = 0, tk = 0;
  if (t < S) {
    Tm = ld_agent(&rec[2 * t]);
    const u64 info = ld_agent(&rec[2 * t + 1]);
    fl = static_cast<uint32_t>(info >> 56);
    cm = static_cast<uint32_t>(info & 0xFFFFFFu);
    tk = static_cast<uint32_t>(info >> 24);
  }
  {
    const uint32_t hiw = wave_max_u32(static_cast<uint32_t>(Tm >> 32));
    const uint32_t low = wave_max_u32(static_cast<uint32_t>(Tm >> 32) == hiw ? static_cast<uint32_t>(Tm) : 0u);
    const uint32_t cmx = wave_max_u32(cm);
    const uint32_t tkx = wave_max_u32(tk);
    if (lane_id() == 0) {
      sm.wred[t >> 6] = (static_cast<u64>(hiw) << 32) | low;
      sm.wred2[t >> 6] = tkx;
      sm.wmax[t >> 6] = cmx;
    }
  }
  status |= block_or(sm, fl, B.par);   // its barrier also publishes wred / wmax
  B.par ^= 1;
  u64 tm = 0, tkm = 0;
  uint32_t cmax = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    tm = sm.wred[w] > tm ? sm.wred[w] : tm;
    tkm = sm.wred2[w] > tkm ? sm.wred2[w] : tkm;
    cmax = max(cmax, sm.wmax[w]);
  }
  Tm = uniform64(tm);
  cmax = uniform(cmax);
  // Every candidate lies in [Tm, the largest chunk key's last composite].
  const u64 range_hi = (uniform64(tkm) << 32) | 0xFFFFFFFFull;

  // Every chunk's slots already in registers: the candidates at or above Tm
  // go to the epilogue from there, with no append.
  // (Values below Tm are dropped in place: the append below drops them too.)
  if (status == 0 && cmax <= (two ? 2u : 1u) * per_round) {
#pragma unroll
    for (int q = 0; q < kRankPerLane; ++q) vr[q] = vr[q] >= Tm ? vr[q] : 0ull;
    if (t == 0) st_agent(&a.ws_arrive[row], 0u);
    if (finish_row_regs<KMAX>(sm, a, BF16, row, vr, two ? 2u * G8 : static_cast<uint32_t>(G8), L,
                              status, B.par, Tm, range_hi)) {
      return;
    }
    // Fewer than min(k, L) at or above Tm: appended below, then read again.
    __syncthreads();
  }

  B.count = 0;
  B.T = Tm;
  const uint32_t rounds = status ? 0u : (cmax + per_round - 1) / per_round;
  __syncthreads();
  for (uint32_t rd = 0; rd < rounds; ++rd) {
    u64 v[G8];
#pragma unroll
    for (int q = 0; q < G8; ++q) {
      const uint32_t j = rd * per_round + q * PL + my_l;
      v[q] = rd == 0 ? vr[q]
           : (rd == 1 && two) ? vr[G8 + q]
           : ((has_s && j < my_c) ? ld_agent(&my_slot[j]) : 0ull);
    }
    uint32_t n = 0;
#pragma unroll
    for (int q = 0; q < G8; ++q) n += v[q] >= B.T ? 1u : 0u;
    uint32_t total;
    uint32_t pre = block_excl(sm, n, B.par, &total);
    B.par ^= 1;
    if (B.count + total > cap) {
      // Cut the buffer to k first; the round's values then fit.
      const u64 Tn = cut_exact(sm, B.count, k);
      if (uniform(sm.err)) break;
      B.T = Tn;
      B.count = k;
      n = 0;
#pragma unroll
      for (int q = 0; q < G8; ++q) n += v[q] >= B.T ? 1u : 0u;
      pre = block_excl(sm, n, B.par, &total);
      B.par ^= 1;
    }
    uint32_t pos = B.count + pre;
#pragma unroll
    for (int q = 0; q < G8; ++q)
      if (v[q] >= B.T) sm.buf[pos++] = v[q];
    B.count += total;
    __syncthreads();
  }
  // The row's counter goes back to zero; slots and records need no clearing
  // (every call writes them before reading).
  if (t == 0) st_agent(&a.ws_arrive[row], 0u);
  if (uniform(sm.err)) status |= DS_ROW_INTERNAL;
  // The check: every chunk kept all of its values at or above its own
  // threshold, so the buffer holds every value of the row at or above T*, the
  // largest of those thresholds (or above a cut's threshold, which is valid).
  // With at least min(k, L) of them, the top min(k, L) are all here.
  if (status == 0 && B.count < min(k, L)) {
    B = restream<BF16>(sm, B.par, xrow, L, k, cap);
    stat_add(a, row, DS_STAT_ROW_REREADS, 1u);
    if (uniform(sm.err)) status |= DS_ROW_INTERNAL;
  }
  finish_row<KMAX>(sm, a, BF16, row, B.count, L, status);
}

// ---------------------------------------------------------------- read ceiling
// A measurement aid, not part of the selection: the chunk kernels' grid and
// loads (a whole row chunk by chunk with the next chunk in flight, or one
// chunk per workgroup), the data only folded into one word per lane, stored
// only if it equals a constant.
template <bool BF16>
__global__ __launch_bounds__(NT) void chunk_read_kernel(CArgs a, uint32_t* sink) {
  using G = Geo<BF16>;
  const int S = a.segments;
  int row = static_cast<int>(blockIdx.x) / S;
  const int seg = static_cast<int>(blockIdx.x) - row * S;
  if (S == 1 && a.reverse_rows) row = a.batch - 1 - row;
  uint32_t status = 0;
  const uint32_t L = row_len(a, row, &status);
  const uint32_t nch = (L + G::CE - 1) / G::CE;
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * G::ESZ;
  const uint32_t c0 = S == 1 ? 0u : static_cast<uint32_t>(seg);
  const uint32_t n = S == 1 ? nch : (c0 < nch ? 1u : 0u);
  uint32_t acc = 0;
  u32x4 ra[V], rb[V];
  if (n > 0) load_chunk<BF16>(ra, xrow, c0, L);
  for (uint32_t j = 0; j < n; ++j) {
    if (j + 1 < n) load_chunk<BF16>(rb, xrow, c0 + j + 1, L);
#pragma unroll
    for (int i = 0; i < V; ++i) acc ^= ra[i].x ^ ra[i].y ^ ra[i].z ^ ra[i].w;
#pragma unroll
    for (int i = 0; i < V; ++i) ra[i] = rb[i];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// This build's kernel: split rows or whole rows.
template <bool BF16>
const void* chunk_fn(int cls) {
  if constexpr (kSplit) {
    return cls == 0 ? reinterpret_cast<const void*>(&chunk_split_kernel<BF16, 0>)
         : cls == 1 ? reinterpret_cast<const void*>(&chunk_split_kernel<BF16, 1>)
         : cls == 2 ? reinterpret_cast<const void*>(&chunk_split_kernel<BF16, 2>)
                    : reinterpret_cast<const void*>(&chunk_split_kernel<BF16, 3>);
  } else {
    return cls == 0 ? reinterpret_cast<const void*>(&chunk_row_kernel<BF16, 0>)
         : cls == 1 ? reinterpret_cast<const void*>(&chunk_row_kernel<BF16, 1>)
         : cls == 2 ? reinterpret_cast<const void*>(&chunk_row_kernel<BF16, 2>)
                    : reinterpret_cast<const void*>(&chunk_row_kernel<BF16, 3>);
  }
}

}  // namespace

#if CHUNK_SPLIT
#define DSTK_LAUNCH_CHUNK launch_chunk_split
#define DSTK_LAUNCH_CHUNK_READ launch_chunk_read_split
#else
#define DSTK_LAUNCH_CHUNK launch_chunk_row
#define DSTK_LAUNCH_CHUNK_READ launch_chunk_read_row
#endif

// The launch's own error code (hipLaunchKernel returns it; an earlier,
// unrelated error left in the runtime is neither returned nor cleared).
int DSTK_LAUNCH_CHUNK(const CArgs& a, int dtype, int cls, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.segments);
  CArgs arg = a;
  void* args[] = {&arg};
  const void* fn = dtype == 0 ? chunk_fn<false>(cls) : chunk_fn<true>(cls);
  return static_cast<int>(hipLaunchKernel(fn, dim3(grid), dim3(NT), args, 0, stream));
}

int DSTK_LAUNCH_CHUNK_READ(const CArgs& a, int dtype, uint32_t* sink, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.segments);
  CArgs arg = a;
  void* args[] = {&arg, &sink};
  const void* fn = dtype == 0 ? reinterpret_cast<const void*>(&chunk_read_kernel<false>)
                              : reinterpret_cast<const void*>(&chunk_read_kernel<true>);
  return static_cast<int>(hipLaunchKernel(fn, dim3(grid), dim3(NT), args, 0, stream));
}

}  // namespace dstk
