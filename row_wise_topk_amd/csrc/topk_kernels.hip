// Row-wise TopK kernels for MI355X (gfx950, wave64).
//
// Method (narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for
// sparse attention and sampling", method paragraph): keep a threshold T that
// starts at -inf and never falls; read the row once in contiguous blocks of B
// elements visited in a random order; append the values that pass T to a
// candidate buffer; when the buffer reaches k + B2 entries, radix-select it back
// to k and raise T.  The pages' CUDA design is prior art only; what follows is
// laid out for CDNA4:
//
//  * one workgroup (256 or 512 lanes) streams a row, or a share of a row's
//    blocks when several workgroups cooperate on one row;
//  * a block is B = 4096 elements: every lane issues 16-byte loads, and the
//    next block's loads are in flight while the current one is filtered;
//  * the filter runs on the raw fp32 values (bf16 is widened by a shift), with
//    a wave-wide early-out on each lane's running maximum; survivors are
//    compacted into LDS with ballot / mbcnt and one LDS atomic per wave;
//  * the cut (radix select) is an 11-bit LDS histogram over the live key range
//    [T, max], refined only when the boundary bin is too full; exact ties on a
//    key are cut by index with the same histogram on the index;
//  * several workgroups on one row share T through a 64-bit atomicMax in
//    device memory; the last to finish merges the others' survivors;
//  * the epilogue orders the k results by value or by index with a histogram
//    grouping plus an in-bin rank, and writes indices / values / status.
//
// Order and tie-break (xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！",
// Q&A on stable results): larger value first, then lower index.  A value v at
// column i has the 64-bit composite  (key(v) << 32) | ~i,  where key() maps
// fp32 sign-magnitude onto unsigned offset binary so that -0.0 and +0.0 share
// one key.  The threshold T is a composite too: an element is admitted iff its
// composite is > T, so T can sit between two equal values with different
// columns.  Every published T leaves at least k composites of the row above it.
//
// NaN (narracomm.com, NaN paragraph): always checked over [0, end); a NaN sets
// a status bit for the row instead of trapping.

#include <hip/hip_runtime.h>

#include "ds_topk.h"
#include "topk_internal.h"

namespace dstk {
namespace {

constexpr int kRadixBits = 11;
constexpr int kBins = 1 << kRadixBits;
constexpr uint32_t kBias = 0x80000000u;
constexpr uint32_t kQNaN32 = 0x7FC00000u;
constexpr uint32_t kNegInf32 = 0xFF800000u;

// ---------------------------------------------------------------- keys
__device__ __forceinline__ uint32_t key_of_bits(uint32_t b) {
  const uint32_t mag = b & 0x7FFFFFFFu;
  return (b & 0x80000000u) ? kBias - mag : kBias + mag;
}

// Inverse of key_of_bits for keys of non-NaN values ([0x00800000, 0xFF800000]).
__device__ __forceinline__ float float_of_key(uint32_t key) {
  const uint32_t b = key >= kBias ? key - kBias : ((kBias - key) | 0x80000000u);
  return __uint_as_float(b);
}

__device__ __forceinline__ uint64_t comp_of(uint32_t key, uint32_t idx) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~idx);
}

// T = -inf with "greater or equal": just below the key of -inf, all columns.
constexpr uint64_t kThrInit = (static_cast<uint64_t>(0x00800000u - 1u) << 32) | 0xFFFFFFFFull;

// The threshold in the form the filter uses: admit v iff v > f, or v == f and
// column < idx_lim.  With idx_lim == ~0u this is simply v >= f.
struct Filter {
  float f;
  uint32_t idx_lim;
};

__device__ __forceinline__ Filter filter_of(uint64_t thr) {
  const uint32_t K = static_cast<uint32_t>(thr >> 32);
  const uint32_t low = static_cast<uint32_t>(thr);
  if (low == 0xFFFFFFFFu) return {float_of_key(K + 1u), 0xFFFFFFFFu};
  return {float_of_key(K), ~low};
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o)));
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o)));
  return v;
}

__device__ __forceinline__ uint32_t bit_length(uint32_t v) { return v ? 32u - __clz(v) : 0u; }

// Relaxed agent-scope accesses to the shared per-row threshold.
__device__ __forceinline__ uint64_t load_thr(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_thr(unsigned long long* p, uint64_t v) {
  __hip_atomic_fetch_max(p, static_cast<unsigned long long>(v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
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
  uint32_t val[CAP];      // candidate value bits (fp32, or bf16 widened to fp32)
  uint32_t idx[CAP];      // candidate columns
  uint32_t hist[kBins];
  uint32_t wsum[NT / 64];
  uint32_t res[4];
  uint32_t cnt[2];        // append counters; cur receives appends, cur^1 the next cut
  uint32_t snap[2][NT / 64];  // per-wave count after its last append, by step parity
  uint32_t segoff[kMaxSegments];  // merge: first flat position of each segment
  uint32_t hikey;         // upper bound of every candidate key
  uint32_t flags;         // row status bits
  uint32_t is_last;
  unsigned long long thr; // the workgroup's threshold (composite)
};

// Suffix search: higher bins first.  Finds b* with
//   sum_{b > b*} hist[b] < need <= sum_{b >= b*} hist[b]
// res = {b*, sum above b*, hist[b*], total}; res[0] = kBins when total < need.
template <int NT, int CAP>
__device__ void hist_find_top(Smem<CAP, NT>& sm, uint32_t need) {
  constexpr int BPT = kBins / NT;
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t h[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = sm.hist[t * BPT + i];
    s += h[i];
  }
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_down(static_cast<int>(x), o));
    if (lane + o < 64) x += y;
  }
  if (lane == 0) sm.wsum[w] = x;
  if (t == 0) sm.res[0] = kBins;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2)
    if (w2 > w) add += sm.wsum[w2];
  const uint32_t incl = x + add;
  const uint32_t excl = incl - s;
  if (excl < need && need <= incl) {
    uint32_t acc = excl;
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
  if (t == 0) sm.res[3] = incl;
  __syncthreads();
}

// In place: hist[b] <- sum_{b' < b} hist[b'].
template <int NT, int CAP>
__device__ void hist_exclusive_scan(Smem<CAP, NT>& sm) {
  constexpr int BPT = kBins / NT;
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t h[BPT];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = sm.hist[t * BPT + i];
    s += h[i];
  }
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_up(static_cast<int>(x), o));
    if (lane >= o) x += y;
  }
  if (lane == 63) sm.wsum[w] = x;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2)
    if (w2 < w) add += sm.wsum[w2];
  uint32_t run = x - s + add;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    sm.hist[t * BPT + i] = run;
    run += h[i];
  }
  __syncthreads();
}

template <int NT, int CAP>
__device__ __forceinline__ void hist_clear(Smem<CAP, NT>& sm) {
#pragma unroll
  for (int i = threadIdx.x; i < kBins; i += NT) sm.hist[i] = 0u;
}

// Among the candidates with key E and composite > T, the column I of the
// need-th smallest column (need >= 1 and at least need such candidates).
template <int NT, int CAP>
__device__ uint32_t index_cut(Smem<CAP, NT>& sm, uint32_t c, uint32_t E, uint32_t need,
                              uint64_t T, uint32_t n_cols) {
  const int t = threadIdx.x;
  uint32_t ibase = 0;
  uint32_t itop = n_cols > 0 ? n_cols - 1u : 0u;
  for (;;) {
    const uint32_t span = itop - ibase;
    const uint32_t shift = bit_length(span) > kRadixBits ? bit_length(span) - kRadixBits : 0u;
    hist_clear(sm);
    __syncthreads();
    for (uint32_t i = t; i < c; i += NT) {
      const uint32_t ci = sm.idx[i];
      if (key_of_bits(sm.val[i]) == E && ci >= ibase && ci <= itop && comp_of(E, ci) > T)
        atomicAdd(&sm.hist[(kBins - 1) - ((ci - ibase) >> shift)], 1u);
    }
    __syncthreads();
    hist_find_top(sm, need);
    const uint32_t b = (kBins - 1) - sm.res[0];   // bin in ascending column order
    const uint32_t below = sm.res[1], bc = sm.res[2];
    need -= below;
    ibase += b << shift;
    const uint32_t bin_top = ibase + ((1u << shift) - 1u);
    if (bc == need) return bin_top < itop ? bin_top : itop;
    if (shift == 0) return ibase;
    itop = bin_top < itop ? bin_top : itop;
  }
}

// Cut the candidate buffer: keep every candidate with composite > T_new, where
// T_new >= sm.thr leaves between k and keep_max candidates (or all of them if
// fewer than keep_max are above sm.thr).  keep_max == k gives the exact top-k.
// Returns the new append counter index.
template <int NT, int CAP>
__device__ int cut_buffer(Smem<CAP, NT>& sm, int cur, uint32_t k, uint32_t keep_max,
                          uint32_t n_cols, float hi_lane) {
  constexpr int E = CAP / NT;
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t hk = wave_max_u32(key_of_bits(__float_as_uint(hi_lane)));
  if (lane == 0) atomicMax(&sm.hikey, hk);
  if (t == 0) sm.cnt[cur ^ 1] = 0u;
  __syncthreads();
  const uint32_t c = sm.cnt[cur];
  const uint64_t T = sm.thr;
  const uint32_t hi = sm.hikey;
  const uint32_t K = static_cast<uint32_t>(T >> 32);
  const uint32_t klo = static_cast<uint32_t>(T) == 0xFFFFFFFFu ? K + 1u : K;

  uint64_t newT = T;
  if (hi >= klo && c > 0) {
    uint32_t need = k, above = 0, base = klo, top = hi;
    bool first = true;
    for (;;) {
      const uint32_t span = top - base;
      const uint32_t shift = bit_length(span) > kRadixBits ? bit_length(span) - kRadixBits : 0u;
      hist_clear(sm);
      __syncthreads();
      for (uint32_t i = t; i < c; i += NT) {
        const uint32_t key = key_of_bits(sm.val[i]);
        if (key >= base && key <= top && comp_of(key, sm.idx[i]) > T)
          atomicAdd(&sm.hist[(key - base) >> shift], 1u);
      }
      __syncthreads();
      hist_find_top(sm, need);
      if (first) {
        first = false;
        if (sm.res[3] <= keep_max) break;   // few enough above T: only drop those at or below T
      }
      const uint32_t b = sm.res[0], ab = sm.res[1], bc = sm.res[2];
      above += ab;
      need -= ab;
      base += b << shift;
      if (above + bc <= keep_max) {
        const uint64_t cand = (static_cast<uint64_t>(base) << 32) - 1u;
        newT = cand > T ? cand : T;
        break;
      }
      if (shift == 0) {
        const uint32_t I = index_cut(sm, c, base, need, T, n_cols);
        const uint64_t cand = comp_of(base, I) - 1u;
        newT = cand > T ? cand : T;
        break;
      }
      top = base + ((1u << shift) - 1u);
    }
  }

  // Compaction into the other counter: read everything first, then write.
  const int nxt = cur ^ 1;
  uint32_t rv[E], ri[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = t + e * NT;
    rv[e] = i < c ? sm.val[i] : 0u;
    ri[e] = i < c ? sm.idx[i] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t i = t + e * NT;
    const bool keep = i < c && comp_of(key_of_bits(rv[e]), ri[e]) > newT;
    const uint64_t m = ballot(keep);
    if (m) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&sm.cnt[nxt], static_cast<uint32_t>(__popcll(m)));
      base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0));
      if (keep) {
        const uint32_t pos = base + mbcnt64(m);
        sm.val[pos] = rv[e];
        sm.idx[pos] = ri[e];
      }
    }
  }
  if (t == 0) sm.thr = newT;
  __syncthreads();
  return nxt;
}

// Filter one block held in registers and append its survivors.
template <bool BF16, bool RAG, int V, int NT, int CAP>
__device__ __forceinline__ uint32_t filter_block(const uint4 (&r)[V], uint32_t blk, uint32_t L,
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
  auto col = [&](int s) { return base_idx + (s / EPV) * (NT * EPV) + (s % EPV); };
  if (RAG) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bool valid = col(s) < L;
      nan_lane |= valid && (f[s] != f[s]);
      if (!valid) f[s] = __uint_as_float(kQNaN32);
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS; s += 2) nan_lane |= __builtin_isunordered(f[s], f[s + 1]);
  }
  float mx = f[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) mx = fmaxf(mx, f[s]);
  hi_lane = fmaxf(hi_lane, mx);
  if (!ballot(mx >= F.f)) return 0u;

  bool p[NS];
  uint64_t m[NS];
  uint32_t total = 0;
  if (F.idx_lim == 0xFFFFFFFFu) {
#pragma unroll
    for (int s = 0; s < NS; ++s) p[s] = f[s] >= F.f;
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) p[s] = f[s] > F.f || (f[s] == F.f && col(s) < F.idx_lim);
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m[s] = ballot(p[s]);
    total += static_cast<uint32_t>(__popcll(m[s]));
  }
  if (total == 0) return 0u;
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(&sm.cnt[cur], total);
  base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0));
  const uint32_t after = base + total;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (m[s]) {
      if (p[s]) {
        const uint32_t pos = base + mbcnt64(m[s]);
        sm.val[pos] = __float_as_uint(f[s]);
        sm.idx[pos] = col(s);
      }
      base += static_cast<uint32_t>(__popcll(m[s]));
    }
  }
  return after;
}

template <bool BF16, int V, int NT>
__device__ __forceinline__ void load_block(uint4 (&r)[V], const char* xrow, uint32_t blk,
                                           uint32_t L) {
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  const uint32_t e0 = blk * static_cast<uint32_t>(kBlockElems) + threadIdx.x * EPV;
  const uint32_t fill = BF16 ? 0x7FC07FC0u : kQNaN32;
  if (blk * static_cast<uint32_t>(kBlockElems) + kBlockElems <= L) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      r[v] = *reinterpret_cast<const uint4*>(xrow + static_cast<size_t>(e0 + v * NT * EPV) * ESZ);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const uint32_t e = e0 + v * NT * EPV;
      if (e < L)
        r[v] = *reinterpret_cast<const uint4*>(xrow + static_cast<size_t>(e) * ESZ);
      else
        r[v] = make_uint4(fill, fill, fill, fill);
    }
  }
}

template <int NT, int CAP, int KMAX>
__device__ __forceinline__ void write_outputs(Smem<CAP, NT>& sm, const KArgs& a, bool bf16, int row, int cur,
                              uint32_t status) {
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t k = a.k;
  const int64_t out0 = static_cast<int64_t>(row) * k;
  uint32_t m = sm.cnt[cur];
  if (status) m = 0;

  if (!status && a.sorted != 0 && m > 1) {
    // Group by bin, then rank inside each bin.  Bins ascend in output order.
    const bool by_value = a.sorted == 1;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (uint32_t i = t; i < m; i += NT) {
      const uint32_t q = by_value ? key_of_bits(sm.val[i]) : sm.idx[i];
      lo = min(lo, q);
      hi = max(hi, q);
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (t == 0) {
      sm.res[0] = 0xFFFFFFFFu;
      sm.res[1] = 0u;
    }
    hist_clear(sm);
    __syncthreads();
    if (lane == 0) {
      atomicMin(&sm.res[0], lo);
      atomicMax(&sm.res[1], hi);
    }
    __syncthreads();
    lo = sm.res[0];
    hi = sm.res[1];
    const uint32_t span = hi - lo;
    const uint32_t shift = bit_length(span) > kRadixBits ? bit_length(span) - kRadixBits : 0u;
    auto bin_of = [&](uint32_t v, uint32_t i) -> uint32_t {
      return by_value ? (hi - key_of_bits(v)) >> shift : (i - lo) >> shift;
    };
    auto better = [&](uint32_t va, uint32_t ia, uint32_t vb, uint32_t ib) -> bool {
      if (!by_value) return ia < ib;
      const uint32_t ka = key_of_bits(va), kb = key_of_bits(vb);
      return ka > kb || (ka == kb && ia < ib);
    };
    for (uint32_t i = t; i < m; i += NT) atomicAdd(&sm.hist[bin_of(sm.val[i], sm.idx[i])], 1u);
    __syncthreads();
    hist_exclusive_scan(sm);
    uint32_t* gval = sm.val + KMAX;
    uint32_t* gidx = sm.idx + KMAX;
    for (uint32_t i = t; i < m; i += NT) {
      const uint32_t v = sm.val[i], ix = sm.idx[i];
      const uint32_t p = atomicAdd(&sm.hist[bin_of(v, ix)], 1u);
      gval[p] = v;
      gidx[p] = ix;
    }
    __syncthreads();
    for (uint32_t p = t; p < m; p += NT) {
      const uint32_t v = gval[p], ix = gidx[p];
      const uint32_t b = bin_of(v, ix);
      const uint32_t s = b ? sm.hist[b - 1] : 0u;
      const uint32_t e = sm.hist[b];
      uint32_t rank = 0;
      for (uint32_t q = s; q < e; ++q) rank += better(gval[q], gidx[q], v, ix) ? 1u : 0u;
      sm.val[s + rank] = v;
      sm.idx[s + rank] = ix;
    }
    __syncthreads();
  }

  for (uint32_t j = t; j < k; j += NT) {
    uint32_t ix, v;
    if (j < m) {
      ix = sm.idx[j];
      v = sm.val[j];
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

template <bool BF16, int CLS>
__global__ __launch_bounds__(class_threads(CLS)) void topk_kernel(KArgs a) {
  constexpr int NT = class_threads(CLS);
  constexpr int CAP = class_cap(CLS);
  constexpr int KMAX = class_kmax(CLS);
  constexpr int EPV = BF16 ? 8 : 4;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int V = kBlockElems / (NT * EPV);
  static_assert(V >= 1 && V * NT * EPV == kBlockElems, "block geometry");
  __shared__ Smem<CAP, NT> sm;

  const int t = threadIdx.x, lane = t & 63;
  const int S = a.segments;
  const int seg = static_cast<int>(blockIdx.x) % S;
  int row = static_cast<int>(blockIdx.x) / S;
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
  if (t == 0) {
    sm.cnt[0] = 0u;
    sm.cnt[1] = 0u;
    sm.hikey = 0u;
    sm.flags = 0u;
    sm.thr = kThrInit;
  }
  __syncthreads();

  unsigned long long* thr_g = S > 1 ? a.ws_thr + row : nullptr;
  const uint32_t k = static_cast<uint32_t>(a.k);
  const uint32_t trigger = static_cast<uint32_t>(a.trigger);
  const uint32_t slack = (trigger - k) / 4u;
  int cur = 0;
  uint64_t thr = kThrInit;
  Filter F = filter_of(thr);
  float hi_lane = __uint_as_float(kNegInf32);
  bool nan_lane = false;

  const uint32_t nb = (L + kBlockElems - 1) / kBlockElems;
  const uint32_t ntl = nb > static_cast<uint32_t>(seg) ? (nb - seg + S - 1) / S : 0u;
  const BlockOrder order(nb, a.perm_seed, static_cast<uint32_t>(row), a.in_order != 0);
  const char* xrow = static_cast<const char*>(a.x) + static_cast<int64_t>(row) * a.row_stride * ESZ;
  const bool ragged_row = (L % kBlockElems) != 0;
  const uint32_t last_blk = nb - 1u;

  uint4 ra[V], rb[V];
  uint64_t g = 0;

  // The decision to cut must be the same in every wave, but a fast wave may
  // append for the next block before a slow wave has looked at the counter.
  // So each wave records the count its own append produced, in a slot chosen
  // by step parity; the maximum over the waves is the count after the block.
  int par = 0;
  auto count_after_step = [&](uint32_t after) -> uint32_t {
    if (lane == 0) sm.snap[par][t >> 6] = after;
    __syncthreads();
    uint32_t c = 0;
#pragma unroll
    for (int w2 = 0; w2 < NT / 64; ++w2) c = max(c, sm.snap[par][w2]);
    par ^= 1;
    return c;
  };

  auto step = [&](uint4 (&cur_r)[V], uint4 (&nxt_r)[V], uint32_t u) {
    const uint32_t blk = order(seg + u * S);
    if (S > 1) g = load_thr(thr_g);
    if (u + 1 < ntl) load_block<BF16, V, NT>(nxt_r, xrow, order(seg + (u + 1) * S), L);
    uint32_t after;
    if (ragged_row && blk == last_blk)
      after = filter_block<BF16, true, V, NT, CAP>(cur_r, blk, L, F, hi_lane, nan_lane, sm, cur);
    else
      after = filter_block<BF16, false, V, NT, CAP>(cur_r, blk, L, F, hi_lane, nan_lane, sm, cur);
    if (S > 1 && g > thr && lane == 0) atomicMax(&sm.thr, static_cast<unsigned long long>(g));
    const uint32_t c = count_after_step(after);
    if (c > trigger) {
      const uint64_t before = sm.thr;
      cur = cut_buffer<NT, CAP>(sm, cur, k, k + slack, L, hi_lane);
      thr = sm.thr;
      if (S > 1 && t == 0 && thr > before) publish_thr(thr_g, thr);
    } else if (S > 1) {
      const uint64_t seen = sm.thr;   // may already include a later wave's raise: still a valid bound
      thr = seen > thr ? seen : thr;
    }
    F = filter_of(thr);
  };

  if (ntl > 0) load_block<BF16, V, NT>(ra, xrow, order(seg), L);
  uint32_t u = 0;
  for (; u + 1 < ntl; u += 2) {
    step(ra, rb, u);
    step(rb, ra, u + 1);
  }
  if (u < ntl) step(ra, rb, u);

  // NaN anywhere in this workgroup's share of [0, L).
  if (ballot(nan_lane) && lane == 0) atomicOr(&sm.flags, static_cast<uint32_t>(DS_ROW_NAN));
  // Exact local top-k (drops anything at or below the current threshold too).
  cur = cut_buffer<NT, CAP>(sm, cur, k, k, L, hi_lane);

  if (S > 1) {
    const uint32_t mine = sm.cnt[cur];
    const int64_t slot = static_cast<int64_t>(row) * S + seg;
    if (t == 0) {
      if (mine >= k) publish_thr(thr_g, sm.thr);
      a.ws_cnt[slot] = mine;
      if (sm.flags) atomicOr(&a.ws_flags[row], sm.flags);
    }
    uint32_t* wv = a.ws_val + slot * k;
    uint32_t* wi = a.ws_idx + slot * k;
    for (uint32_t j = t; j < mine; j += NT) {
      wv[j] = sm.val[j];
      wi[j] = sm.idx[j];
    }
    __threadfence();
    __syncthreads();
    if (t == 0) {
      const uint32_t prev = atomicAdd(&a.ws_done[row], 1u);
      sm.is_last = prev == static_cast<uint32_t>(S - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!sm.is_last) return;
    __threadfence();

    // Last arrival: merge the other workgroups' survivors.
    const uint64_t gfin = load_thr(thr_g);
    if (t == 0) {
      if (gfin > sm.thr) sm.thr = gfin;
      sm.flags |= __hip_atomic_load(&a.ws_flags[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // The workspace must be all zero again when the call ends, whatever layout
    // the next call uses: clear this workgroup's own survivors now, and every
    // other slot and count as it is read below.
    for (uint32_t j = t; j < mine; j += NT) {
      wv[j] = 0u;
      wi[j] = 0u;
    }
    // Per-segment counts -> exclusive offsets (own segment counted as 0).
    hist_clear(sm);
    __syncthreads();
    for (int s2 = t; s2 < S; s2 += NT) {
      const int64_t sl = static_cast<int64_t>(row) * S + s2;
      sm.hist[s2] = s2 == seg ? 0u : a.ws_cnt[sl];
      a.ws_cnt[sl] = 0u;
    }
    __syncthreads();
    hist_exclusive_scan(sm);   // hist[s] = first flat position of segment s
    for (int s2 = t; s2 < S; s2 += NT) sm.segoff[s2] = sm.hist[s2];
    const uint32_t total = sm.hist[kBins - 1];
    __syncthreads();
    thr = sm.thr;
    F = filter_of(thr);
    constexpr int PER = kBlockElems / NT;
    for (uint32_t c0 = 0; c0 < total; c0 += kBlockElems) {
      uint32_t mv[PER], mi[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const uint32_t fpos = c0 + t + q * NT;
        mv[q] = kQNaN32;
        mi[q] = 0u;
        if (fpos < total) {
          // segment: the last one whose first position is <= fpos (empty ones share it)
          int lo = 0, hi = S - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sm.segoff[mid] <= fpos) lo = mid; else hi = mid - 1;
          }
          const int64_t sl = static_cast<int64_t>(row) * S + lo;
          const uint32_t j = fpos - sm.segoff[lo];
          mv[q] = a.ws_val[sl * k + j];
          mi[q] = a.ws_idx[sl * k + j];
          a.ws_val[sl * k + j] = 0u;
          a.ws_idx[sl * k + j] = 0u;
        }
      }
      uint64_t mm[PER];
      bool p[PER];
      uint32_t tot = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const float fv = __uint_as_float(mv[q]);
        p[q] = fv > F.f || (fv == F.f && mi[q] < F.idx_lim);   // the NaN fill never passes
        if (p[q]) hi_lane = fmaxf(hi_lane, fv);
        mm[q] = ballot(p[q]);
        tot += static_cast<uint32_t>(__popcll(mm[q]));
      }
      uint32_t after = 0;
      if (tot) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&sm.cnt[cur], tot);
        base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0));
        after = base + tot;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          if (mm[q]) {
            if (p[q]) {
              const uint32_t pos = base + mbcnt64(mm[q]);
              sm.val[pos] = mv[q];
              sm.idx[pos] = mi[q];
            }
            base += static_cast<uint32_t>(__popcll(mm[q]));
          }
        }
      }
      if (count_after_step(after) > trigger) {
        cur = cut_buffer<NT, CAP>(sm, cur, k, k + slack, L, hi_lane);
        F = filter_of(sm.thr);
      }
    }
    cur = cut_buffer<NT, CAP>(sm, cur, k, k, L, hi_lane);
    if (t == 0) {
      a.ws_done[row] = 0u;
      a.ws_thr[row] = 0ull;
      a.ws_flags[row] = 0u;
    }
  }

  status |= sm.flags;
  write_outputs<NT, CAP, KMAX>(sm, a, BF16, row, cur, status);
}

}  // namespace

WsLayout ws_layout(int64_t batch, int segments, int k) {
  auto up = [](size_t v) { return (v + 15) & ~static_cast<size_t>(15); };
  WsLayout l{};
  const size_t b = static_cast<size_t>(batch);
  const size_t s = static_cast<size_t>(segments);
  l.thr = 0;
  l.done = up(l.thr + b * 8);
  l.flags = up(l.done + b * 4);
  l.cnt = up(l.flags + b * 4);
  l.val = up(l.cnt + b * s * 4);
  l.idx = up(l.val + b * s * static_cast<size_t>(k) * 4);
  l.total = up(l.idx + b * s * static_cast<size_t>(k) * 4);
  return l;
}

template <bool BF16, int CLS>
static int launch_one(const KArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.batch) * a.segments));
  const dim3 block(class_threads(CLS));
  hipLaunchKernelGGL((topk_kernel<BF16, CLS>), grid, block, 0, stream, a);
  return static_cast<int>(hipGetLastError());
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
