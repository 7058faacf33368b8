// CPU oracle for row-wise TopK.  TEST INFRASTRUCTURE ONLY: the tests, the
// smoke check and the benchmark's CPU-baseline leg load this; the product path
// never does.  It shares no code, header, table or helper with the HIP library.
//
// What it computes is the plain definition of the result that the streaming
// threshold method reaches exactly, written out with a library sort:
//
//   [NC]  narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for sparse
//         attention and sampling": the method paragraph (threshold T, blocks B
//         and B2, radix select back to k) -- the method only discards values
//         that cannot be among the k largest, so its result is the plain top-k;
//         the coverage paragraph (bf16 / fp32 inputs, k <= 4096, int32 / int64
//         indices); the install/API paragraph (sorted_index, return_value,
//         contiguous last dimension); the NaN paragraph (NaN is always checked).
//   [AF]  aifluxnews.com, "DeepSeek 在 GitHub 发布 DeepSelect v1.0.0", section
//         "PyTorch 接口与 CUDA 环境要求": per-row `end` gives each row its own
//         valid range.
//   [XH]  xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！", Q&A: the
//         call deep_select.topk(x, topk, sorted_index, indices_type,
//         return_value), and results are stable (the same input always gives
//         the same result).
//
// Readings where the pages are silent (each is listed in the design notes):
//   * order: a precedes b iff v[a] > v[b], or v[a] == v[b] and a < b
//     (numeric IEEE comparison, so -0.0 == +0.0 and +-inf are ordinary values);
//   * NaN anywhere in [0, end) marks the row (status 1) instead of aborting, and
//     the row's outputs become index -1 / value qNaN; this is checked for every
//     row, including rows no longer than k;
//   * end outside [0, n_cols] marks the row (status 2), outputs as for NaN;
//   * a row with fewer than k valid elements is padded with index -1 / -inf;
//   * sorted: 1 = by value (the order above), 2 = by index ascending (the
//     pages' sorted_index), 0 = any order -- the oracle emits index order;
//   * values are bit copies of the selected inputs.
// The padding values, the NaN-row fill and the status codes are this
// library's own conventions, not fixed by any page: parity unpinned for those
// three (the tests check them only as closed forms).  Everything else is
// pinned by brute force, library routines, hand-derived cases and invariants.
//
// bf16 inputs are widened exactly (the 16 bits become the top half of an
// fp32); every comparison is done on doubles, which is exact for both dtypes.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

constexpr int kFp32 = 0;
constexpr int kBf16 = 1;
constexpr int kIdx32 = 0;

constexpr int kRowNan = 1;
constexpr int kRowBadEnd = 2;

struct Args {
  const void* x;
  int dtype;
  int64_t batch, n_cols, row_stride;
  const int32_t* end;
  int32_t k, sorted, return_values, index_dtype;
  void* values;
  void* indices;
  int32_t* row_status;
};

// Element j of row i as a double, exactly.
double load(const Args& a, int64_t i, int64_t j) {
  const int64_t off = i * a.row_stride + j;
  float f;
  if (a.dtype == kFp32) {
    std::memcpy(&f, static_cast<const char*>(a.x) + off * 4, 4);
  } else {
    uint16_t h;
    std::memcpy(&h, static_cast<const char*>(a.x) + off * 2, 2);
    const uint32_t w = static_cast<uint32_t>(h) << 16;
    std::memcpy(&f, &w, 4);
  }
  return static_cast<double>(f);
}

void put_index(const Args& a, int64_t i, int64_t slot, int64_t v) {
  const int64_t off = i * a.k + slot;
  if (a.index_dtype == kIdx32) {
    static_cast<int32_t*>(a.indices)[off] = static_cast<int32_t>(v);
  } else {
    static_cast<int64_t*>(a.indices)[off] = v;
  }
}

// Copy the raw bits of x[i, j] (j >= 0) or a fixed pattern (fp32 bits given,
// narrowed to the top half for bf16) into values[i, slot].
void put_value_bits(const Args& a, int64_t i, int64_t slot, int64_t j, uint32_t fp32_pattern) {
  if (!a.return_values) return;
  const int64_t off = i * a.k + slot;
  if (a.dtype == kFp32) {
    uint32_t w = fp32_pattern;
    if (j >= 0) std::memcpy(&w, static_cast<const char*>(a.x) + (i * a.row_stride + j) * 4, 4);
    std::memcpy(static_cast<char*>(a.values) + off * 4, &w, 4);
  } else {
    uint16_t h = static_cast<uint16_t>(fp32_pattern >> 16);
    if (j >= 0) std::memcpy(&h, static_cast<const char*>(a.x) + (i * a.row_stride + j) * 2, 2);
    std::memcpy(static_cast<char*>(a.values) + off * 2, &h, 2);
  }
}

constexpr uint32_t kQNaN = 0x7FC00000u;
constexpr uint32_t kNegInf = 0xFF800000u;

void fill_row(const Args& a, int64_t i, int64_t from, uint32_t pattern) {
  for (int64_t s = from; s < a.k; ++s) {
    put_index(a, i, s, -1);
    put_value_bits(a, i, s, -1, pattern);
  }
}

// One row: the definition of top-k under the total order above, via a stable
// sort of positions by value descending (stability supplies the lower-index
// tie-break).  [NC] method/coverage/API paragraphs; [AF] `end`; [XH] stability.
void oracle_row(const Args& a, int64_t i) {
  const int64_t L = a.end ? static_cast<int64_t>(a.end[i]) : a.n_cols;
  if (L < 0 || L > a.n_cols) {
    a.row_status[i] = kRowBadEnd;
    fill_row(a, i, 0, kQNaN);
    return;
  }
  std::vector<double> v(static_cast<size_t>(L));
  bool has_nan = false;
  for (int64_t j = 0; j < L; ++j) {
    v[j] = load(a, i, j);
    if (std::isnan(v[j])) has_nan = true;
  }
  if (has_nan) {  // [NC] NaN paragraph: always checked; here a status, not an abort
    a.row_status[i] = kRowNan;
    fill_row(a, i, 0, kQNaN);
    return;
  }
  std::vector<int64_t> perm(static_cast<size_t>(L));
  std::iota(perm.begin(), perm.end(), int64_t{0});
  std::stable_sort(perm.begin(), perm.end(),
                   [&](int64_t p, int64_t q) { return v[p] > v[q]; });
  const int64_t m = std::min<int64_t>(a.k, L);
  std::vector<int64_t> sel(perm.begin(), perm.begin() + m);
  if (a.sorted != 1) std::sort(sel.begin(), sel.end());  // 2: by index; 0: any (index order)
  for (int64_t s = 0; s < m; ++s) {
    put_index(a, i, s, sel[s]);
    put_value_bits(a, i, s, sel[s], 0);
  }
  fill_row(a, i, m, kNegInf);
  a.row_status[i] = 0;
}

}  // namespace

extern "C" {

// Returns 0 on success, -1 on an argument the oracle does not accept.
// Host pointers only.  Rows are dealt round-robin to `n_threads` threads
// (<= 0: one per hardware thread).
int oracle_topk(const void* x, int dtype, int64_t batch, int64_t n_cols, int64_t row_stride,
                const int32_t* end, int32_t k, int32_t sorted, int32_t return_values,
                int32_t index_dtype, void* values, void* indices, int32_t* row_status,
                int32_t n_threads) {
  if (dtype != kFp32 && dtype != kBf16) return -1;
  if (index_dtype != 0 && index_dtype != 1) return -1;
  if (sorted < 0 || sorted > 2) return -1;
  if (k < 1 || batch < 0 || n_cols < 0 || row_stride < n_cols) return -1;
  if (batch > 0 && (!indices || !row_status || (return_values && !values))) return -1;
  if (batch > 0 && n_cols > 0 && !x) return -1;
  Args a{x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values, index_dtype,
         values, indices, row_status};
  int nt = n_threads > 0 ? n_threads : static_cast<int>(std::thread::hardware_concurrency());
  if (nt < 1) nt = 1;
  if (nt > batch) nt = static_cast<int>(std::max<int64_t>(batch, 1));
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&a, t, nt]() {
      for (int64_t i = t; i < a.batch; i += nt) oracle_row(a, i);
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}

}  // extern "C"
