// Host-only test of the C ABI's argument checks, launch plans and workspace
// layouts (row_wise_topk_amd/csrc/topk_api.cpp), built with
// -fsanitize=address,undefined.  The kernel launchers are replaced by stubs
// that check the arguments the API hands them: every pointer they receive
// into the workspace lies inside it, and every field is in range.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "ds_topk.h"
#include "topk_internal.h"

static int fails = 0;
static int launches = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static const char* g_ws = nullptr;
static size_t g_ws_bytes = 0;
static bool in_ws(const void* p, size_t bytes) {
  const char* c = static_cast<const char*>(p);
  return g_ws && c >= g_ws && c + bytes <= g_ws + g_ws_bytes;
}

namespace dstk {
int launch_topk(const KArgs& a, int dtype, int cls, hipStream_t) {
  ++launches;
  CHECK(dtype == 0 || dtype == 1);
  CHECK(cls >= 0 && cls < kNumClasses);
  CHECK(a.segments >= 1 && a.segments <= kMaxSegments);
  CHECK(a.k >= 1 && a.k <= DS_TOPK_MAX_K);
  if (a.segments > 1) {
    const WsLayout l = ws_layout(a.batch, a.segments, a.k);
    CHECK(in_ws(a.ws_comp, l.total - l.comp));
    CHECK(in_ws(a.ws_thr, 8));
  }
  return 0;
}
int launch_read(const KArgs& a, int, int, uint32_t* sink, hipStream_t) {
  ++launches;
  CHECK(sink != nullptr);
  CHECK(a.segments >= 1);
  return 0;
}
static void check_chunk(const CArgs& a, int dtype, int cls, int nt, bool split) {
  ++launches;
  CHECK(dtype == 0 || dtype == 1);
  CHECK(cls >= 0 && cls < kNumClasses);
  CHECK(a.segments >= 1 && a.segments <= kMaxSegments);
  CHECK((a.segments > 1) == split);
  CHECK(a.cap_eff >= static_cast<uint32_t>(a.k + chunk_room(nt)) ||
        a.cap_eff == static_cast<uint32_t>(chunk_cap(cls, nt)));
  CHECK(a.cap_eff <= static_cast<uint32_t>(chunk_cap(cls, nt)));
  if (a.segments > 1) {
    const ChunkWs l = chunk_ws_layout(a.batch, a.segments, a.k);
    CHECK(in_ws(a.ws_arrive, static_cast<size_t>(a.batch) * 4));
    CHECK(in_ws(a.ws_rec, static_cast<size_t>(a.batch) * a.segments * 16));
    CHECK(in_ws(a.ws_slot, static_cast<size_t>(a.batch) * a.segments * a.k * 8));
    CHECK(l.total <= g_ws_bytes);
  }
}
int launch_chunk_row(const CArgs& a, int dtype, int cls, hipStream_t) {
  check_chunk(a, dtype, cls, kChunkThreadsRow, false);
  return 0;
}
int launch_chunk_split(const CArgs& a, int dtype, int cls, hipStream_t) {
  check_chunk(a, dtype, cls, kChunkThreadsSplit, true);
  return 0;
}
static void check_read(const CArgs& a, uint32_t* sink) {
  ++launches;
  CHECK(sink != nullptr);
  CHECK(a.segments >= 1);
}
int launch_chunk_read_row(const CArgs& a, int, uint32_t* sink, hipStream_t) {
  check_read(a, sink);
  return 0;
}
int launch_chunk_read_split(const CArgs& a, int, uint32_t* sink, hipStream_t) {
  check_read(a, sink);
  return 0;
}
}  // namespace dstk

int main() {
  std::mt19937_64 rng(7);
  alignas(16) static char x[64];
  alignas(16) static char out[64];
  alignas(16) static int32_t st[16];
  for (int trial = 0; trial < 20000; ++trial) {
    // Odd trials: arguments drawn around their limits (most invalid).  Even
    // trials: valid arguments of every shape class.
    const bool wild = trial & 1;
    const ds_dtype_t dt = static_cast<ds_dtype_t>(rng() % (wild ? 3 : 2));   // 2 is invalid
    const int64_t batch = wild ? static_cast<int64_t>(rng() % 5000) - 1 : 1 + static_cast<int64_t>(rng() % 5000);
    const int64_t n_cols = trial % 7 == 0 ? static_cast<int64_t>(rng() % 3000000000ull)
                                          : static_cast<int64_t>(rng() % 600000);
    const int64_t step = dt == DS_BF16 ? 8 : 4;
    const int64_t stride = wild ? n_cols + static_cast<int64_t>(rng() % 16) - 2
                                : (n_cols + step - 1) / step * step + step * static_cast<int64_t>(rng() % 3);
    const int32_t k = wild ? static_cast<int32_t>(rng() % 4200) : 1 + static_cast<int32_t>(rng() % 4096);
    const int32_t sorted = static_cast<int32_t>(rng() % (wild ? 4 : 3));
    ds_topk_plan_t plan{static_cast<int32_t>(rng() % 300) - (wild ? 20 : 0), static_cast<uint32_t>(rng()),
                        static_cast<int32_t>(rng() % (wild ? 3 : 2)),
                        wild || rng() % 2 ? static_cast<int32_t>(rng() % 9000) : 0,
                        static_cast<int32_t>(rng() % (wild ? 4 : 3))};
    const bool use_plan = rng() % 2;
    const size_t need = ds_topk_workspace_size_ex(dt, batch, n_cols, k, use_plan ? &plan : nullptr);
    // The host side never touches the workspace: a fake, aligned address range.
    char* wsp = reinterpret_cast<char*>(uintptr_t{1} << 40);
    g_ws = wsp;
    g_ws_bytes = need;
    const ds_status_t v = ds_topk_validate(x, dt, batch, n_cols, stride, nullptr, k, sorted, 1,
                                           DS_INT32, out, out, st, need ? wsp : nullptr, need,
                                           use_plan ? &plan : nullptr);
    const int before = launches;
    const ds_status_t r = ds_topk_ex(x, dt, batch, n_cols, stride, nullptr, k, sorted, 1, DS_INT32,
                                     out, out, st, need ? wsp : nullptr, need, nullptr,
                                     use_plan ? &plan : nullptr);
    CHECK(r == v);
    CHECK((r == DS_OK && batch > 0) == (launches == before + 1));
    // One byte short of the workspace is refused.
    if (v == DS_OK && need > 0) {
      CHECK(ds_topk_validate(x, dt, batch, n_cols, stride, nullptr, k, sorted, 1, DS_INT32, out,
                             out, st, wsp, need - 1, use_plan ? &plan : nullptr) == DS_ERR_WORKSPACE);
    }
    uint32_t sink = 0;
    ds_read_ceiling(x, dt, batch, n_cols, stride, nullptr, k, use_plan ? &plan : nullptr, &sink, nullptr);
  }
  for (int s = 0; s <= 12; ++s) CHECK(ds_topk_status_string(static_cast<ds_status_t>(s)) != nullptr);
  printf(fails ? "api sanitize: %d failures\n" : "api sanitize: ok (%d launches)\n", fails ? fails : launches);
  return fails ? 1 : 0;
}
