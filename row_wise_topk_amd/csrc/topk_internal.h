// Internal interface between the host API (topk_api.cpp) and the kernels
// (topk_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "ds_topk.h"

namespace dstk {

// Fixed geometry shared by host planning and the kernels.
constexpr int kBlockElems = 4096;   // B: contiguous elements per block (both dtypes)
constexpr int kNumCU = 256;         // MI355X compute units (planning constant)
constexpr int kMaxSegments = 256;
// Rows a plan may share between workgroups, and the workspace header that
// holds their counters (DS_TOPK_MAX_SPLIT_ROWS, DS_TOPK_WS_HEADER_BYTES).
constexpr int64_t kMaxSplitRows = DS_TOPK_MAX_SPLIT_ROWS;
constexpr size_t kWsHeaderBytes = DS_TOPK_WS_HEADER_BYTES;

// k classes: each has its own buffer capacity, threads per workgroup and trigger.
constexpr int kNumClasses = 4;
constexpr int class_kmax(int c) { return c == 0 ? 256 : c == 1 ? 1024 : c == 2 ? 2048 : 4096; }
// Threads per workgroup: 512 for the largest k class, and for fp32 rows
// shared by several workgroups (a 16-byte-per-lane block of 512 threads
// keeps 48 KB in flight per CU, as two workgroups of 256 do; the post-stream
// passes of the one workgroup per CU then run on twice the waves).  256
// otherwise: bf16 blocks are half the bytes, and rows with one workgroup
// each want two workgroups per CU.
constexpr int kernel_threads(int c, int dtype, bool multi) {
  return (c == 3 || (dtype == 0 && multi)) ? 512 : 256;
}
// B2 (extra candidates collected before a cut) per class.
constexpr int class_b2(int c) { return c == 0 ? 1024 : c == 1 ? 3072 : class_kmax(c); }
// Buffer capacity: k + B2 candidates plus one whole block admitted at once.
constexpr int class_cap(int c) { return class_kmax(c) + class_b2(c) + kBlockElems; }
constexpr int class_trigger(int c) { return class_cap(c) - kBlockElems; }
// LDS bytes per workgroup (candidate composites, histogram, scalars).
constexpr int class_lds_bytes(int c) { return class_cap(c) * 8 + 2048 * 4 + 1536; }
// The kernels are built for two waves per SIMD (up to 256 VGPRs a lane), so
// a CU (4 SIMDs) holds 8 waves: 2 workgroups of 256 threads or 1 of 512.
constexpr int kWavesPerSimd = 2;
// Workgroups of class c with nt threads resident on one CU: the smaller of
// the LDS and the register limits.
constexpr int wgs_per_cu(int c, int nt) {
  const int lds = (160 * 1024) / class_lds_bytes(c);
  const int regs = kWavesPerSimd * 4 * 64 / nt;
  const int w = lds < regs ? lds : regs;
  return w > 0 ? w : 1;
}
inline int class_of_k(int k) { return k <= 256 ? 0 : k <= 1024 ? 1 : k <= 2048 ? 2 : 3; }

// ---- chunk kernels (chunk_kernels.hip)
// A chunk: kChunkLoads 16-byte loads per lane of the workgroup, all in
// flight at once.  chunk_kernels.hip is built twice, for whole rows and for
// split rows; both use 512-lane workgroups, two per CU, so that a row's
// merge and exact selection run on 8 waves.
constexpr int kChunkThreadsRow = 512;
constexpr int kChunkThreadsSplit = 512;
constexpr int kChunkLoads = 8;
constexpr int64_t chunk_elems(int dtype, int nt) { return int64_t{nt} * kChunkLoads * (dtype == 0 ? 4 : 8); }
// Candidate buffer: k plus room for the larger of k and one bf16 vector per
// lane (8 values per lane).
constexpr int chunk_room(int nt) { return nt * 8; }
constexpr int chunk_cap(int c, int nt) {
  return class_kmax(c) + (class_kmax(c) > chunk_room(nt) ? class_kmax(c) : chunk_room(nt));
}
// Rows of at most this many whole-row chunks go to the chunk kernels by default.
constexpr int64_t kChunkMaxPerRow = 64;
// Below this many rows, a row is split into one workgroup per chunk.
constexpr int64_t kChunkSplitBatch = 512;

struct CArgs {
  const void* x;
  int64_t row_stride;     // elements
  int32_t n_cols;
  int32_t batch;
  const int32_t* end;     // nullable
  int32_t k;
  int32_t sorted;
  int32_t return_values;
  int32_t idx64;
  void* values;
  void* indices;
  int32_t* row_status;
  int32_t segments;       // 1 (a whole row per workgroup) or the row's chunk count
  uint32_t perm_seed;     // chunk visiting order of a whole row
  int32_t in_order;
  int32_t reverse_rows;   // segments == 1: workgroup g takes row batch-1-g
  uint32_t cap_eff;       // candidate count that triggers a cut (<= chunk_cap)
  // workspace (segments > 1)
  uint32_t* ws_arrive;            // [batch] arrivals per row, zero at rest
  unsigned long long* ws_rec;     // [batch * segments * 2] threshold, (status << 32) | count
  unsigned long long* ws_slot;    // [batch * segments * k] candidate composites
  uint32_t* stats;                // nullable: [batch * 4] counts added per row (DS_STAT_*)
};

struct ChunkWs {
  size_t arrive, rec, slot, total;
};
ChunkWs chunk_ws_layout(int64_t batch, int segments, int k);

// Queue the chunk kernel for k class `cls` and dtype (0 fp32, 1 bf16).
// Returns the hipError_t of the launch.
int launch_chunk_row(const CArgs& a, int dtype, int cls, hipStream_t stream);
int launch_chunk_split(const CArgs& a, int dtype, int cls, hipStream_t stream);
// Queue the read-ceiling kernel of the chunk kernels' access pattern.
int launch_chunk_read_row(const CArgs& a, int dtype, uint32_t* sink, hipStream_t stream);
int launch_chunk_read_split(const CArgs& a, int dtype, uint32_t* sink, hipStream_t stream);

// Survivor slots a shared row's workgroup may hand over beyond k.
constexpr int kStreamSlotSlack = 64;

struct KArgs {
  const void* x;
  int64_t row_stride;     // elements
  int32_t n_cols;
  int32_t batch;
  const int32_t* end;     // nullable
  int32_t k;
  int32_t sorted;
  int32_t return_values;
  int32_t idx64;
  void* values;
  void* indices;
  int32_t* row_status;
  int32_t segments;       // workgroups per row
  uint32_t perm_seed;
  int32_t in_order;
  int32_t trigger;        // candidate count that triggers a cut
  // workspace (segments > 1), all device pointers into one caller buffer
  unsigned long long* ws_thr;   // [batch]  shared threshold per row
  uint32_t* ws_done;            // [batch]  arrivals per row
  uint32_t* ws_flags;           // [batch]  OR of row status bits
  uint32_t* ws_fill;            // [batch]  survivors written so far per row
  unsigned long long* ws_x;     // [batch * segments]  per-workgroup merge bound
  unsigned long long* ws_spec;  // [batch]  largest estimated start used on the row (0: none)
  unsigned long long* ws_comp;  // [batch * segments * (k + 64)]  candidate composites, contiguous per row
  uint32_t* stats;              // nullable: [batch * 4] counts added per row (DS_STAT_*)
};

// Workspace layout for `segments` workgroups per row (bytes, 16-B aligned parts).
struct WsLayout {
  size_t thr, done, flags, fill, x, spec, comp, total;
};
WsLayout ws_layout(int64_t batch, int segments, int k);

// Queue the kernel for class `cls` and dtype (0 fp32, 1 bf16).  Returns the
// hipError_t of the launch.
int launch_topk(const KArgs& a, int dtype, int cls, hipStream_t stream);

// Queue the read-ceiling kernel (same grid and loads as launch_topk, no
// selection).  Returns the hipError_t of the launch.
int launch_read(const KArgs& a, int dtype, int cls, uint32_t* sink, hipStream_t stream);

}  // namespace dstk
