// Host side of the C ABI in include/ds_topk.h: argument checks, launch plan,
// workspace layout, one kernel launch on the caller's stream.
//
// The interface follows the pages' description of DeepSelect's topk call
// (xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！", Q&A; narracomm.com,
// "DeepSeek releases DeepSelect, a TopK kernel for sparse attention and
// sampling", coverage and install/API paragraphs; aifluxnews.com,
// "DeepSeek 在 GitHub 发布 DeepSelect v1.0.0", section "PyTorch 接口与 CUDA
// 环境要求").  The kernels are chosen per problem shape, as those pages say the
// fastest TopK depends on dtype, batch, vocabulary and k.

#include <stdint.h>

#include <climits>

#include "ds_topk.h"
#include "topk_internal.h"

namespace {

using namespace dstk;

struct Plan {
  int kernel;     // DS_KERNEL_STREAM or DS_KERNEL_CHUNK
  int cls;
  int segments;
  uint32_t seed;
  int in_order;
  int trigger;
};

int elem_size(ds_dtype_t d) { return d == DS_FP32 ? 4 : 2; }

bool misaligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0;
}

// Workgroups per row: enough to fill every CU's workgroup slots, at least two
// blocks each.  Shared fp32 rows use 512-thread workgroups, one per CU, so
// they are planned for that.
int auto_segments(int64_t batch, int64_t n_cols, int cls, int dtype) {
  const int64_t nb = (n_cols + kBlockElems - 1) / kBlockElems;
  if (batch <= 0 || nb <= 1) return 1;
  auto plan_for = [&](int nt) {
    const int64_t target = static_cast<int64_t>(kNumCU) * wgs_per_cu(cls, nt);
    int64_t s = (target + batch - 1) / batch;
    const int64_t most = (nb + 1) / 2;   // at least two blocks per workgroup
    if (s > most) s = most;
    if (s > kMaxSegments) s = kMaxSegments;
    if (s < 1) s = 1;
    return s;
  };
  int64_t s = plan_for(kernel_threads(cls, dtype, false));
  if (s > 1 && kernel_threads(cls, dtype, true) != kernel_threads(cls, dtype, false)) {
    const int64_t s2 = plan_for(kernel_threads(cls, dtype, true));
    if (s2 > 1) s = s2;
  }
  return static_cast<int>(s);
}

// Chunks of a row of n_cols values, for workgroups of nt lanes.
int64_t chunks_of(int64_t n_cols, int dtype, int nt) {
  const int64_t ce = chunk_elems(dtype, nt);
  return (n_cols + ce - 1) / ce;
}

// Workgroups per row for the chunk kernels: one (1024-lane) workgroup per
// split chunk when the batch is too small to fill the chip with whole rows,
// else one (256-lane) workgroup per row.
int chunk_segments(int64_t batch, int64_t n_cols, int dtype) {
  const int64_t nch = chunks_of(n_cols, dtype, kChunkThreadsSplit);
  return (batch < kChunkSplitBatch && nch > 1 && nch <= kMaxSegments) ? static_cast<int>(nch) : 1;
}

// Fills `out`; returns DS_ERR_PLAN for an out-of-range override.
ds_status_t resolve_plan(int64_t batch, int64_t n_cols, int32_t k, ds_dtype_t dtype,
                         const ds_topk_plan_t* p, Plan* out) {
  const int dt = dtype == DS_BF16 ? 1 : 0;
  Plan pl{};
  pl.cls = class_of_k(k);
  pl.kernel = chunks_of(n_cols, dt, kChunkThreadsRow) <= kChunkMaxPerRow ? DS_KERNEL_CHUNK
                                                                         : DS_KERNEL_STREAM;
  const int64_t nch = chunks_of(n_cols, dt, kChunkThreadsSplit);   // split chunks
  pl.seed = 0x5EEDu;
  pl.in_order = 0;
  if (p) {
    if (p->kernel < DS_KERNEL_AUTO || p->kernel > DS_KERNEL_CHUNK) return DS_ERR_PLAN;
    if (p->kernel != DS_KERNEL_AUTO) pl.kernel = p->kernel;
  }
  if (pl.kernel == DS_KERNEL_CHUNK) {
    pl.segments = chunk_segments(batch, n_cols, dt);
  } else {
    pl.segments = auto_segments(batch, n_cols, pl.cls, dt);
    pl.trigger = class_trigger(pl.cls);
  }
  if (p) {
    if (p->segments < 0 || p->segments > kMaxSegments) return DS_ERR_PLAN;
    if (p->in_order != 0 && p->in_order != 1) return DS_ERR_PLAN;
    if (p->flush_at != 0 && (p->flush_at <= k || p->flush_at > class_trigger(pl.cls)))
      return DS_ERR_PLAN;
    if (pl.kernel == DS_KERNEL_CHUNK) {
      if (p->segments == 1) pl.segments = 1;
      else if (p->segments > 1) {
        if (nch > kMaxSegments) return DS_ERR_PLAN;
        pl.segments = nch > 1 ? static_cast<int>(nch) : 1;
      }
    } else {
      if (p->segments > 0) pl.segments = p->segments;
      if (p->flush_at) pl.trigger = p->flush_at;
    }
    pl.seed = p->perm_seed;
    pl.in_order = p->in_order;
  }
  // Rows shared by several workgroups keep their counters in the
  // workspace's fixed header, which has room for kMaxSplitRows of them.
  if (pl.segments > 1 && batch > kMaxSplitRows) {
    if (p && p->segments > 1) return DS_ERR_PLAN;
    pl.segments = 1;
  }
  if (pl.kernel == DS_KERNEL_CHUNK) {
    // The buffer's trigger: its capacity, or a requested flush point raised
    // to at least k plus one vector per lane.
    const int nt = pl.segments > 1 ? kChunkThreadsSplit : kChunkThreadsRow;
    pl.trigger = chunk_cap(pl.cls, nt);
    if (p && p->flush_at) {
      const int lo = k + chunk_room(nt);
      const int f = p->flush_at < lo ? lo : p->flush_at;
      pl.trigger = f < pl.trigger ? f : pl.trigger;
    }
  }
  *out = pl;
  return DS_OK;
}

size_t workspace_bytes_for(const Plan& pl, int64_t batch, int32_t k) {
  if (pl.segments <= 1 || batch <= 0) return 0;
  if (pl.kernel == DS_KERNEL_CHUNK) return chunk_ws_layout(batch, pl.segments, k).total;
  return ws_layout(batch, pl.segments, k).total;
}

ds_status_t check_scalars(ds_dtype_t dtype, int64_t batch, int64_t n_cols, int64_t row_stride,
                          int32_t k, int32_t sorted, ds_index_dtype_t index_dtype) {
  if (dtype != DS_FP32 && dtype != DS_BF16) return DS_ERR_DTYPE;
  if (index_dtype != DS_INT32 && index_dtype != DS_INT64) return DS_ERR_INDEX_DTYPE;
  if (sorted < 0 || sorted > 2) return DS_ERR_SORTED_MODE;
  if (k < 1 || k > DS_TOPK_MAX_K) return DS_ERR_K_RANGE;
  if (batch < 0 || batch > INT32_MAX || n_cols < 0 || n_cols > INT32_MAX || row_stride < n_cols)
    return DS_ERR_SHAPE;
  if (batch > 0 && row_stride > (INT64_MAX / 8) / batch) return DS_ERR_SHAPE;
  return DS_OK;
}

ds_status_t validate(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                     int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                     int32_t return_values, ds_index_dtype_t index_dtype, const void* values,
                     const void* indices, const int32_t* row_status, const void* workspace,
                     size_t workspace_bytes, const ds_topk_plan_t* plan, Plan* pl) {
  ds_status_t st = check_scalars(dtype, batch, n_cols, row_stride, k, sorted, index_dtype);
  if (st != DS_OK) return st;
  st = resolve_plan(batch, n_cols, k, dtype, plan, pl);
  if (st != DS_OK) return st;
  if (batch == 0) return DS_OK;
  if (!indices || !row_status || (return_values && !values) || (n_cols > 0 && !x))
    return DS_ERR_NULL;
  const int es = elem_size(dtype);
  if ((x && misaligned(x, 16)) || (row_stride * es) % 16 != 0) return DS_ERR_ALIGN;
  if (misaligned(indices, index_dtype == DS_INT64 ? 8 : 4)) return DS_ERR_ALIGN;
  if (return_values && misaligned(values, static_cast<uintptr_t>(es))) return DS_ERR_ALIGN;
  if (misaligned(row_status, 4) || (end && misaligned(end, 4))) return DS_ERR_ALIGN;
  if (plan && plan->stats && misaligned(plan->stats, 4)) return DS_ERR_ALIGN;
  if (batch * static_cast<int64_t>(pl->segments) > INT32_MAX) return DS_ERR_SHAPE;
  const size_t need = workspace_bytes_for(*pl, batch, k);
  if (need > 0 && (!workspace || workspace_bytes < need || misaligned(workspace, 16)))
    return DS_ERR_WORKSPACE;
  return DS_OK;
}

}  // namespace

namespace dstk {

// The workspace starts with a header of per-row counters at fixed offsets,
// the same for every (batch, segments, k) and both kernels: the only words
// that must be zero when a call starts, and every call leaves them zero.
// Everything after it is written before it is read within a call, so calls
// with different layouts can share one workspace without clearing it.
//   [0, 8R)    u64 shared threshold per row (stream kernel)
//   [8R, 16R)  u64 largest estimated start per row (stream kernel)
//   [16R, 20R) u32 arrival count per row (both kernels)
//   [20R, 24R) u32 status OR per row (stream kernel)
//   [24R, 28R) u32 fill cursor per row (stream kernel)
// with R = kMaxSplitRows.
namespace {
constexpr size_t kR = static_cast<size_t>(kMaxSplitRows);
static_assert(28 * kR <= kWsHeaderBytes, "the header holds every counter");
}  // namespace

WsLayout ws_layout(int64_t batch, int segments, int k) {
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  WsLayout l{};
  const size_t b = static_cast<size_t>(batch);
  const size_t s = static_cast<size_t>(segments);
  l.thr = 0;
  l.spec = 8 * kR;
  l.done = 16 * kR;
  l.flags = 20 * kR;
  l.fill = 24 * kR;
  l.x = kWsHeaderBytes;
  l.comp = up(l.x + b * s * 8);
  l.total = up(l.comp + b * s * (static_cast<size_t>(k) + kStreamSlotSlack) * 8);
  return l;
}

ChunkWs chunk_ws_layout(int64_t batch, int segments, int k) {
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  ChunkWs l{};
  const size_t b = static_cast<size_t>(batch);
  const size_t s = static_cast<size_t>(segments);
  l.arrive = 16 * kR;
  l.rec = kWsHeaderBytes;
  l.slot = up(l.rec + b * s * 16);
  l.total = up(l.slot + b * s * static_cast<size_t>(k) * 8);
  return l;
}

}  // namespace dstk

extern "C" {

ds_status_t ds_topk_validate(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                             int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                             int32_t return_values, ds_index_dtype_t index_dtype,
                             const void* values, const void* indices, const int32_t* row_status,
                             const void* workspace, size_t workspace_bytes,
                             const ds_topk_plan_t* plan) {
  Plan pl;
  return validate(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                  index_dtype, values, indices, row_status, workspace, workspace_bytes, plan,
                  &pl);
}

ds_status_t ds_topk_ex(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                       int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                       int32_t return_values, ds_index_dtype_t index_dtype, void* values,
                       void* indices, int32_t* row_status, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, const ds_topk_plan_t* plan) {
  Plan pl;
  ds_status_t st = validate(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                            index_dtype, values, indices, row_status, workspace,
                            workspace_bytes, plan, &pl);
  if (st != DS_OK || batch == 0) return st;

  if (pl.kernel == DS_KERNEL_CHUNK) {
    CArgs c{};
    c.x = x;
    c.row_stride = row_stride;
    c.n_cols = static_cast<int32_t>(n_cols);
    c.batch = static_cast<int32_t>(batch);
    c.end = end;
    c.k = k;
    c.sorted = sorted;
    c.return_values = return_values ? 1 : 0;
    c.idx64 = index_dtype == DS_INT64 ? 1 : 0;
    c.values = return_values ? values : nullptr;
    c.indices = indices;
    c.row_status = row_status;
    c.segments = pl.segments;
    c.perm_seed = pl.seed;
    c.in_order = pl.in_order;
    // Rows of a causal prefill grow with the row index: whole rows go
    // longest-first when their lengths vary.
    c.reverse_rows = (pl.segments == 1 && end != nullptr) ? 1 : 0;
    c.cap_eff = static_cast<uint32_t>(pl.trigger);
    c.stats = plan ? plan->stats : nullptr;
    if (pl.segments > 1) {
      const ChunkWs l = chunk_ws_layout(batch, pl.segments, k);
      char* w = static_cast<char*>(workspace);
      c.ws_arrive = reinterpret_cast<uint32_t*>(w + l.arrive);
      c.ws_rec = reinterpret_cast<unsigned long long*>(w + l.rec);
      c.ws_slot = reinterpret_cast<unsigned long long*>(w + l.slot);
    }
    const int dt = dtype == DS_BF16 ? 1 : 0;
    const int err = pl.segments > 1 ? launch_chunk_split(c, dt, pl.cls, stream)
                                    : launch_chunk_row(c, dt, pl.cls, stream);
    return err == 0 ? DS_OK : DS_ERR_HIP;
  }

  KArgs a{};
  a.x = x;
  a.row_stride = row_stride;
  a.n_cols = static_cast<int32_t>(n_cols);
  a.batch = static_cast<int32_t>(batch);
  a.end = end;
  a.k = k;
  a.sorted = sorted;
  a.return_values = return_values ? 1 : 0;
  a.idx64 = index_dtype == DS_INT64 ? 1 : 0;
  a.values = return_values ? values : nullptr;
  a.indices = indices;
  a.row_status = row_status;
  a.segments = pl.segments;
  a.perm_seed = pl.seed;
  a.in_order = pl.in_order;
  a.trigger = pl.trigger;
  a.stats = plan ? plan->stats : nullptr;
  if (pl.segments > 1) {
    const WsLayout l = ws_layout(batch, pl.segments, k);
    char* w = static_cast<char*>(workspace);
    a.ws_thr = reinterpret_cast<unsigned long long*>(w + l.thr);
    a.ws_done = reinterpret_cast<uint32_t*>(w + l.done);
    a.ws_flags = reinterpret_cast<uint32_t*>(w + l.flags);
    a.ws_fill = reinterpret_cast<uint32_t*>(w + l.fill);
    a.ws_x = reinterpret_cast<unsigned long long*>(w + l.x);
    a.ws_spec = reinterpret_cast<unsigned long long*>(w + l.spec);
    a.ws_comp = reinterpret_cast<unsigned long long*>(w + l.comp);
  }
  const int err = launch_topk(a, dtype == DS_BF16 ? 1 : 0, pl.cls, stream);
  return err == 0 ? DS_OK : DS_ERR_HIP;
}

ds_status_t ds_topk(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                    int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                    int32_t return_values, ds_index_dtype_t index_dtype, void* values,
                    void* indices, int32_t* row_status, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return ds_topk_ex(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                    index_dtype, values, indices, row_status, workspace, workspace_bytes, stream,
                    nullptr);
}

size_t ds_topk_workspace_size_ex(ds_dtype_t dtype, int64_t batch, int64_t n_cols, int32_t k,
                                 const ds_topk_plan_t* plan) {
  if (check_scalars(dtype, batch, n_cols, n_cols, k, 1, DS_INT32) != DS_OK) return 0;
  Plan pl;
  if (resolve_plan(batch, n_cols, k, dtype, plan, &pl) != DS_OK) return 0;
  return workspace_bytes_for(pl, batch, k);
}

size_t ds_topk_workspace_size(ds_dtype_t dtype, int64_t batch, int64_t n_cols, int32_t k) {
  return ds_topk_workspace_size_ex(dtype, batch, n_cols, k, nullptr);
}

ds_status_t ds_read_ceiling(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                            int64_t row_stride, const int32_t* end, int32_t k,
                            const ds_topk_plan_t* plan, uint32_t* sink, hipStream_t stream) {
  ds_status_t st = check_scalars(dtype, batch, n_cols, row_stride, k, 1, DS_INT32);
  if (st != DS_OK) return st;
  Plan pl;
  st = resolve_plan(batch, n_cols, k, dtype, plan, &pl);
  if (st != DS_OK || batch == 0) return st;
  if (!sink || (n_cols > 0 && !x)) return DS_ERR_NULL;
  if ((x && misaligned(x, 16)) || (row_stride * elem_size(dtype)) % 16 != 0) return DS_ERR_ALIGN;
  if (misaligned(sink, 4) || (end && misaligned(end, 4))) return DS_ERR_ALIGN;
  if (batch * static_cast<int64_t>(pl.segments) > INT32_MAX) return DS_ERR_SHAPE;
  if (pl.kernel == DS_KERNEL_CHUNK) {
    CArgs c{};
    c.x = x;
    c.row_stride = row_stride;
    c.n_cols = static_cast<int32_t>(n_cols);
    c.batch = static_cast<int32_t>(batch);
    c.end = end;
    c.k = k;
    c.segments = pl.segments;
    c.perm_seed = pl.seed;
    c.in_order = pl.in_order;
    c.reverse_rows = (pl.segments == 1 && end != nullptr) ? 1 : 0;
    const int dt = dtype == DS_BF16 ? 1 : 0;
    const int err = pl.segments > 1 ? launch_chunk_read_split(c, dt, sink, stream)
                                    : launch_chunk_read_row(c, dt, sink, stream);
    return err == 0 ? DS_OK : DS_ERR_HIP;
  }
  KArgs a{};
  a.x = x;
  a.row_stride = row_stride;
  a.n_cols = static_cast<int32_t>(n_cols);
  a.batch = static_cast<int32_t>(batch);
  a.end = end;
  a.k = k;
  a.segments = pl.segments;
  a.perm_seed = pl.seed;
  a.in_order = pl.in_order;
  a.trigger = pl.trigger;
  const int err = launch_read(a, dtype == DS_BF16 ? 1 : 0, pl.cls, sink, stream);
  return err == 0 ? DS_OK : DS_ERR_HIP;
}

int64_t ds_topk_stride_requirement(ds_dtype_t dtype) {
  if (dtype == DS_FP32) return 4;
  if (dtype == DS_BF16) return 8;
  return 0;
}

const char* ds_topk_status_string(ds_status_t status) {
  switch (status) {
    case DS_OK: return "ok";
    case DS_ERR_NULL: return "a required pointer is NULL";
    case DS_ERR_DTYPE: return "unsupported input dtype (fp32 or bf16)";
    case DS_ERR_INDEX_DTYPE: return "unsupported index dtype (int32 or int64)";
    case DS_ERR_K_RANGE: return "k must be in 1..4096";
    case DS_ERR_SHAPE: return "invalid shape (batch, n_cols, row_stride)";
    case DS_ERR_ALIGN: return "misaligned pointer or row stride (16-byte rows required)";
    case DS_ERR_SORTED_MODE: return "sorted must be 0 (unsorted), 1 (by value) or 2 (by index)";
    case DS_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case DS_ERR_HIP: return "HIP launch error";
    case DS_ERR_PLAN: return "plan field out of range";
    case DS_ERR_SCRATCH_LIMIT: return "problem needs more workspace than the allocation-free entry point's scratch";
    case DS_ERR_SAMPLER_PARAM: return "temperature is NaN, or top_p is NaN or not above zero";
  }
  return "unknown status";
}

}  // extern "C"
