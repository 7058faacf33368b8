// ds_topk_noalloc: ds_topk_ex with the library's own scratch memory, for
// callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array of DS_TOPK_NOALLOC_SCRATCH_BYTES.
// Every GPU the library runs on holds its own copy of it, at its own address,
// until the process ends.  In host code the array's name only stands in for
// the symbol: its device address comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call that needs scratch,
// and only that address is ever handed to a kernel.  The same first call
// clears the array with a kernel on the caller's stream, so the workspace is
// zero before its first use; every call then leaves it zero again, as
// ds_topk_ex does with a caller's workspace.  All calls on one GPU share the
// array: calls that may overlap on one GPU (different streams without
// ordering between them) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ds_topk.h"

namespace {

constexpr size_t kScratchBytes = DS_TOPK_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size is a whole number of 256-B lines");

__device__ __align__(256) unsigned long long scratch[kScratchBytes / 8];

__global__ __launch_bounds__(256) void clear_scratch(unsigned long long* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = 0ull;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` per device, once set up

// The current device's scratch address, set up on first use; nullptr with
// *st set on a HIP error.
void* scratch_for_current_device(hipStream_t stream, ds_status_t* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = DS_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev]) return g_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    *st = DS_ERR_HIP;
    return nullptr;
  }
  unsigned long long* p64 = static_cast<unsigned long long*>(ptr);
  size_t n = kScratchBytes / 8;
  void* args[] = {&p64, &n};
  // The launch's own error code (an earlier error of the thread is left alone).
  if (hipLaunchKernel(reinterpret_cast<const void*>(&clear_scratch), dim3(1024), dim3(256), args, 0,
                      stream) != hipSuccess) {
    *st = DS_ERR_HIP;
    return nullptr;
  }
  g_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" ds_status_t ds_topk_noalloc(const void* x, ds_dtype_t dtype, int64_t batch,
                                       int64_t n_cols, int64_t row_stride, const int32_t* end,
                                       int32_t k, int32_t sorted, int32_t return_values,
                                       ds_index_dtype_t index_dtype, void* values, void* indices,
                                       int32_t* row_status, hipStream_t stream,
                                       const ds_topk_plan_t* plan) {
  const size_t need = ds_topk_workspace_size_ex(dtype, batch, n_cols, k, plan);
  if (need > kScratchBytes) return DS_ERR_SCRATCH_LIMIT;
  // Argument errors come back before any HIP call: checked with a stand-in
  // workspace pointer (256-B aligned, never dereferenced by the checks).
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  ds_status_t st = ds_topk_validate(x, dtype, batch, n_cols, row_stride, end, k, sorted,
                                    return_values, index_dtype, values, indices, row_status,
                                    need ? stand_in : nullptr, need, plan);
  if (st != DS_OK || batch == 0) return st;
  void* ws = nullptr;
  if (need) {
    ws = scratch_for_current_device(stream, &st);
    if (!ws) return st;
  }
  return ds_topk_ex(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                    index_dtype, values, indices, row_status, ws, need, stream, plan);
}
