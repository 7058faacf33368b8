// The sampler tail after the sampler's TopK, for MI355X (gfx950, wave64).
//
// narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for sparse
// attention and sampling" (motive paragraph): during sampling, TopK selects
// the candidate tokens from a large vocabulary.  The generation settings
// that follow it include a temperature and a top-p (deepseek-v4-pro.uk,
// "Inside DeepSeek V4.1's New Open Inference Toolkit").  This kernel takes
// that next step on each row's top-k output, sorted by value (larger first):
//
//   weights   w_j = exp((v_j - v_max) / temperature) over the candidates
//             (index >= 0); if v_max is infinite, w_j = 1 where v_j == v_max,
//             else 0; temperature <= 0 draws the first candidate (greedy);
//   nucleus   c_j = w_0 + ... + w_j, S = the weights' total; keep the
//             K = 1 + #{j : c_j < top_p * S} first candidates (at most all);
//   draw      the first j < K with c_j > u * c_{K-1}, u the row's uniform
//             (clamped to [0, 1]); its index is the token, w_j / c_{K-1} its
//             probability.
//
// One 256-lane workgroup per row.  Lane t holds the contiguous candidates
// [t*per, (t+1)*per), per = ceil(k / 256) <= 16 (its slots i >= per hold no
// candidate and stand for no position), so the prefix sum is a
// sequential sum in the lane, then a wave scan and a scan over the four
// waves.  The work is a few microseconds of latency at the sampler's batch
// sizes, far from any roofline; it runs in fp32 with a fixed summation order,
// so a row's draw is the same on every call.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ds_topk.h"

namespace dstk {
namespace {

constexpr int kNT = 256;
constexpr int kNW = kNT / 64;
constexpr int kPer = DS_TOPK_MAX_K / kNT;

struct TailArgs {
  const void* values;
  const void* indices;
  const int32_t* row_status;   // nullable
  const float* uniforms;
  int64_t* tokens;
  float* probs;                // nullable
  int32_t k;
  int32_t bf16;
  int32_t idx64;
  float temperature;
  float top_p;
};

__device__ __forceinline__ float wave_incl_sum_f(float x) {
  const int lane = static_cast<int>(threadIdx.x & 63u);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, static_cast<unsigned>(d), 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
  return x;
}

__device__ __forceinline__ uint32_t wave_sum_u(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x += static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), d, 64));
  return x;
}

// Sum of a per-lane count over the workgroup (part: kNW slots of LDS used by
// this call only).
__device__ __forceinline__ uint32_t block_sum_u(uint32_t x, uint32_t* part) {
  x = wave_sum_u(x);
  if ((threadIdx.x & 63u) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int q = 0; q < kNW; ++q) s += part[q];
  return s;
}

__global__ __launch_bounds__(kNT) void sampler_tail_kernel(TailArgs a) {
  __shared__ float s_max[kNW];
  __shared__ float s_wsum[kNW];
  __shared__ uint32_t s_cnt[4][kNW];
  __shared__ float s_at[1];
  const int row = static_cast<int>(blockIdx.x);
  const int t = static_cast<int>(threadIdx.x);
  const int w = t >> 6;
  const int lane = t & 63;
  const int k = a.k;
  const int per = (k + kNT - 1) / kNT;
  const int j0 = t * per;
  const int64_t base = static_cast<int64_t>(row) * k;

  // The row's candidates: values as fp32 and indices (negative: padding).
  float v[kPer];
  int64_t ix[kPer];
  float mx = -INFINITY;
  uint32_t nc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + i;
    int64_t id = -1;
    float x = -INFINITY;
    if (i < per && j < k) {
      id = a.idx64 ? static_cast<const int64_t*>(a.indices)[base + j]
                   : static_cast<int64_t>(static_cast<const int32_t*>(a.indices)[base + j]);
      x = a.bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.values)[base + j]) << 16)
                 : static_cast<const float*>(a.values)[base + j];
    }
    ix[i] = id;
    v[i] = x;
    if (id >= 0) {
      mx = fmaxf(mx, x);
      ++nc;
    }
  }
  mx = wave_max_f(mx);
  if (lane == 0) s_max[w] = mx;
  const uint32_t m = block_sum_u(nc, s_cnt[0]);   // its barrier also publishes s_max
  float M = s_max[0];
#pragma unroll
  for (int q = 1; q < kNW; ++q) M = fmaxf(M, s_max[q]);

  const bool flagged = a.row_status != nullptr && a.row_status[row] != 0;
  if (flagged || m == 0u) {
    if (t == 0) {
      a.tokens[row] = -1;
      if (a.probs) a.probs[row] = __uint_as_float(0x7FC00000u);
    }
    return;
  }
  const float tau = a.temperature;
  if (!(tau > 0.0f)) {   // greedy: the first candidate (the padding comes last)
    if (t == 0) {
      a.tokens[row] = ix[0];
      if (a.probs) a.probs[row] = 1.0f;
    }
    return;
  }

  // Weights and their prefix sums: in the lane, then over the lanes.
  const bool inf_top = isinf(M);
  float c[kPer];
  float run = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    float wt = 0.0f;
    if (ix[i] >= 0) wt = inf_top ? (v[i] == M ? 1.0f : 0.0f) : expf((v[i] - M) / tau);
    v[i] = wt;
    run += wt;
    c[i] = run;
  }
  const float incl = wave_incl_sum_f(run);
  float excl = __shfl_up(incl, 1u, 64);
  if (lane == 0) excl = 0.0f;
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  float off = 0.0f, total = 0.0f;
#pragma unroll
  for (int q = 0; q < kNW; ++q) {
    off += q < w ? s_wsum[q] : 0.0f;
    total += s_wsum[q];
  }
  off += excl;
#pragma unroll
  for (int i = 0; i < kPer; ++i) c[i] = off + c[i];

  // S: the weights' total (the waves' sums in order; padding weighs 0).
  const float pS = a.top_p * total;
  uint32_t below = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) below += (ix[i] >= 0 && c[i] < pS) ? 1u : 0u;
  const uint32_t K = min(block_sum_u(below, s_cnt[1]) + 1u, m);

  // The draw: j* = #{j < K : c_j <= u * c_{K-1}}, at most K - 1.
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (i < per && j0 + i == static_cast<int>(K) - 1) s_at[0] = c[i];
  __syncthreads();
  const float CK = s_at[0];
  const float u = fminf(fmaxf(a.uniforms[row], 0.0f), 1.0f);
  const float target = u * CK;
  uint32_t le = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) le += (i < per && j0 + i < static_cast<int>(K) && c[i] <= target) ? 1u : 0u;
  const uint32_t js = min(block_sum_u(le, s_cnt[2]), K - 1u);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i < per && j0 + i == static_cast<int>(js)) {
      a.tokens[row] = ix[i];
      if (a.probs) a.probs[row] = v[i] / CK;
    }
  }
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

}  // namespace
}  // namespace dstk

extern "C" ds_status_t ds_sampler_tail(const void* values, ds_dtype_t dtype, const void* indices,
                                       ds_index_dtype_t index_dtype, const int32_t* row_status,
                                       int64_t batch, int32_t k, float temperature, float top_p,
                                       const float* uniforms, int64_t* tokens, float* probs,
                                       hipStream_t stream) {
  using namespace dstk;
  if (dtype != DS_FP32 && dtype != DS_BF16) return DS_ERR_DTYPE;
  if (index_dtype != DS_INT32 && index_dtype != DS_INT64) return DS_ERR_INDEX_DTYPE;
  if (k < 1 || k > DS_TOPK_MAX_K) return DS_ERR_K_RANGE;
  if (batch < 0 || batch > INT32_MAX) return DS_ERR_SHAPE;
  if (isnan(temperature) || isnan(top_p) || !(top_p > 0.0f)) return DS_ERR_SAMPLER_PARAM;
  if (batch == 0) return DS_OK;
  if (!values || !indices || !uniforms || !tokens) return DS_ERR_NULL;
  if (misaligned(values, dtype == DS_BF16 ? 2 : 4) || misaligned(indices, index_dtype == DS_INT64 ? 8 : 4) ||
      misaligned(uniforms, 4) || misaligned(tokens, 8) || (probs && misaligned(probs, 4)) ||
      (row_status && misaligned(row_status, 4)))
    return DS_ERR_ALIGN;
  TailArgs a{};
  a.values = values;
  a.indices = indices;
  a.row_status = row_status;
  a.uniforms = uniforms;
  a.tokens = tokens;
  a.probs = probs;
  a.k = k;
  a.bf16 = dtype == DS_BF16 ? 1 : 0;
  a.idx64 = index_dtype == DS_INT64 ? 1 : 0;
  a.temperature = temperature;
  a.top_p = top_p;
  void* args[] = {&a};
  // The launch's own error code (an earlier error of the thread is left alone).
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sampler_tail_kernel),
                                       dim3(static_cast<uint32_t>(batch)), dim3(kNT), args, 0, stream);
  return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}
