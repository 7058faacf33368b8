/*
 * ds_topk.h -- row-wise TopK on AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation and its options follow the public descriptions of DeepSelect:
 *   [NC] narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for sparse
 *        attention and sampling": the method paragraph (a monotone threshold T,
 *        rows read once in contiguous blocks of B visited in random order, a
 *        candidate buffer cut back to k by radix select when it reaches k+B2);
 *        the coverage paragraph (bf16 and fp32 inputs, k <= 4096, int32 or
 *        int64 indices); the install/API paragraph (rows contiguous in the last
 *        dimension, a stride requirement with padding for unaligned rows,
 *        sorted_index, return_value); the NaN paragraph (always checked).
 *   [AF] aifluxnews.com, "DeepSeek 在 GitHub 发布 DeepSelect v1.0.0", section
 *        "PyTorch 接口与 CUDA 环境要求": per-row `end` for variable-length rows,
 *        stride constraints on inputs and outputs.
 *   [XH] xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！", Q&A: the
 *        call topk(x, topk, sorted_index, indices_type, return_value); results
 *        are stable.
 *   [IT] deepseek-v4-pro.uk, "Inside DeepSeek V4.1's New Open Inference
 *        Toolkit", section "DeepSelect: a fast, deliberately narrow TopK": a
 *        NaN trap aborts the process, which a service has to isolate.
 *
 * Result of a row i (the same definition the method reaches exactly):
 *   L = end ? end[i] : n_cols; the row is x[i*row_stride + j], 0 <= j < L.
 *   Order: a precedes b iff x[a] > x[b], or x[a] == x[b] and a < b (numeric
 *   comparison: -0.0 == +0.0; -inf and +inf are ordinary values).
 *   The result is the first m = min(k, L) elements in that order.
 *
 * Conventions for every entry point:
 *   - All array pointers passed to ds_topk / ds_topk_ex are DEVICE pointers
 *     owned by the caller.  The library allocates no memory and keeps no
 *     state between calls (ds_topk_noalloc's static scratch array, one per
 *     device, is the one exception).
 *   - Calls are asynchronous on `stream`; the library never synchronises and
 *     never prints.  Argument errors are returned before anything is launched.
 *   - Data errors never abort (unlike the trap of [NC]/[IT]): they set bits in
 *     row_status[i] and that row's outputs become index -1, value qNaN.
 */
#ifndef DS_TOPK_H_
#define DS_TOPK_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input dtypes: fp32 (sampler path) and bf16 (Lightning Indexer path) [NC coverage]. */
typedef enum { DS_FP32 = 0, DS_BF16 = 1 } ds_dtype_t;

/* Index dtypes of the output [NC coverage; XH indices_type]. */
typedef enum { DS_INT32 = 0, DS_INT64 = 1 } ds_index_dtype_t;

/* Output order.  1 (also "true") = by value, larger first, then lower index;
 * 2 = by index ascending (the pages' sorted_index); 0 = unsorted: the m
 * results in an unspecified order [NC install/API]. */
typedef enum { DS_UNSORTED = 0, DS_SORTED_VALUE = 1, DS_SORTED_INDEX = 2 } ds_sorted_t;

typedef enum {
  DS_OK = 0,
  DS_ERR_NULL = 1,          /* a required pointer is NULL                          */
  DS_ERR_DTYPE = 2,         /* dtype is not DS_FP32 / DS_BF16                      */
  DS_ERR_INDEX_DTYPE = 3,   /* index_dtype is not DS_INT32 / DS_INT64              */
  DS_ERR_K_RANGE = 4,       /* k < 1 or k > DS_TOPK_MAX_K                          */
  DS_ERR_SHAPE = 5,         /* batch < 0, n_cols < 0, n_cols > INT32_MAX, row_stride < n_cols */
  DS_ERR_ALIGN = 6,         /* x not 16-B aligned, row_stride*elem not a multiple of 16 B,
                               or an output / end / row_status pointer misaligned   */
  DS_ERR_SORTED_MODE = 7,   /* sorted not in {0, 1, 2}                             */
  DS_ERR_WORKSPACE = 8,     /* workspace NULL, too small or not 16-B aligned       */
  DS_ERR_HIP = 9,           /* the HIP runtime reported an error at launch         */
  DS_ERR_PLAN = 10,         /* a ds_topk_plan_t field is out of range              */
  DS_ERR_SCRATCH_LIMIT = 11, /* ds_topk_noalloc: the problem needs more workspace than
                               DS_TOPK_NOALLOC_SCRATCH_BYTES                        */
  DS_ERR_SAMPLER_PARAM = 12 /* ds_sampler_tail: temperature is NaN, or top_p is NaN or <= 0 */
} ds_status_t;

#define DS_TOPK_MAX_K 4096            /* [NC coverage]: topk must be 4096 or less   */
#define DS_TOPK_WS_HEADER_BYTES (256u << 10) /* the workspace's counter header: 32 B for
                                               each of at most 8192 rows shared by
                                               several workgroups (DS_TOPK_MAX_SPLIT_ROWS) */
#define DS_TOPK_MAX_SPLIT_ROWS 8192   /* batch limit of a plan with segments > 1  */
#define DS_ROW_NAN 1                  /* row_status bit: a NaN in x[i, 0:L)          */
#define DS_ROW_BAD_END 2              /* row_status bit: end[i] < 0 or end[i] > n_cols */
#define DS_ROW_INTERNAL 4             /* row_status bit: a consistency check inside the
                                         kernel failed (never expected); the row is
                                         written as -1 / qNaN instead of looping on */

/*
 * ds_topk -- top-k of every row of a 2-D array [IT "DeepSelect" section; NC
 * method, coverage, install/API and NaN paragraphs; AF "PyTorch 接口" section].
 *
 *   x            device, row-major [batch, row_stride] of dtype; the last
 *                dimension is contiguous.  Base 16-B aligned and
 *                row_stride * sizeof(dtype) a multiple of 16 B (see
 *                ds_topk_stride_requirement); callers with other layouts pad.
 *                The allocation must span batch * row_stride elements: reads
 *                use 16-B vectors, and a vector that starts inside [0, L) may
 *                cover elements up to the next 16-B boundary (never past
 *                row_stride).  Elements at or past L are never used or checked.
 *   dtype        DS_FP32 or DS_BF16.
 *   batch        rows (>= 0; 0 launches nothing).
 *   n_cols       row length when `end` is NULL, and the upper bound of end[i].
 *   row_stride   elements between row starts (>= n_cols).
 *   end          device int32 [batch] or NULL: row i uses columns [0, end[i]).
 *   k            1..DS_TOPK_MAX_K; k > L is allowed (the tail is padded).
 *   sorted       ds_sorted_t.
 *   return_values  0: `values` is not written and may be NULL ([NC]: skipping
 *                the values output is faster).
 *   index_dtype  DS_INT32 or DS_INT64.
 *   values       device [batch, k] of dtype (dense, natural alignment): bit
 *                copies of the selected inputs; slots m..k-1 hold -inf.
 *   indices      device [batch, k] of index_dtype (dense, natural alignment):
 *                0-based columns; slots m..k-1 hold -1.
 *   row_status   device int32 [batch]: 0, or DS_ROW_NAN / DS_ROW_BAD_END, in
 *                which case the row's indices are -1 and values qNaN.
 *   workspace    device scratch of at least ds_topk_workspace_size(...)
 *                bytes, 16-B aligned, ZEROED before its first use.  Its first
 *                DS_TOPK_WS_HEADER_BYTES hold the per-row counters of rows
 *                shared by several workgroups; every call leaves them zero
 *                again.  The rest is scratch that every call writes before
 *                it reads, so any content is fine there.  May be NULL when
 *                that size is 0.  Calls that may overlap in time need
 *                distinct workspaces.
 *   stream       HIP stream the single kernel launch is queued on.
 * Returns DS_OK or the first argument error found (nothing launched), or
 * DS_ERR_HIP if the launch failed.
 */
ds_status_t ds_topk(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                    int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                    int32_t return_values, ds_index_dtype_t index_dtype, void* values,
                    void* indices, int32_t* row_status, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Launch plan.  Any plan gives bit-identical indices and values (for
 * DS_UNSORTED: the same set); the plan only changes speed.  ds_topk uses the
 * automatic plan.  [NC method]: blocks are visited in a random order and B,
 * B2 are tuning parameters.
 *   segments     workgroups that share one row (0 = automatic, else 1..256;
 *                above 1 needs batch <= DS_TOPK_MAX_SPLIT_ROWS).
 *                With the chunk kernels any value above 1 means one
 *                workgroup per chunk of the row (at most 256 chunks).
 *   perm_seed    seed of the per-row block permutation (any value).
 *   in_order     1 = visit blocks in address order instead.
 *   flush_at     candidate count that triggers a cut back to k (0 = automatic;
 *                else k+1 .. the buffer's fixed trigger for this k class; the
 *                chunk kernels raise it to at least k plus one vector per
 *                lane: k + 4096).
 *   kernel       DS_KERNEL_AUTO (0), DS_KERNEL_STREAM (1): one or more
 *                workgroups stream a row block by block (long rows), or
 *                DS_KERNEL_CHUNK (2): a 512-lane workgroup holds 64 KiB of a
 *                row in registers at a time; rows of up to 64 such chunks
 *                (1,048,576 fp32 or 2,097,152 bf16 values).
 *   stats        NULL, or a device uint32 array [batch * 4], 4-B aligned, to
 *                which the call ADDS per-row counts at [4 i + DS_STAT_*] (the
 *                caller zeroes it); results are unchanged.  A debug aid.
 */
typedef struct {
  int32_t segments;
  uint32_t perm_seed;
  int32_t in_order;
  int32_t flush_at;
  int32_t kernel;
  uint32_t* stats;
} ds_topk_plan_t;

/* Per-row statistics (plan.stats): the debug counters of the method's
 * data-dependent paths.  A re-read is the only extra input traffic the
 * method makes: a start estimated from part of a row that turns out too high
 * makes the row (or one chunk of a split row) be read again. */
#define DS_STAT_ROW_REREADS 0        /* whole-row re-reads                               */
#define DS_STAT_CHUNK_REREADS 1      /* chunks of a split row appended again from memory */
#define DS_STAT_CUTS 2               /* radix cuts back to k (streaming, merge, final)   */
#define DS_STAT_FINAL_CANDIDATES 3   /* candidates entering the row's final selection    */

#define DS_KERNEL_AUTO 0
#define DS_KERNEL_STREAM 1
#define DS_KERNEL_CHUNK 2

/* ds_topk with an explicit plan (plan may be NULL = automatic).  Same
 * arguments, ownership and errors as ds_topk, plus DS_ERR_PLAN. */
ds_status_t ds_topk_ex(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                       int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                       int32_t return_values, ds_index_dtype_t index_dtype, void* values,
                       void* indices, int32_t* row_status, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, const ds_topk_plan_t* plan);

/* The argument checks of ds_topk_ex alone: no HIP call, no launch, pointers
 * are only tested for NULL and alignment.  Returns what ds_topk_ex would
 * return before launching. */
ds_status_t ds_topk_validate(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                             int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                             int32_t return_values, ds_index_dtype_t index_dtype,
                             const void* values, const void* indices, const int32_t* row_status,
                             const void* workspace, size_t workspace_bytes,
                             const ds_topk_plan_t* plan);

/* Workspace bytes ds_topk needs for this problem (0 when one workgroup per
 * row suffices).  Host only; needs no GPU.  Invalid arguments give 0. */
size_t ds_topk_workspace_size(ds_dtype_t dtype, int64_t batch, int64_t n_cols, int32_t k);

/* Workspace bytes ds_topk_ex needs with `plan` (NULL = automatic).  Host
 * only: the automatic plan depends on the problem shape alone. */
size_t ds_topk_workspace_size_ex(ds_dtype_t dtype, int64_t batch, int64_t n_cols, int32_t k,
                                 const ds_topk_plan_t* plan);

/*
 * ds_topk_noalloc -- ds_topk_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, meaning, ownership and errors as
 * ds_topk_ex, without workspace / workspace_bytes: the workspace is a static
 * device array of DS_TOPK_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends.  The caller still passes x, end and the
 * outputs.  The call allocates nothing and calls no allocating routine; its
 * first call on a device that needs scratch takes the array's address on
 * that device (the device must be current) and clears it with one kernel on
 * `stream`, ahead of the selection.
 *   Returns DS_ERR_SCRATCH_LIMIT, before any HIP call, when
 *   ds_topk_workspace_size_ex(dtype, batch, n_cols, k, plan) exceeds
 *   DS_TOPK_NOALLOC_SCRATCH_BYTES (16 MiB: rows split over several
 *   workgroups, batch * segments * k * 8 bytes and a little more); DS_ERR_HIP
 *   if the address cannot be taken or the clearing kernel cannot be queued.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (streams with no ordering between them) race on it.  Calls
 *   ordered on one stream are safe; each leaves the array zero.
 */
#define DS_TOPK_NOALLOC_SCRATCH_BYTES (16u << 20)
ds_status_t ds_topk_noalloc(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                            int64_t row_stride, const int32_t* end, int32_t k, int32_t sorted,
                            int32_t return_values, ds_index_dtype_t index_dtype, void* values,
                            void* indices, int32_t* row_status, hipStream_t stream,
                            const ds_topk_plan_t* plan);

/* Row strides must be a multiple of this many elements (16 B / sizeof(dtype));
 * the counterpart of the pages' get_stride_requirement [NC install/API].
 * Returns 0 for an unknown dtype. */
int64_t ds_topk_stride_requirement(ds_dtype_t dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* ds_topk_status_string(ds_status_t status);

/*
 * Measurement aid, not part of the selection.  The pages rate a TopK by its
 * effective bandwidth, the input bytes it must read over its time [XH,
 * "torch.topk 的性能痛点"].  This call reads exactly the bytes ds_topk_ex
 * would read for the same arguments -- each valid element x[i, 0:L) once,
 * in the same blocks, block order, workgroups and 16-byte loads -- and does
 * nothing else, so its time is the read ceiling of that access pattern.
 *   x, dtype, batch, n_cols, row_stride, end, k, plan   as for ds_topk_ex
 *                (k and plan fix the workgroup layout only).
 *   sink         device pointer to one uint32_t, 4-B aligned; the kernel
 *                writes it only in the rare case that the folded data equals
 *                a fixed constant, so its content means nothing.
 *   stream       HIP stream the single kernel launch is queued on.
 * Returns DS_OK, the argument error ds_topk_ex would return for these
 * arguments (DS_ERR_NULL also for a NULL sink), or DS_ERR_HIP.
 */
ds_status_t ds_read_ceiling(const void* x, ds_dtype_t dtype, int64_t batch, int64_t n_cols,
                            int64_t row_stride, const int32_t* end, int32_t k,
                            const ds_topk_plan_t* plan, uint32_t* sink, hipStream_t stream);

/*
 * ds_sampler_tail -- the sampling step after the sampler's TopK, on its
 * output.  During sampling TopK selects the candidate tokens from a large
 * vocabulary [NC motive paragraph]; the generation settings around it include
 * a temperature and a top-p [IT, the recipe's generation settings].  Per row i
 * of the top-k output (candidates: the entries with index >= 0, sorted by
 * value, larger first, as ds_topk returns them with sorted = 1):
 *   w_j = exp((v_j - v_max) / temperature) (if v_max is infinite: 1 where
 *   v_j == v_max, else 0); c_j = w_0 + ... + w_j; S = the weights' total;
 *   K = min(1 + #{j : c_j < top_p * S}, number of candidates);
 *   token = indices[i][j*] with j* the first j < K such that
 *   c_j > u_i * c_{K-1}; its probability after the cut is w_j* / c_{K-1}.
 *   temperature <= 0 takes the first candidate (greedy, probability 1).
 * Computed in fp32 with a fixed summation order (the same draw on every call).
 *
 *   values       device [batch, k] of dtype (fp32 or bf16), sorted by value
 *                within each row.
 *   indices      device [batch, k] of index_dtype; negative entries are not
 *                candidates (ds_topk pads a row shorter than k with -1).
 *   row_status   device [batch] or NULL: a row with a non-zero status (a NaN
 *                row of ds_topk) draws nothing.
 *   batch, k     rows and candidates per row (1 <= k <= DS_TOPK_MAX_K).
 *   temperature  > 0: the softmax temperature; <= 0: greedy.
 *   top_p        the nucleus mass, > 0; 1 or more keeps every candidate.
 *   uniforms     device [batch] fp32: the row's uniform draw u in [0, 1)
 *                (clamped to [0, 1]; NaN counts as 0).  The caller owns the
 *                random numbers.
 *   tokens       device [batch] int64 out: the drawn index, or -1 for a row
 *                that draws nothing (a status bit set, or no candidate).
 *   probs        device [batch] fp32 out or NULL: the drawn token's
 *                probability after the nucleus cut (qNaN when none).
 *   stream       HIP stream the single launch is queued on.
 * Every pointer is caller-owned device memory, naturally aligned for its
 * element type.  Returns DS_OK, DS_ERR_DTYPE, DS_ERR_INDEX_DTYPE,
 * DS_ERR_K_RANGE, DS_ERR_SHAPE (batch < 0 or > INT32_MAX),
 * DS_ERR_SAMPLER_PARAM, DS_ERR_NULL, DS_ERR_ALIGN (checked in that order,
 * before any launch) or DS_ERR_HIP.  batch == 0 queues nothing.
 */
ds_status_t ds_sampler_tail(const void* values, ds_dtype_t dtype, const void* indices,
                            ds_index_dtype_t index_dtype, const int32_t* row_status,
                            int64_t batch, int32_t k, float temperature, float top_p,
                            const float* uniforms, int64_t* tokens, float* probs,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DS_TOPK_H_ */
