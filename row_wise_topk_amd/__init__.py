"""row_wise_topk_amd -- row-wise TopK on AMD MI355X (gfx950).

A thin ctypes binding over ``libdstopk.so``, whose C ABI is declared in
``include/ds_topk.h``.  Every step of the selection runs in the library's HIP
kernels; this module only marshals arguments.  PyTorch supplies device memory
and the current stream.

Raw entry points carry the C names and arguments (``ds_topk``, ``ds_topk_ex``,
``ds_topk_validate``, ``ds_topk_workspace_size``, ``ds_topk_workspace_size_ex``,
``ds_topk_stride_requirement``, ``ds_topk_status_string``, the allocation-free
``ds_topk_noalloc``, the sampling step ``ds_sampler_tail`` and the measurement
aid ``ds_read_ceiling``).  :func:`topk` is the
tensor-level call, the counterpart of ``deep_select.topk(x, topk, sorted_index,
indices_type, return_value)`` described on xhh.club, "DeepSeek开源DeepSelect：
比torch.topk快二十倍！" (Q&A), with a per-row ``end`` as described on
aifluxnews.com, "DeepSeek 在 GitHub 发布 DeepSelect v1.0.0" (section
"PyTorch 接口与 CUDA 环境要求").

The library must be built (``python -m row_wise_topk_amd.build`` or
``__graft_entry__.build()``); importing without it raises ImportError.  There
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch  # loads the HIP runtime that libdstopk.so then shares

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdstopk.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "ds_topk.h")

DS_FP32, DS_BF16 = 0, 1
DS_INT32, DS_INT64 = 0, 1
DS_UNSORTED, DS_SORTED_VALUE, DS_SORTED_INDEX = 0, 1, 2
DS_OK = 0
DS_ROW_NAN, DS_ROW_BAD_END, DS_ROW_INTERNAL = 1, 2, 4
DS_KERNEL_AUTO, DS_KERNEL_STREAM, DS_KERNEL_CHUNK = 0, 1, 2
DS_TOPK_MAX_K = 4096
STATUS_NAMES = ["DS_OK", "DS_ERR_NULL", "DS_ERR_DTYPE", "DS_ERR_INDEX_DTYPE", "DS_ERR_K_RANGE",
                "DS_ERR_SHAPE", "DS_ERR_ALIGN", "DS_ERR_SORTED_MODE", "DS_ERR_WORKSPACE",
                "DS_ERR_HIP", "DS_ERR_PLAN", "DS_ERR_SCRATCH_LIMIT", "DS_ERR_SAMPLER_PARAM"]
DS_ERR_SCRATCH_LIMIT = 11
DS_ERR_SAMPLER_PARAM = 12
DS_TOPK_NOALLOC_SCRATCH_BYTES = 16 << 20
DS_TOPK_WS_HEADER_BYTES = 256 << 10
DS_STAT_ROW_REREADS, DS_STAT_CHUNK_REREADS, DS_STAT_CUTS, DS_STAT_FINAL_CANDIDATES = 0, 1, 2, 3
DS_TOPK_MAX_SPLIT_ROWS = 8192


class Plan(ctypes.Structure):
    """ds_topk_plan_t: segments, perm_seed, in_order, flush_at, kernel (0 =
    automatic), stats (device pointer to uint32 [batch * 4] or None)."""
    _fields_ = [("segments", ctypes.c_int32), ("perm_seed", ctypes.c_uint32),
                ("in_order", ctypes.c_int32), ("flush_at", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("stats", ctypes.c_void_p)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m row_wise_topk_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _i64, _u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_TOPK_ARGS = [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _i32, _i32, ctypes.c_int, _vp,
              _vp, _vp, _vp, _u64, _vp]
_lib.ds_topk.argtypes = _TOPK_ARGS
_lib.ds_topk.restype = ctypes.c_int
_lib.ds_topk_ex.argtypes = _TOPK_ARGS + [ctypes.POINTER(Plan)]
_lib.ds_topk_ex.restype = ctypes.c_int
_lib.ds_topk_validate.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _i32, _i32,
                                  ctypes.c_int, _vp, _vp, _vp, _vp, _u64, ctypes.POINTER(Plan)]
_lib.ds_topk_validate.restype = ctypes.c_int
_lib.ds_topk_workspace_size.argtypes = [ctypes.c_int, _i64, _i64, _i32]
_lib.ds_topk_workspace_size.restype = ctypes.c_size_t
_lib.ds_topk_workspace_size_ex.argtypes = [ctypes.c_int, _i64, _i64, _i32, ctypes.POINTER(Plan)]
_lib.ds_topk_workspace_size_ex.restype = ctypes.c_size_t
_lib.ds_topk_stride_requirement.argtypes = [ctypes.c_int]
_lib.ds_topk_stride_requirement.restype = ctypes.c_int64
_lib.ds_topk_status_string.argtypes = [ctypes.c_int]
_lib.ds_topk_status_string.restype = ctypes.c_char_p
_lib.ds_read_ceiling.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32,
                                ctypes.POINTER(Plan), _vp, _vp]
_lib.ds_read_ceiling.restype = ctypes.c_int
_lib.ds_topk_noalloc.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _i32, _i32,
                                 ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.POINTER(Plan)]
_lib.ds_topk_noalloc.restype = ctypes.c_int
_lib.ds_sampler_tail.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _i64, _i32,
                                 ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, _vp]
_lib.ds_sampler_tail.restype = ctypes.c_int


def exported_names() -> list[str]:
    """Function names declared in include/ds_topk.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(ds_\w+)\s*\(", text, re.M)))


def _plan_ptr(plan):
    if plan is None:
        return None
    if isinstance(plan, Plan):
        return ctypes.pointer(plan)
    p = Plan(int(plan.get("segments", 0)), int(plan.get("perm_seed", 0x5EED)) & 0xFFFFFFFF,
             int(plan.get("in_order", 0)), int(plan.get("flush_at", 0)),
             int(plan.get("kernel", 0)), plan.get("stats"))
    return ctypes.pointer(p)


# ---------------------------------------------------------------- raw C entry points
def ds_topk(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values, index_dtype,
            values, indices, row_status, workspace, workspace_bytes, stream) -> int:
    return _lib.ds_topk(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                        index_dtype, values, indices, row_status, workspace, workspace_bytes,
                        stream)


def ds_topk_ex(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values, index_dtype,
               values, indices, row_status, workspace, workspace_bytes, stream, plan) -> int:
    return _lib.ds_topk_ex(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                           index_dtype, values, indices, row_status, workspace, workspace_bytes,
                           stream, _plan_ptr(plan))


def ds_topk_noalloc(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                    index_dtype, values, indices, row_status, stream, plan=None) -> int:
    return _lib.ds_topk_noalloc(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                                index_dtype, values, indices, row_status, stream, _plan_ptr(plan))


def ds_topk_validate(x, dtype, batch, n_cols, row_stride, end, k, sorted, return_values,
                     index_dtype, values, indices, row_status, workspace, workspace_bytes,
                     plan=None) -> int:
    return _lib.ds_topk_validate(x, dtype, batch, n_cols, row_stride, end, k, sorted,
                                 return_values, index_dtype, values, indices, row_status,
                                 workspace, workspace_bytes, _plan_ptr(plan))


def ds_topk_workspace_size(dtype, batch, n_cols, k) -> int:
    return _lib.ds_topk_workspace_size(dtype, batch, n_cols, k)


def ds_topk_workspace_size_ex(dtype, batch, n_cols, k, plan=None) -> int:
    return _lib.ds_topk_workspace_size_ex(dtype, batch, n_cols, k, _plan_ptr(plan))


def ds_topk_stride_requirement(dtype) -> int:
    return _lib.ds_topk_stride_requirement(dtype)


def ds_topk_status_string(status) -> str:
    return _lib.ds_topk_status_string(status).decode()


def ds_read_ceiling(x, dtype, batch, n_cols, row_stride, end, k, plan, sink, stream) -> int:
    return _lib.ds_read_ceiling(x, dtype, batch, n_cols, row_stride, end, k, _plan_ptr(plan),
                                sink, stream)


def ds_sampler_tail(values, dtype, indices, index_dtype, row_status, batch, k, temperature,
                    top_p, uniforms, tokens, probs, stream) -> int:
    return _lib.ds_sampler_tail(values, dtype, indices, index_dtype, row_status, batch, k,
                                temperature, top_p, uniforms, tokens, probs, stream)


# ---------------------------------------------------------------- tensor-level call
class TopkError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {ds_topk_status_string(status)}")


_workspaces: dict = {}


def workspace_for(device: torch.device, stream_ptr: int, nbytes: int) -> torch.Tensor:
    """A device buffer of at least ``nbytes`` for calls on one stream, zeroed
    when allocated.

    Every call leaves the workspace's counter header zero again (the rest is
    scratch), so one buffer serves all calls that are ordered on the same
    stream.
    """
    key = (device.index, stream_ptr)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


_DT = {torch.float32: DS_FP32, torch.bfloat16: DS_BF16}
_IT = {torch.int32: DS_INT32, torch.int64: DS_INT64}


def _check_out(values, indices, status, batch, k, dtype, index_dtype, return_values, dev):
    """Caller-supplied outputs must be exactly what the kernel writes: dense
    [batch, k] of the right dtypes (values only with return_values) and an
    int32 [batch] status, all contiguous on x's device."""
    want = [("indices", indices, index_dtype, (batch, k)), ("row_status", status, torch.int32, (batch,))]
    if return_values:
        want.append(("values", values, dtype, (batch, k)))
    for name, t, dt, shape in want:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"out: {name} must be a tensor")
        if t.dtype != dt or tuple(t.shape) != shape or t.device != dev or not t.is_contiguous():
            raise ValueError(f"out: {name} must be a contiguous {dt} tensor of shape {shape} "
                             f"on {dev} (got {t.dtype} {tuple(t.shape)} on {t.device})")


def topk(x: torch.Tensor, k: int, *, end: torch.Tensor | None = None, sorted: int = 1,
         return_values: bool = True, index_dtype: torch.dtype = torch.int32,
         n_cols: int | None = None, plan=None, out=None):
    """Top-k of every row of a 2-D fp32 / bf16 CUDA tensor.

    ``sorted``: 1 (or True) by value, larger first, ties by lower index;
    2 by index; 0 (or False) unsorted.  ``end`` (int32, [batch]) gives each row
    its own length.  Returns ``(values or None, indices, row_status)``.
    """
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D CUDA tensor")
    if x.dtype not in _DT:
        raise TypeError("x must be float32 or bfloat16")
    if index_dtype not in _IT:
        raise TypeError("index_dtype must be torch.int32 or torch.int64")
    batch = x.shape[0]
    n_cols = x.shape[1] if n_cols is None else int(n_cols)
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("the last dimension must be contiguous")
    row_stride = x.stride(0) if batch > 1 else max(x.stride(0), x.shape[1])
    esz = x.element_size()
    avail = x.untyped_storage().nbytes() - x.storage_offset() * esz
    if batch and avail < batch * row_stride * esz:
        raise ValueError("x's storage must span batch * row_stride elements (pad the last row)")
    dev = x.device
    if end is not None:
        if end.dtype != torch.int32 or end.device != dev or end.shape != (batch,):
            raise ValueError("end must be an int32 tensor of shape [batch] on x's device")
        end = end.contiguous()
    sorted_i = int(sorted)
    if out is None:
        values = torch.empty((batch, k), dtype=x.dtype, device=dev) if return_values else None
        indices = torch.empty((batch, k), dtype=index_dtype, device=dev)
        status = torch.empty((batch,), dtype=torch.int32, device=dev)
    else:
        values, indices, status = out
        _check_out(values, indices, status, batch, k, x.dtype, index_dtype, return_values, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    dt = _DT[x.dtype]
    ws_bytes = ds_topk_workspace_size_ex(dt, batch, n_cols, k, plan)
    ws = workspace_for(dev, stream, ws_bytes) if ws_bytes else None
    rc = ds_topk_ex(x.data_ptr(), dt, batch, n_cols, row_stride,
                    end.data_ptr() if end is not None else None, int(k), sorted_i,
                    int(bool(return_values)), _IT[index_dtype],
                    values.data_ptr() if values is not None else None, indices.data_ptr(),
                    status.data_ptr(), ws.data_ptr() if ws is not None else None,
                    ws.numel() if ws is not None else 0, stream, plan)
    if rc != DS_OK:
        raise TopkError(rc)
    return values, indices, status


def read_ceiling(x: torch.Tensor, k: int, *, end: torch.Tensor | None = None,
                 n_cols: int | None = None, plan=None, sink: torch.Tensor | None = None) -> None:
    """Queue the read-ceiling kernel on the current stream: the bytes
    :func:`topk` would read for the same arguments, read the same way, and
    nothing else (a measurement aid; see ``ds_read_ceiling``)."""
    if x.dim() != 2 or not x.is_cuda or x.dtype not in _DT:
        raise ValueError("x must be a 2-D float32 / bfloat16 CUDA tensor")
    batch = x.shape[0]
    n_cols = x.shape[1] if n_cols is None else int(n_cols)
    row_stride = x.stride(0) if batch > 1 else max(x.stride(0), x.shape[1])
    if sink is None:
        sink = torch.empty((1,), dtype=torch.int32, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = ds_read_ceiling(x.data_ptr(), _DT[x.dtype], batch, n_cols, row_stride,
                         end.data_ptr() if end is not None else None, int(k), plan,
                         sink.data_ptr(), stream)
    if rc != DS_OK:
        raise TopkError(rc)


def sample_from_topk(values: torch.Tensor, indices: torch.Tensor, row_status=None, *,
                     temperature: float, top_p: float, uniforms: torch.Tensor):
    """The sampling step after :func:`topk` (sorted by value): temperature
    softmax over each row's candidates, nucleus cut at ``top_p``, inverse-CDF
    draw with the row's ``uniforms`` entry (see ``ds_sampler_tail``).  Returns
    ``(tokens int64 [batch], probs float32 [batch])``; a row that draws
    nothing gets token -1."""
    if values.dim() != 2 or values.shape != indices.shape or not values.is_cuda:
        raise ValueError("values and indices must be CUDA tensors of one shape [batch, k]")
    if values.dtype not in _DT or indices.dtype not in _IT:
        raise TypeError("values must be float32 / bfloat16 and indices int32 / int64")
    batch, k = values.shape
    dev = values.device
    for name, t in (("values", values), ("indices", indices)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if uniforms.dtype != torch.float32 or uniforms.shape != (batch,) or uniforms.device != dev:
        raise ValueError("uniforms must be a float32 tensor of shape [batch] on values' device")
    if row_status is not None and (row_status.dtype != torch.int32 or row_status.shape != (batch,)
                                   or row_status.device != dev):
        raise ValueError("row_status must be an int32 tensor of shape [batch] on values' device")
    uniforms = uniforms.contiguous()
    tokens = torch.empty((batch,), dtype=torch.int64, device=dev)
    probs = torch.empty((batch,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = ds_sampler_tail(values.data_ptr(), _DT[values.dtype], indices.data_ptr(), _IT[indices.dtype],
                         row_status.contiguous().data_ptr() if row_status is not None else None,
                         batch, k, float(temperature), float(top_p), uniforms.data_ptr(),
                         tokens.data_ptr(), probs.data_ptr(), stream)
    if rc != DS_OK:
        raise TopkError(rc)
    return tokens, probs


def pad_rows(x: torch.Tensor) -> torch.Tensor:
    """Copy ``x`` into a buffer whose row stride meets the 16-byte requirement
    (the padding the pages ask callers to do for unaligned rows); the returned
    view has ``x``'s shape."""
    req = ds_topk_stride_requirement(_DT[x.dtype])
    n = x.shape[1]
    stride = (n + req - 1) // req * req
    buf = torch.empty((x.shape[0], stride), dtype=x.dtype, device=x.device)
    buf[:, :n].copy_(x)
    return buf[:, :n]
