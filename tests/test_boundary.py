"""The C-ABI boundary on the CPU: the library loads, exports every function the
header declares, and its host-side checks return the documented codes.  No
compute call is made (nothing here needs a GPU)."""
from __future__ import annotations

import ctypes

import pytest

from tests.build_util import ensure_built

ensure_built()
import row_wise_topk_amd as rt  # noqa: E402

A16 = 0x100000      # fake, 16-byte aligned device addresses (never dereferenced)
A16b = 0x200000
A16c = 0x300000
A16d = 0x400000
A16w = 0x500000


def test_every_declared_symbol_is_exported():
    names = rt.exported_names()
    assert {"ds_topk", "ds_topk_ex", "ds_topk_validate", "ds_topk_workspace_size",
            "ds_topk_workspace_size_ex", "ds_topk_stride_requirement",
            "ds_topk_status_string", "ds_read_ceiling", "ds_sampler_tail"} <= set(names)
    lib = ctypes.CDLL(rt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_stride_requirement():
    assert rt.ds_topk_stride_requirement(rt.DS_FP32) == 4
    assert rt.ds_topk_stride_requirement(rt.DS_BF16) == 8
    assert rt.ds_topk_stride_requirement(7) == 0


def test_status_strings():
    for code in range(len(rt.STATUS_NAMES)):
        s = rt.ds_topk_status_string(code)
        assert isinstance(s, str) and s
    assert rt.ds_topk_status_string(99) == "unknown status"


def _v(**kw):
    a = dict(x=A16, dtype=rt.DS_FP32, batch=4, n_cols=1000, row_stride=1000, end=None, k=10,
             sorted=1, return_values=1, index_dtype=rt.DS_INT32, values=A16b, indices=A16c,
             row_status=A16d, workspace=None, workspace_bytes=0, plan=None)
    a.update(kw)
    return rt.ds_topk_validate(a["x"], a["dtype"], a["batch"], a["n_cols"], a["row_stride"],
                               a["end"], a["k"], a["sorted"], a["return_values"],
                               a["index_dtype"], a["values"], a["indices"], a["row_status"],
                               a["workspace"], a["workspace_bytes"], a["plan"])


ERR = {n: i for i, n in enumerate(rt.STATUS_NAMES)}


@pytest.mark.parametrize("kw,code", [
    ({}, "DS_OK"),
    ({"dtype": 2}, "DS_ERR_DTYPE"),
    ({"index_dtype": 5}, "DS_ERR_INDEX_DTYPE"),
    ({"sorted": 3}, "DS_ERR_SORTED_MODE"),
    ({"sorted": -1}, "DS_ERR_SORTED_MODE"),
    ({"k": 0}, "DS_ERR_K_RANGE"),
    ({"k": 4097}, "DS_ERR_K_RANGE"),
    ({"k": 4096}, "DS_OK"),
    ({"k": 2000}, "DS_OK"),                      # k > n_cols is allowed (padding)
    ({"batch": -1}, "DS_ERR_SHAPE"),
    ({"n_cols": -1}, "DS_ERR_SHAPE"),
    ({"row_stride": 996}, "DS_ERR_SHAPE"),       # stride < n_cols
    ({"n_cols": 2**31, "row_stride": 2**31}, "DS_ERR_SHAPE"),
    ({"x": None}, "DS_ERR_NULL"),
    ({"indices": None}, "DS_ERR_NULL"),
    ({"row_status": None}, "DS_ERR_NULL"),
    ({"values": None}, "DS_ERR_NULL"),
    ({"values": None, "return_values": 0}, "DS_OK"),
    ({"x": A16 + 4}, "DS_ERR_ALIGN"),
    ({"row_stride": 1002}, "DS_ERR_ALIGN"),      # 4008 B is not a multiple of 16
    ({"dtype": rt.DS_BF16, "row_stride": 1004}, "DS_ERR_ALIGN"),
    ({"dtype": rt.DS_BF16, "row_stride": 1008}, "DS_OK"),
    ({"indices": A16c + 2}, "DS_ERR_ALIGN"),
    ({"indices": A16c + 4, "index_dtype": rt.DS_INT64}, "DS_ERR_ALIGN"),
    ({"values": A16b + 2}, "DS_ERR_ALIGN"),
    ({"row_status": A16d + 2}, "DS_ERR_ALIGN"),
    ({"end": A16 + 2}, "DS_ERR_ALIGN"),
    ({"batch": 0, "x": None, "indices": None, "row_status": None, "values": None}, "DS_OK"),
    ({"n_cols": 0, "row_stride": 0, "x": None}, "DS_OK"),
    ({"plan": {"segments": -1}}, "DS_ERR_PLAN"),
    ({"plan": {"segments": 257}}, "DS_ERR_PLAN"),
    ({"plan": {"in_order": 2}}, "DS_ERR_PLAN"),
    ({"plan": {"flush_at": 10}}, "DS_ERR_PLAN"),       # must exceed k
    ({"plan": {"flush_at": 100000}}, "DS_ERR_PLAN"),   # beyond the buffer's trigger
    ({"plan": {"flush_at": 11}}, "DS_OK"),
    ({"plan": {"segments": 1}}, "DS_OK"),
    ({"plan": {"kernel": 3}}, "DS_ERR_PLAN"),
    ({"plan": {"kernel": -1}}, "DS_ERR_PLAN"),
    ({"plan": {"kernel": 1}}, "DS_OK"),
    ({"plan": {"kernel": 2, "segments": 9}}, "DS_OK"),
])
def test_validate_codes(kw, code):
    assert _v(**kw) == ERR[code]


def test_workspace_rules():
    # A sampler-shaped problem spreads rows over several workgroups: needs a workspace.
    need = rt.ds_topk_workspace_size(rt.DS_FP32, 64, 129280, 1024)
    assert need > 0
    base = dict(batch=64, n_cols=129280, row_stride=129280, k=1024)
    assert _v(**base) == ERR["DS_ERR_WORKSPACE"]
    assert _v(**base, workspace=A16w, workspace_bytes=need - 1) == ERR["DS_ERR_WORKSPACE"]
    assert _v(**base, workspace=A16w + 8, workspace_bytes=need) == ERR["DS_ERR_WORKSPACE"]
    assert _v(**base, workspace=A16w, workspace_bytes=need) == ERR["DS_OK"]
    # Many rows: one workgroup per row, no workspace.
    assert rt.ds_topk_workspace_size(rt.DS_BF16, 4096, 65536, 2048) == 0
    # Explicit single-segment plan needs none; more segments need more (the
    # stream kernel takes any count; the chunk kernels one per chunk).
    for kern in (1, 2):
        one = {"segments": 1, "kernel": kern}
        assert rt.ds_topk_workspace_size_ex(rt.DS_FP32, 64, 129280, 1024, one) == 0
    s4 = rt.ds_topk_workspace_size_ex(rt.DS_FP32, 64, 129280, 1024, {"segments": 4, "kernel": 1})
    s16 = rt.ds_topk_workspace_size_ex(rt.DS_FP32, 64, 129280, 1024, {"segments": 16, "kernel": 1})
    assert 0 < s4 < s16
    # The chunk kernels split a row into its chunks (32768 fp32 values each:
    # four for 129,280 columns): a fixed header of counters, a record and k
    # slots per chunk.
    c = rt.ds_topk_workspace_size_ex(rt.DS_FP32, 64, 129280, 1024, {"kernel": 2, "segments": 2})
    assert c == rt.ds_topk_workspace_size(rt.DS_FP32, 64, 129280, 1024)
    assert c >= rt.DS_TOPK_WS_HEADER_BYTES + 64 * 4 * 1024 * 8
    # Every split layout starts after the fixed counter header.
    assert c > rt.DS_TOPK_WS_HEADER_BYTES and s4 > rt.DS_TOPK_WS_HEADER_BYTES
    # Rows shared by workgroups are limited to the header's capacity: an
    # explicit split beyond it is refused, the automatic plan does not split.
    big = rt.DS_TOPK_MAX_SPLIT_ROWS + 1
    assert rt.ds_topk_workspace_size_ex(rt.DS_FP32, big, 129280, 64, {"segments": 4, "kernel": 1}) == 0
    assert _v(batch=big, n_cols=8192, row_stride=8192, k=64, plan={"segments": 4, "kernel": 1}) == ERR["DS_ERR_PLAN"]
    assert rt.ds_topk_workspace_size(rt.DS_FP32, big, 8192, 64) == 0
    # A plan's kernel field is checked.
    assert rt.ds_topk_workspace_size_ex(rt.DS_FP32, 64, 129280, 1024, {"kernel": 3}) == 0
    # Invalid arguments give 0.
    assert rt.ds_topk_workspace_size(rt.DS_FP32, 64, 129280, 0) == 0
    assert rt.ds_topk_workspace_size(9, 64, 129280, 10) == 0


def test_invalid_call_returns_before_launch():
    # Argument errors come back synchronously; nothing touches the GPU.
    rc = rt.ds_topk(A16, rt.DS_FP32, 4, 1000, 1000, None, 0, 1, 1, rt.DS_INT32, A16b, A16c,
                    A16d, None, 0, None)
    assert rc == ERR["DS_ERR_K_RANGE"]
    rc = rt.ds_topk_ex(A16, rt.DS_FP32, 0, 1000, 1000, None, 5, 1, 1, rt.DS_INT32, None, None,
                       None, None, 0, None, None)
    assert rc == ERR["DS_OK"]   # batch == 0: nothing to do


@pytest.mark.parametrize("kw,code", [
    ({"sink": None}, "DS_ERR_NULL"),
    ({"x": None}, "DS_ERR_NULL"),
    ({"sink": A16b + 2}, "DS_ERR_ALIGN"),
    ({"x": A16 + 4}, "DS_ERR_ALIGN"),
    ({"row_stride": 1002}, "DS_ERR_ALIGN"),
    ({"end": A16 + 2}, "DS_ERR_ALIGN"),
    ({"k": 0}, "DS_ERR_K_RANGE"),
    ({"dtype": 3}, "DS_ERR_DTYPE"),
    ({"row_stride": 996}, "DS_ERR_SHAPE"),
    ({"plan": {"segments": 300}}, "DS_ERR_PLAN"),
    ({"batch": 0, "x": None, "sink": None}, "DS_OK"),
])
def test_read_ceiling_argument_errors(kw, code):
    # Every case returns before a launch (batch == 0 launches nothing).
    a = dict(x=A16, dtype=rt.DS_FP32, batch=4, n_cols=1000, row_stride=1000, end=None, k=10,
             plan=None, sink=A16b, stream=None)
    a.update(kw)
    rc = rt.ds_read_ceiling(a["x"], a["dtype"], a["batch"], a["n_cols"], a["row_stride"],
                            a["end"], a["k"], a["plan"], a["sink"], a["stream"])
    assert rc == ERR[code]


def test_product_path_has_no_oracle_or_fallback():
    import inspect
    src = inspect.getsource(rt)
    assert "oracle" not in src.replace("no fallback", "")
    assert "import numpy" not in src


def test_out_tensors_are_checked():
    """topk(out=...) refuses buffers the kernel would write past or misread
    (checked before anything is launched, so no GPU is needed)."""
    import pytest
    import torch

    x = torch.empty((4, 1000), dtype=torch.float32)
    ok = (torch.empty((4, 8), dtype=torch.float32), torch.empty((4, 8), dtype=torch.int32),
          torch.empty((4,), dtype=torch.int32))
    bad = [
        (ok[0], torch.empty((4, 8), dtype=torch.int64), ok[2]),      # index dtype
        (ok[0], torch.empty((4, 7), dtype=torch.int32), ok[2]),      # k
        (torch.empty((4, 8), dtype=torch.bfloat16), ok[1], ok[2]),   # value dtype
        (ok[0], ok[1], torch.empty((3,), dtype=torch.int32)),        # status shape
        (ok[0], torch.empty((8, 4), dtype=torch.int32).t(), ok[2]),  # not contiguous
    ]
    for out in bad:
        with pytest.raises(ValueError):
            rt._check_out(*out, 4, 8, torch.float32, torch.int32, True, x.device)
    rt._check_out(*ok, 4, 8, torch.float32, torch.int32, True, x.device)
    rt._check_out(None, ok[1], ok[2], 4, 8, torch.float32, torch.int32, False, x.device)


def test_noalloc_refusals_need_no_gpu():
    """The allocation-free entry point refuses, before any HIP call, a problem
    whose workspace exceeds its static scratch, and bad arguments."""
    plan = rt.Plan(segments=16, perm_seed=1, kernel=rt.DS_KERNEL_CHUNK)
    assert rt.ds_topk_workspace_size_ex(rt.DS_FP32, 256, 129280, 4096, plan) > rt.DS_TOPK_NOALLOC_SCRATCH_BYTES
    rc = rt.ds_topk_noalloc(None, rt.DS_FP32, 256, 129280, 129280, None, 4096, 1, 0, rt.DS_INT32,
                            None, None, None, None, plan)
    assert rc == rt.DS_ERR_SCRATCH_LIMIT
    rc = rt.ds_topk_noalloc(None, rt.DS_BF16, 4, 1000, 1000, None, 10, 1, 0, rt.DS_INT32, None,
                            None, None, None, None)
    assert rt.STATUS_NAMES[rc] == "DS_ERR_NULL"
    rc = rt.ds_topk_noalloc(None, rt.DS_BF16, 4, 1000, 1000, None, 0, 1, 0, rt.DS_INT32, None,
                            None, None, None, None)
    assert rt.STATUS_NAMES[rc] == "DS_ERR_K_RANGE"


_C = {name: i for i, name in enumerate(rt.STATUS_NAMES)}


# ds_sampler_tail's argument checks, in their documented order, before any
# launch (fake device addresses: nothing is dereferenced).
_TAIL = dict(values=A16, dtype=rt.DS_FP32, indices=A16b, index_dtype=rt.DS_INT64, row_status=None,
             batch=4, k=1024, temperature=0.7, top_p=0.9, uniforms=A16c, tokens=A16d, probs=A16w,
             stream=None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), _C["DS_ERR_DTYPE"]),
    (dict(index_dtype=9), _C["DS_ERR_INDEX_DTYPE"]),
    (dict(k=0), _C["DS_ERR_K_RANGE"]),
    (dict(k=4097), _C["DS_ERR_K_RANGE"]),
    (dict(batch=-1), _C["DS_ERR_SHAPE"]),
    (dict(batch=1 << 31), _C["DS_ERR_SHAPE"]),
    (dict(temperature=float("nan")), _C["DS_ERR_SAMPLER_PARAM"]),
    (dict(top_p=0.0), _C["DS_ERR_SAMPLER_PARAM"]),
    (dict(top_p=-0.5), _C["DS_ERR_SAMPLER_PARAM"]),
    (dict(top_p=float("nan")), _C["DS_ERR_SAMPLER_PARAM"]),
    (dict(values=None), _C["DS_ERR_NULL"]),
    (dict(indices=None), _C["DS_ERR_NULL"]),
    (dict(uniforms=None), _C["DS_ERR_NULL"]),
    (dict(tokens=None), _C["DS_ERR_NULL"]),
    (dict(values=A16 + 2), _C["DS_ERR_ALIGN"]),
    (dict(indices=A16b + 4), _C["DS_ERR_ALIGN"]),
    (dict(tokens=A16d + 4), _C["DS_ERR_ALIGN"]),
    (dict(probs=A16w + 2), _C["DS_ERR_ALIGN"]),
    (dict(batch=0, values=None, tokens=None), _C["DS_OK"]),
])
def test_sampler_tail_argument_errors(kw, code):
    a = dict(_TAIL, **kw)
    assert rt.ds_sampler_tail(a["values"], a["dtype"], a["indices"], a["index_dtype"], a["row_status"],
                              a["batch"], a["k"], a["temperature"], a["top_p"], a["uniforms"],
                              a["tokens"], a["probs"], a["stream"]) == code
