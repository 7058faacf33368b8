"""ds_topk_noalloc, the allocation-free entry point, against ds_topk_ex.

Two calls in a row through the C ABI, the second with a smaller input, each
compared bit for bit with ds_topk_ex on the same input (with a workspace the
test allocates); the sampler shape runs split over several workgroups, so the
library's static scratch is what its kernels use.  A problem whose workspace
exceeds the scratch is refused before anything is launched.
"""
from __future__ import annotations

import pytest

import workloads
from tests.gpu_util import BF16, FP32, to_device

pytestmark = pytest.mark.gpu


def _outputs(torch, batch, k, dtype, return_values, it):
    vals = torch.empty((batch, k), dtype=torch.float32 if dtype == FP32 else torch.bfloat16,
                       device="cuda") if return_values else None
    idx = torch.full((batch, k), -7, dtype=it, device="cuda")
    st = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
    return vals, idx, st


def _call(rt, torch, fn, xt, dtype, batch, n, stride, k, sorted_, rv, it, plan):
    vals, idx, st = _outputs(torch, batch, k, dtype, rv, it)
    stream = torch.cuda.current_stream().cuda_stream
    idt = rt.DS_INT64 if it == torch.int64 else rt.DS_INT32
    vp = vals.data_ptr() if vals is not None else None
    if fn == "ex":
        nbytes = rt.ds_topk_workspace_size_ex(dtype, batch, n, k, plan)
        ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        rc = rt.ds_topk_ex(xt.data_ptr(), dtype, batch, n, stride, None, k, sorted_, int(rv), idt,
                           vp, idx.data_ptr(), st.data_ptr(), ws.data_ptr(), ws.numel(), stream, plan)
    else:
        rc = rt.ds_topk_noalloc(xt.data_ptr(), dtype, batch, n, stride, None, k, sorted_, int(rv),
                                idt, vp, idx.data_ptr(), st.data_ptr(), stream, plan)
    torch.cuda.synchronize()
    assert rc == rt.DS_OK, rt.ds_topk_status_string(rc)
    return [None if t is None else t.cpu() for t in (vals, idx, st)]


def _same(torch, a, b, sorted_):
    if sorted_ == 0:   # any order is valid: compare in index order
        for o in (a, b):
            order = o[1].argsort(dim=1)
            o[1] = o[1].gather(1, order)
            if o[0] is not None:
                o[0] = o[0].gather(1, order)
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        xi = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32) if x.dtype == torch.float32 else x
        yi = y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32) if y.dtype == torch.float32 else y
        assert torch.equal(xi, yi)


def test_noalloc_matches_ex_twice_then_smaller():
    import torch
    import row_wise_topk_amd as rt
    cases = [
        # (workload, batch, n_cols, plan): the sampler shape split by chunks, then a smaller bf16 problem
        (2, 64, 129280, None),
        (3, 16, 140000, rt.Plan(segments=3, perm_seed=7, kernel=rt.DS_KERNEL_CHUNK)),
    ]
    for num, batch, n, plan in cases:
        w = workloads.workload(num, batch=batch, n_cols=n)
        x, _ = workloads.make_input(w)
        xt = to_device(x, w.dtype)
        it = torch.int64 if w.index_dtype == "int64" else torch.int32
        need = rt.ds_topk_workspace_size_ex(w.dtype, batch, n, w.k, plan)
        print(f"noalloc {w.name} batch={batch} n={n} plan={plan and plan.segments} "
              f"workspace {need} bytes", flush=True)
        assert 0 < need <= rt.DS_TOPK_NOALLOC_SCRATCH_BYTES
        ref = _call(rt, torch, "ex", xt, w.dtype, batch, n, w.row_stride, w.k, w.sorted,
                    w.return_values, it, plan)
        got = _call(rt, torch, "noalloc", xt, w.dtype, batch, n, w.row_stride, w.k, w.sorted,
                    w.return_values, it, plan)
        assert int(got[2].abs().sum()) == 0
        _same(torch, got, ref, w.sorted)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    import torch
    import row_wise_topk_amd as rt
    batch, n, k = 256, 129280, 4096
    plan = rt.Plan(segments=16, perm_seed=1, kernel=rt.DS_KERNEL_CHUNK)
    need = rt.ds_topk_workspace_size_ex(FP32, batch, n, k, plan)
    assert need > rt.DS_TOPK_NOALLOC_SCRATCH_BYTES
    # Pointers are never dereferenced: the size check comes before anything else.
    x = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((batch, k), dtype=torch.int32, device="cuda")
    st = torch.empty((batch,), dtype=torch.int32, device="cuda")
    rc = rt.ds_topk_noalloc(x.data_ptr(), FP32, batch, n, n, None, k, 1, 0, rt.DS_INT32, None,
                            idx.data_ptr(), st.data_ptr(), torch.cuda.current_stream().cuda_stream,
                            plan)
    assert rc == rt.DS_ERR_SCRATCH_LIMIT
    assert "scratch" in rt.ds_topk_status_string(rc)


def test_noalloc_argument_errors_before_any_launch():
    import row_wise_topk_amd as rt
    # NULL indices: refused by the argument checks.
    rc = rt.ds_topk_noalloc(None, BF16, 4, 1000, 1000, None, 10, 1, 0, rt.DS_INT32, None, None,
                            None, None, None)
    assert rt.STATUS_NAMES[rc] == "DS_ERR_NULL"
