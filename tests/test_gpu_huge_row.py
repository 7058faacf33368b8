"""GPU checks for one very long fp32 row, top 1000.

This is the pages' torch.topk pathology case: the top 1000 of a billion
floats (xhh.club, "DeepSeek开源DeepSelect：比torch.topk快二十倍！", section
"torch.topk 的性能痛点与版本波动").  Its values are i.i.d. N(0, 1).  The
planner gives it every resident workgroup (one row shared by 256).

The oracle's full sort of a billion values is out of reach. So at full size
the result is checked by properties that fix the exact top k at any size,
computed with plain torch operations on the GPU:
- the indices are distinct and in range;
- the values are bit copies of the inputs at those indices;
- the output is ordered by value, larger first, ties by lower index;
- exactly k - 1 elements of the row come before the last result in that order.
Together these pin the result to the k first elements of the row in that order.

A row of 2^24 values with the same k and planner (16 blocks per workgroup,
so the estimated start applies) is compared with the oracle element by
element, and so is a row of 2^27 values shared by all 256 workgroups, as at
full size: 128 blocks per workgroup, many cuts each.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import FP32, check_case

pytestmark = pytest.mark.gpu


def test_billion_row_top1000_properties():
    import row_wise_topk_amd as rt
    w = workloads.workload(6)
    print(f"[huge row] {w.name}: generating", flush=True)
    x_np, _ = workloads.make_input(w)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(x_np).to(dev)
    del x_np
    print("[huge row] running", flush=True)
    v, ix, st = rt.topk(x, w.k, sorted=1, return_values=True, index_dtype=torch.int64)
    torch.cuda.synchronize()
    assert int(st[0].item()) == 0
    row, v, ix = x[0], v[0], ix[0]
    assert int(ix.min().item()) >= 0 and int(ix.max().item()) < w.n_cols
    assert torch.unique(ix).numel() == w.k
    assert torch.equal(v.view(torch.int32), row[ix].view(torch.int32))
    ordered = (v[:-1] > v[1:]) | ((v[:-1] == v[1:]) & (ix[:-1] < ix[1:]))
    assert bool(ordered.all().item())
    vk, ik = v[-1], int(ix[-1].item())
    before = int((row > vk).sum().item()) + int((row[:ik] == vk).sum().item())
    assert before == w.k - 1


@pytest.mark.parametrize("sorted_mode", [1, 0])
def test_long_row_top1000_vs_oracle(sorted_mode):
    w = workloads.workload(6, n_cols=1 << 24)
    x, _ = workloads.make_input(w)
    check_case(x, FP32, w.n_cols, w.k, sorted_mode, True, "int64",
               name=f"long row 1x{w.n_cols} k={w.k} sorted={sorted_mode}")


def test_long_row_256_workgroups_vs_oracle():
    w = workloads.workload(6, n_cols=1 << 27)
    x, _ = workloads.make_input(w)
    check_case(x, FP32, w.n_cols, w.k, 1, True, "int64", plan={"kernel": 1, "segments": 256},
               name=f"long row 1x{w.n_cols} k={w.k}, 256 workgroups")
