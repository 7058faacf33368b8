"""The read-ceiling measurement kernel runs through the C ABI on the shapes
the benchmark times (one and several workgroups per row, bf16 with a per-row
`end`, the 512-lane class, a ragged tail) and returns without error.  It
computes nothing to compare: it only reads what the selection reads."""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,n,k,bf16,with_end", [
    (8, 129280, 1024, False, False),
    (16, 131072, 512, True, False),
    (64, 65536, 2048, True, True),
    (2, 1 << 20, 4096, False, False),
    (5, 50001, 7, False, True),
])
def test_read_ceiling_runs(batch, n, k, bf16, with_end):
    import torch
    import row_wise_topk_amd as rt
    say(f"read ceiling batch={batch} n={n} k={k} bf16={bf16} end={with_end}")
    step = 8 if bf16 else 4
    stride = (n + step - 1) // step * step
    dt = torch.bfloat16 if bf16 else torch.float32
    x = torch.randn((batch, stride), device="cuda").to(dt)
    end = None
    if with_end:
        rng = np.random.Generator(np.random.PCG64(5))
        end = torch.from_numpy(rng.integers(0, n + 1, batch).astype(np.int32)).cuda()
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    rt.read_ceiling(x, k, end=end, n_cols=n, sink=sink)
    rt.read_ceiling(x, k, end=end, n_cols=n, sink=sink, plan=rt.Plan(segments=3))
    torch.cuda.synchronize()
