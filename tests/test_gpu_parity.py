"""GPU parity: the HIP path against the CPU oracle, element by element.

Workloads at reduced sizes (several 4096-element blocks and a ragged tail) and
at full size, in the launch configuration the benchmark uses; edge cases of the
method (ties, signed zeros, infinities, NaN inside and past `end`, short and
empty rows, k at each class boundary, strides wider than the row).  Indices
and values must match bit for bit; unsorted results are compared as sets.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.gpu_util import BF16, FP32, check_case, say

pytestmark = pytest.mark.gpu


def _wl_case(num, name, **shape):
    w = workloads.workload(num, **shape)
    x, end = workloads.make_input(w, poison_tail=True)
    check_case(x, w.dtype, w.n_cols, w.k, w.sorted, w.return_values, w.index_dtype, end,
               name=name)


# ---------------------------------------------------------------- workloads, reduced
@pytest.mark.parametrize("num,shape", [
    (1, {}),
    (2, {"batch": 8}),
    (2, {"batch": 5, "n_cols": 50001}),
    (3, {"batch": 8}),
    (3, {"batch": 3, "n_cols": 30007}),
    (4, {"batch": 256, "n_cols": 8192}),
    (5, {"batch": 2, "n_cols": 1 << 20}),
])
def test_workload_reduced(num, shape):
    _wl_case(num, f"workload{num} {shape}", **shape)


# ---------------------------------------------------------------- workloads, full size
@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_workload_full(num):
    _wl_case(num, f"workload{num} full")


# ---------------------------------------------------------------- every option
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("sorted_mode", [0, 1, 2])
@pytest.mark.parametrize("return_values", [True, False])
@pytest.mark.parametrize("index_dtype", ["int32", "int64"])
def test_options(dtype, sorted_mode, return_values, index_dtype):
    rng = np.random.Generator(np.random.PCG64(21))
    f = rng.standard_normal((6, 20000)).astype(np.float32)
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    check_case(x, dtype, 20000, 300, sorted_mode, return_values, index_dtype, name="options")


# ---------------------------------------------------------------- k classes
@pytest.mark.parametrize("k", [1, 2, 63, 256, 257, 1000, 1024, 1025, 2048, 2049, 3000, 4096])
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_k_classes(k, dtype):
    rng = np.random.Generator(np.random.PCG64(k))
    f = rng.standard_normal((4, 40000)).astype(np.float32)
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    check_case(x, dtype, 40000, k, 1, name=f"k={k}")


# ---------------------------------------------------------------- edge cases
def _bits_rows(f32, dtype):
    return workloads.to_bf16_bits(f32) if dtype == BF16 else np.ascontiguousarray(f32, np.float32)


@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("sorted_mode", [0, 1, 2])
def test_all_equal_rows(dtype, sorted_mode):
    f = np.full((3, 12000), 1.25, dtype=np.float32)
    for k in (1, 100, 1024, 4096):
        check_case(_bits_rows(f, dtype), dtype, 12000, k, sorted_mode, name=f"all-equal k={k}")


@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_signed_zeros_and_infinities(dtype):
    rng = np.random.Generator(np.random.PCG64(3))
    alpha = np.array([-0.0, 0.0, 1.0, -1.0, np.inf, -np.inf], dtype=np.float32)
    f = alpha[rng.integers(0, len(alpha), size=(5, 9000))]
    for k in (7, 500, 3000):
        for sm in (0, 1, 2):
            check_case(_bits_rows(f, dtype), dtype, 9000, k, sm, name=f"zeros/inf k={k}")


@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_masked_logits(dtype):
    rng = np.random.Generator(np.random.PCG64(4))
    f = np.full((4, 30000), -np.inf, dtype=np.float32)
    for i in range(4):
        pos = rng.choice(30000, 40 * (i + 1), replace=False)
        f[i, pos] = rng.standard_normal(len(pos)).astype(np.float32)
    for k in (10, 200, 1024):
        check_case(_bits_rows(f, dtype), dtype, 30000, k, 1, name=f"masked k={k}")


@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_nan_inside_and_past_end(dtype):
    rng = np.random.Generator(np.random.PCG64(5))
    batch, n = 16, 20000
    f = rng.standard_normal((batch, n)).astype(np.float32)
    x = _bits_rows(f, dtype)
    end = rng.integers(0, n + 1, size=batch).astype(np.int32)
    end[0], end[1] = n, 0
    pats = ([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF] if dtype == FP32
            else [0x7FC0, 0xFFC0, 0x7F81, 0xFFFF])
    view = x.view(np.uint32) if dtype == FP32 else x
    for i in range(batch):
        if i % 3 == 0 and end[i] > 0:
            view[i, rng.integers(0, end[i])] = pats[i % 4]
        if i % 3 == 1 and end[i] < n:
            view[i, rng.integers(end[i], n)] = pats[i % 4]   # past end: ignored
    for sm in (0, 1):
        check_case(x, dtype, n, 64, sm, end=end, name="nan")


def test_bad_end_and_short_rows():
    rng = np.random.Generator(np.random.PCG64(6))
    f = rng.standard_normal((8, 5000)).astype(np.float32)
    end = np.array([-1, 5001, 0, 1, 99, 100, 4999, 5000], dtype=np.int32)
    for sm in (0, 1, 2):
        check_case(f, FP32, 5000, 100, sm, end=end, name="ends")


@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_odd_tails_and_wide_strides(dtype):
    rng = np.random.Generator(np.random.PCG64(8))
    for n, stride in ((4097, 4104), (1, 8), (13, 16), (8191, 8200), (12345, 20000)):
        f = np.full((3, stride), np.nan, dtype=np.float32)
        f[:, :n] = rng.standard_normal((3, n)).astype(np.float32)
        x = _bits_rows(f, dtype)
        if dtype == BF16:
            x[:, n:] = 0x7FC0
        for k in (1, 5, 300):
            check_case(x, dtype, n, k, 1, name=f"n={n} stride={stride} k={k}")


def test_k_larger_than_row():
    f = np.arange(300, dtype=np.float32)[None, :].repeat(2, axis=0)
    check_case(f, FP32, 300, 1000, 1, name="k>n")
    check_case(f, FP32, 300, 4096, 2, name="k>n idx")


def test_one_huge_row():
    rng = np.random.Generator(np.random.PCG64(9))
    f = rng.standard_normal((1, 1 << 22)).astype(np.float32)
    check_case(f, FP32, 1 << 22, 1000, 1, name="1x4M k=1000")


def test_ascending_and_descending_rows():
    n = 1 << 18
    asc = (np.arange(n, dtype=np.float64) / float(1 << 24)).astype(np.float32)
    f = np.stack([asc, asc[::-1].copy()])
    for k in (1, 512, 4096):
        got = check_case(f, FP32, n, k, 1, name=f"monotone k={k}")
        assert got[1][0].tolist() == list(range(n - 1, n - 1 - k, -1))
        assert got[1][1].tolist() == list(range(k))


# ---------------------------------------------------------------- plans: same answer
@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("plan", [
    {"segments": 1}, {"segments": 2}, {"segments": 3}, {"segments": 7}, {"segments": 16},
    {"segments": 64}, {"perm_seed": 1}, {"perm_seed": 0xDEADBEEF}, {"in_order": 1},
    {"in_order": 1, "segments": 5}, {"flush_at": 1100}, {"flush_at": 1030, "segments": 3},
])
def test_plan_independence(plan, kernel):
    plan = dict(plan, kernel=kernel)
    w = workloads.workload(2, batch=6)
    x, _ = workloads.make_input(w)
    check_case(x, w.dtype, w.n_cols, w.k, 1, True, "int64", plan=plan, name=f"plan {plan}")
    w3 = workloads.workload(3, batch=6)
    x3, _ = workloads.make_input(w3)
    p3 = dict(plan)
    if "flush_at" in p3:
        p3["flush_at"] = p3["flush_at"] - 1024 + 520
    check_case(x3, w3.dtype, w3.n_cols, w3.k, 2, False, "int32", plan=p3, name=f"plan3 {p3}")


def test_adversarial_plans_many_cuts():
    n = 1 << 19
    asc = (np.arange(n, dtype=np.float64) / float(1 << 24)).astype(np.float32)
    rng = np.random.Generator(np.random.PCG64(10))
    f = np.stack([asc + np.float32(1e-3) * rng.random(n, dtype=np.float32) for _ in range(2)])
    for plan in ({"in_order": 1}, {"in_order": 1, "flush_at": 4100}, {"segments": 32},
                 {"segments": 1, "flush_at": 4097}):
        for kernel in (1, 2):
            p = dict(plan, kernel=kernel)
            check_case(f, FP32, n, 4096, 1, plan=p, name=f"ascending {p}")


def test_repeat_determinism():
    import torch
    from tests.gpu_util import gpu_topk, to_device
    w = workloads.workload(3, batch=16)
    x, _ = workloads.make_input(w)
    xt = to_device(x, w.dtype)
    say("repeat determinism x100 (sorted=1 and sorted=0)")
    first = gpu_topk(x, w.dtype, w.n_cols, w.k, 1, True, xt=xt)
    first0 = gpu_topk(x, w.dtype, w.n_cols, w.k, 0, False, xt=xt)
    for _ in range(100):
        again = gpu_topk(x, w.dtype, w.n_cols, w.k, 1, True, xt=xt)
        assert all(np.array_equal(a, b) for a, b in zip(first, again))
        again0 = gpu_topk(x, w.dtype, w.n_cols, w.k, 0, False, xt=xt)
        assert np.array_equal(np.sort(first0[1], axis=1), np.sort(again0[1], axis=1))
    torch.cuda.synchronize()


def test_workspace_header_zero_after_every_call():
    """Calls with different (batch, segments, k) share one workspace.  Only its
    fixed header of per-row counters must be zero when a call starts, and each
    call leaves it zero; the rest is filled with garbage before every call
    (all-ones words, which would rank first if a kernel read them as
    candidates, or random bytes), and the results must not change."""
    import torch
    import row_wise_topk_amd as rt
    from tests.gpu_util import to_device
    rng = np.random.Generator(np.random.PCG64(12))
    shapes = [(8, 129280, 1024, {}), (5, 50001, 1024, {}), (8, 131072, 512, {}),
              (3, 9000, 7, {}), (2, 262144, 1, {}), (6, 129280, 1024, {"segments": 64, "kernel": 1}),
              (1, 1 << 20, 4096, {}), (64, 20000, 300, {"segments": 3, "kernel": 1}),
              (8, 129280, 1024, {"kernel": 1}), (6, 131072, 512, {"kernel": 2}),
              (3, 200000, 2048, {"kernel": 2, "segments": 2}), (40, 70000, 64, {"kernel": 1})]
    for i, (batch, n, k, plan) in enumerate(shapes):
        dtype = BF16 if i % 2 else FP32
        step = 8 if dtype == BF16 else 4
        stride = (n + step - 1) // step * step
        f = np.full((batch, stride), np.nan, dtype=np.float32)
        f[:, :n] = rng.standard_normal((batch, n)).astype(np.float32)
        x = workloads.to_bf16_bits(f) if dtype == BF16 else f
        say(f"workspace reuse batch={batch} n={n} k={k} plan={plan}")
        H = rt.DS_TOPK_WS_HEADER_BYTES
        for buf in rt._workspaces.values():
            if buf.numel() > H:
                if i % 2:
                    g = torch.Generator().manual_seed(i)
                    buf[H:] = torch.randint(0, 256, (buf.numel() - H,), generator=g,
                                            dtype=torch.uint8).to(buf.device)
                else:
                    buf[H:] = 0xFF
        torch.cuda.synchronize()
        check_case(x, dtype, n, k, 1, plan=plan or None, name="workspace reuse")
        torch.cuda.synchronize()
        for buf in rt._workspaces.values():
            assert int(torch.count_nonzero(buf[:H]).item()) == 0, "workspace header left dirty"
