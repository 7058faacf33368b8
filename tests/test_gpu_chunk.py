"""GPU parity for the data-dependent paths of the chunk kernels.

A 512-lane workgroup of the chunk kernels holds a chunk of a row in
registers, 16384 fp32 or 32768 bf16 values: a row is either split into one
workgroup per chunk (the last to finish merges the others' candidates) or
taken whole by one workgroup, chunk by chunk.  The first chunk of a workgroup sets the start
threshold: exact when the chunk is the whole row, otherwise an estimate of
the row's k-th value for the chunk's share, checked once the row is
complete (the row is read again from -inf when fewer than min(k, L)
candidates passed it).  A chunk whose candidates would overflow the buffer is
appended one vector per lane at a time, with cuts in between.

Each case here forces one of those paths with rows built for it, and the
result must still be the oracle's, bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.gpu_util import BF16, CHUNK_ELEMS, CHUNK_ELEMS_ROW, FP32, check_case

pytestmark = pytest.mark.gpu

SPLIT = {"kernel": 2, "segments": 2}
WHOLE = {"kernel": 2, "segments": 1}


def ce_of(dtype, plan):
    """Values per chunk for the plan (whole rows: segments 1)."""
    return (CHUNK_ELEMS_ROW if plan.get("segments") == 1 else CHUNK_ELEMS)[dtype]


def _bits(f, dtype):
    """Rows as the kernels take them: bf16 bit patterns or fp32, the row
    stride padded to 16 bytes with NaN (past n_cols: never read as data)."""
    n = f.shape[1]
    step = 8 if dtype == BF16 else 4
    stride = (n + step - 1) // step * step
    p = np.full((f.shape[0], stride), np.nan, dtype=np.float32)
    p[:, :n] = f
    return workloads.to_bf16_bits(p) if dtype == BF16 else p


# One chunk holds every large value: its share of the top k far exceeds the
# estimate's margin, so the merge check (split rows) or the final count (whole
# rows, when that chunk is visited first) fails and the row is read again.
@pytest.mark.parametrize("plan", [SPLIT, WHOLE, dict(WHOLE, in_order=1)])
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("k", [64, 1024])
def test_estimate_rejected_hot_chunk(plan, dtype, k):
    rng = np.random.Generator(np.random.PCG64(500 + k + dtype))
    ce = ce_of(dtype, plan)
    n = 6 * ce
    f = rng.standard_normal((3, n)).astype(np.float32)
    for r in range(3):
        c = r % 6
        f[r, c * ce:(c + 1) * ce] += np.float32(50.0)
    x = _bits(f, dtype)
    check_case(x, dtype, n, k, 1, True, "int32", plan=plan, name=f"hot chunk k={k} {plan}")
    check_case(x, dtype, n, k, 0, False, "int64", plan=plan, name=f"hot chunk unsorted k={k} {plan}")


# Descending rows: the first chunk in address order holds the whole top k.
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_descending_rows_whole(dtype):
    for plan in (dict(WHOLE, in_order=1), WHOLE, SPLIT):
        n = 5 * ce_of(dtype, plan) + 777
        f = (np.arange(n, dtype=np.float64)[::-1] / n).astype(np.float32)[None, :].repeat(2, axis=0)
        x = _bits(f, dtype)
        for k in (100, 2048):
            check_case(x, dtype, n, k, 1, True, "int32", plan=plan, name=f"descending k={k} {plan}")


# Ascending rows and a small flush point: every chunk overflows the buffer and
# is appended piecewise, with a cut before each vector that might not fit.
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("flush_at", [0, 1])
def test_piecewise_appends(dtype, flush_at):
    rng = np.random.Generator(np.random.PCG64(77 + dtype))
    for plan in (dict(WHOLE, in_order=1), SPLIT):
        n = 7 * ce_of(dtype, plan) + 5
        f = (np.arange(n, dtype=np.float64) / n).astype(np.float32)[None, :] \
            + np.float32(1e-4) * rng.random((2, n), dtype=np.float32)
        x = _bits(f, dtype)
        for k, sm, idx in ((4096, 1, "int32"), (1000, 2, "int64")):
            # flush_at = k + 1: the chunk kernels raise it to their least,
            # k plus one vector per lane
            p = dict(plan, flush_at=k + 1) if flush_at else plan
            check_case(x, dtype, n, k, sm, True, idx, plan=p, name=f"ascending k={k} {p}")


# Rows of one value: every start histogram puts the whole chunk in one bin,
# the chunk overflows the buffer, and every cut resolves the tie by column.
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("plan", [SPLIT, WHOLE])
def test_one_value_rows(dtype, plan):
    n = 3 * ce_of(dtype, plan) - 11
    f = np.full((2, n), -2.5, dtype=np.float32)
    x = _bits(f, dtype)
    for k in (1, 700, 4096):
        for sm in (0, 1, 2):
            check_case(x, dtype, n, k, sm, True, "int32", plan=plan, name=f"one value k={k} {plan}")


# Few distinct values (heavy ties in every histogram bin), including both
# zeros and -inf: starts and cuts land on tie groups and on zero.
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("plan", [SPLIT, WHOLE, {"kernel": 2}])
def test_tie_groups_and_signed_zeros(dtype, plan):
    rng = np.random.Generator(np.random.PCG64(91 + dtype))
    alpha = np.array([-0.0, 0.0, 0.5, -0.5, 1.0, -np.inf, 2.0], dtype=np.float32)
    n = 4 * ce_of(dtype, plan) + 3
    f = alpha[rng.integers(0, len(alpha), size=(3, n))]
    x = _bits(f, dtype)
    for k in (5, 512, 3000):
        for sm in (0, 1):
            check_case(x, dtype, n, k, sm, True, "int32", plan=plan, name=f"ties k={k} {plan}")


# Subnormals of both signs next to both zeros, around the k-th value: the
# kernels compare values as floats, which must order subnormals exactly (no
# flush to zero).  One and several workgroups per row.
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("plan", [SPLIT, WHOLE, {"kernel": 1}, {"kernel": 1, "segments": 3}])
def test_subnormals_around_kth(dtype, plan):
    rng = np.random.Generator(np.random.PCG64(13 + dtype))
    n = 3 * ce_of(dtype, plan)
    if dtype == FP32:
        tiny = np.array([1, 2, 3, 0x7FFFFF], dtype=np.uint32)
        sub = np.concatenate([tiny, tiny | 0x80000000]).view(np.float32)
    else:
        tiny = np.array([1, 2, 3, 0x7F], dtype=np.uint32) << 16
        sub = np.concatenate([tiny, tiny | 0x80000000]).astype(np.uint32).view(np.float32)
    pool = np.concatenate([sub, np.array([0.0, -0.0], dtype=np.float32)])
    f = pool[rng.integers(0, len(pool), size=(3, n))].astype(np.float32)
    big = rng.random((3, n)) < 0.01
    f[big] = np.float32(1.0) + rng.random(int(big.sum()), dtype=np.float32)
    x = _bits(f, dtype)
    for k in (100, 400, 1500):
        check_case(x, dtype, n, k, 1, True, "int32", plan=plan, name=f"subnormals k={k} {plan}")
        check_case(x, dtype, n, k, 0, False, "int32", plan=plan, name=f"subnormals unsorted k={k} {plan}")


# NaN in the last, partial chunk of a row (before end: flagged) and past end
# (ignored), on both layouts; end cuts rows at and near chunk boundaries.
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("plan", [SPLIT, WHOLE])
def test_ragged_ends_and_nan(dtype, plan):
    rng = np.random.Generator(np.random.PCG64(19 + dtype))
    ce = ce_of(dtype, plan)
    n = 3 * ce
    batch = 10
    f = rng.standard_normal((batch, n)).astype(np.float32)
    x = _bits(f, dtype)
    end = np.array([0, 1, ce - 1, ce, ce + 1, 2 * ce + 5, n - 1, n, 17, 2 * ce], dtype=np.int32)
    view = x.view(np.uint32) if dtype == FP32 else x
    nan = 0x7FC00000 if dtype == FP32 else 0x7FC0
    view[2, end[2] - 1] = nan          # inside: flagged
    view[3, end[3]] = nan              # just past end: ignored
    view[5, end[5] - 2] = nan          # inside the ragged chunk: flagged
    view[6, end[6]] = nan              # past end: ignored
    for k in (1, 300, 2048):
        check_case(x, dtype, n, k, 1, True, "int32", end=end, plan=plan, name=f"ends k={k} {plan}")


# A split row whose chunks hand over their exact top k (the share estimate
# would exceed k): k large against the row.
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_split_hand_over_capped_at_k(dtype):
    rng = np.random.Generator(np.random.PCG64(23 + dtype))
    n = 2 * CHUNK_ELEMS[dtype] + 100
    f = rng.standard_normal((4, n)).astype(np.float32)
    x = _bits(f, dtype)
    for k in (2048, 4096):
        check_case(x, dtype, n, k, 1, True, "int64", plan=SPLIT, name=f"capped k={k}")


# Rows whose values span about 240 octaves: a whole row's start then finds
# its m-th representative only in the widest window (every key), after the
# one-value-per-bin and the 32-octave windows hold too few.
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_wide_dynamic_range_start(dtype):
    rng = np.random.Generator(np.random.PCG64(41 + dtype))
    for n, k in ((8192, 2000), (40000, 1500), (3000, 700)):
        e = rng.uniform(-120.0, 120.0, size=(3, n))
        f = (np.exp2(e) * np.where(rng.random((3, n)) < 0.3, -1.0, 1.0)).astype(np.float32)
        x = _bits(f, dtype)
        for sm in (1, 0):
            check_case(x, dtype, n, k, sm, True, "int32", plan=WHOLE, name=f"wide range n={n} k={k}")


# The value-order epilogue's 32-bit form (bf16 rows of at most 2^16 columns):
# both zeros, negative values, -inf and heavy ties, on one and two chunks.
@pytest.mark.parametrize("n", [20000, 40000, 65536])
def test_narrow_rank_signed_zeros_and_ties(n):
    rng = np.random.Generator(np.random.PCG64(57 + n))
    alpha = np.array([-0.0, 0.0, 0.5, -0.5, 1.0, -np.inf, 2.0, -3.0], dtype=np.float32)
    f = alpha[rng.integers(0, len(alpha), size=(3, n))]
    f[1] = rng.standard_normal(n).astype(np.float32) * np.float32(0.01)   # many values near zero
    x = _bits(f, BF16)
    for k in (5, 512, 2048, 3000):
        check_case(x, BF16, n, k, 1, True, "int32", plan=WHOLE, name=f"narrow rank n={n} k={k}")
