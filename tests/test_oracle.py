"""Pins of the CPU oracle against things other than itself (CPU only).

* hand-derived cases (tests/golden/hand_cases.txt);
* brute-force rank counting on tiny rows, random and exhaustive over a small
  alphabet with -inf, -0.0, +0.0 and +inf;
* numpy's stable argsort (a different library routine from the oracle's
  std::stable_sort) and torch.topk's value multiset on the workload shapes;
* closed forms (all-equal, strictly increasing / decreasing rows, short rows,
  the noise-free ascending workload);
* invariants on every output row (tests/checks.py).

The definition pinned here: the k largest valid elements, value descending then
lower index (narracomm.com, "DeepSeek releases DeepSelect...", method and API
paragraphs; xhh.club Q&A on stable results).
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle
import workloads
from tests.checks import as_f64, bits, brute_force_row, check_row
from tests.golden_cases import load_cases

FP32, BF16 = 0, 1


# ---------------------------------------------------------------- golden
@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    x = case["x"][None, :]
    end = None if case["end"] is None else np.array([case["end"]], dtype=np.int32)
    vals, idx, st = oracle.topk(x, case["k"], dtype=case["dtype"], end=end, sorted=case["sorted"])
    assert st[0] == case["status"]
    got = idx[0].astype(np.int64)
    if case["sorted"] == 0:
        assert sorted(got.tolist()) == sorted(case["idx"].tolist())
    else:
        assert got.tolist() == case["idx"].tolist()
    if case["val"] is not None:
        assert bits(vals[0]).astype(np.uint32).tolist() == case["val"].tolist()


# ---------------------------------------------------------------- brute force
def _rows_with_ties(rng, batch, n, dtype):
    # few distinct values -> many ties; sprinkle -0.0/+0.0 and infinities
    alphabet = np.array([-np.inf, -2.5, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0, np.inf], dtype=np.float32)
    x = alphabet[rng.integers(0, len(alphabet), size=(batch, n))]
    noise = rng.random((batch, n)) < 0.3
    x[noise] = rng.standard_normal(int(noise.sum())).astype(np.float32)
    if dtype == BF16:
        return workloads.to_bf16_bits(x)
    return x


@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("sorted_mode", [0, 1, 2])
def test_brute_force_random(dtype, sorted_mode):
    rng = np.random.Generator(np.random.PCG64(100 + 3 * dtype + sorted_mode))
    batch, n = 300, 40
    x = _rows_with_ties(rng, batch, n, dtype)
    end = rng.integers(0, n + 1, size=batch).astype(np.int32)
    for k in (1, 2, 7, 16, 40, 57):
        for idx_t in (np.int32, np.int64):
            vals, idx, st = oracle.topk(x, k, dtype=dtype, end=end, sorted=sorted_mode,
                                        index_dtype=idx_t)
            assert (st == 0).all()
            for i in range(batch):
                L = int(end[i])
                want = brute_force_row(as_f64(x[i, :L], dtype), k, sorted_mode)
                got = idx[i, :min(k, L)].astype(np.int64)
                if sorted_mode == 0:
                    got = np.sort(got)
                assert got.tolist() == want.tolist(), (i, k)
                check_row(x[i], L, k, dtype, sorted_mode, vals[i], idx[i], st[i], f"row {i}")


def _alphabet_rows(dtype, L):
    alpha = np.array([-np.inf, -1.5, -0.0, 0.0, 1.5, np.inf], dtype=np.float32)
    combos = np.array(list(itertools.product(range(len(alpha)), repeat=L)), dtype=np.int64)
    x = alpha[combos]
    if dtype == BF16:
        x = workloads.to_bf16_bits(x)
    return x


def _brute_rank(v):
    """Vectorised rank over many rows: rank[r, a] = #{b : b precedes a}."""
    L = v.shape[1]
    a = np.arange(L)
    gt = v[:, None, :] > v[:, :, None]
    eq_lower = (v[:, None, :] == v[:, :, None]) & (a[None, None, :] < a[None, :, None])
    return (gt | eq_lower).sum(axis=2)


@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("L", [1, 2, 3, 4, 5, 6])
def test_exhaustive_alphabet(dtype, L):
    x = _alphabet_rows(dtype, L)
    v = as_f64(x, dtype)
    rank = _brute_rank(v)
    for k in range(1, 9):
        for sorted_mode in (0, 1, 2):
            vals, idx, st = oracle.topk(x, k, dtype=dtype, sorted=sorted_mode)
            assert (st == 0).all()
            m = min(k, L)
            got = idx[:, :m].astype(np.int64)
            if sorted_mode == 1:
                # slot j holds the element of rank j
                want = np.argsort(rank, axis=1, kind="stable")[:, :m]
                assert (got == want).all()
            else:
                chosen = rank < k
                want_mask = np.zeros_like(chosen)
                np.put_along_axis(want_mask, got, True, axis=1)
                assert (want_mask == chosen).all()
                if sorted_mode == 2:
                    assert (np.diff(got, axis=1) > 0).all()
            assert (idx[:, m:] == -1).all()
            xb = bits(x)
            assert (bits(vals)[:, :m] == np.take_along_axis(xb, got, axis=1)).all()


def test_exhaustive_alphabet_length7_fp32():
    x = _alphabet_rows(FP32, 7)
    rank = _brute_rank(as_f64(x, FP32))
    for k in (1, 3, 4, 7, 8):
        _, idx, _ = oracle.topk(x, k, dtype=FP32, sorted=1)
        m = min(k, 7)
        want = np.argsort(rank, axis=1, kind="stable")[:, :m]
        assert (idx[:, :m] == want).all()


# ---------------------------------------------------------------- NaN / end
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_nan_rows_and_poison_past_end(dtype):
    rng = np.random.Generator(np.random.PCG64(7))
    batch, n = 64, 200
    f = rng.standard_normal((batch, n)).astype(np.float32)
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    end = rng.integers(0, n + 1, size=batch).astype(np.int32)
    nan_patterns32 = [0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF, 0x7FBFFFFF]
    nan_patterns16 = [0x7FC0, 0xFFC0, 0x7F81, 0xFFFF]
    want_flag = np.zeros(batch, dtype=bool)
    for i in range(batch):
        kind = i % 4
        if kind == 0 and end[i] > 0:      # NaN inside the row
            j = rng.integers(0, end[i])
            want_flag[i] = True
        elif kind == 1 and end[i] < n:    # NaN past end: must be ignored
            j = rng.integers(end[i], n)
        else:
            continue
        if dtype == FP32:
            x.view(np.uint32)[i, j] = nan_patterns32[i % len(nan_patterns32)]
        else:
            x[i, j] = nan_patterns16[i % len(nan_patterns16)]
    vals, idx, st = oracle.topk(x, 16, dtype=dtype, end=end, sorted=1)
    assert ((st == 1) == want_flag).all()
    for i in range(batch):
        check_row(x[i], int(end[i]), 16, dtype, 1, vals[i], idx[i], st[i], f"row {i}")


def test_bad_end_flagged():
    x = np.arange(12, dtype=np.float32).reshape(3, 4)
    end = np.array([5, -2, 4], dtype=np.int32)
    vals, idx, st = oracle.topk(x, 2, dtype=FP32, end=end)
    assert st.tolist() == [2, 2, 0]
    assert (idx[:2] == -1).all() and (bits(vals[:2]) == 0x7FC00000).all()
    assert idx[2].tolist() == [3, 2]


def test_n_cols_narrower_than_stride():
    x = np.full((2, 8), np.nan, dtype=np.float32)
    x[:, :5] = [[1, 5, 2, 4, 3], [0, 0, 0, 0, 0]]
    vals, idx, st = oracle.topk(x, 3, dtype=FP32, n_cols=5)
    assert (st == 0).all()
    assert idx.tolist() == [[1, 3, 4], [0, 1, 2]]


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_closed_forms(dtype):
    # integers 0..255 are exact in bf16 (8 significant bits) and in fp32
    n, k = (1000, 37) if dtype == FP32 else (256, 37)
    inc = np.arange(n, dtype=np.float32)
    x32 = np.stack([inc, inc[::-1].copy(), np.full(n, 2.5, np.float32)])
    x = workloads.to_bf16_bits(x32) if dtype == BF16 else x32
    _, idx, st = oracle.topk(x, k, dtype=dtype, sorted=1)
    assert (st == 0).all()
    assert idx[0].tolist() == list(range(n - 1, n - 1 - k, -1))   # strictly increasing
    assert idx[1].tolist() == list(range(k))                      # strictly decreasing
    assert idx[2].tolist() == list(range(k))                      # all equal
    _, idx, _ = oracle.topk(x, k, dtype=dtype, sorted=2)
    assert idx[0].tolist() == list(range(n - k, n))
    # L <= k: every index, then padding
    _, idx2, _ = oracle.topk(x[:, :10].copy(), 16, dtype=dtype, sorted=2)
    assert (idx2[:, :10] == np.arange(10)).all() and (idx2[:, 10:] == -1).all()


def test_noise_free_ascending_closed_form():
    n, k = 1 << 16, 4096
    x = (np.arange(n, dtype=np.float64) / float(1 << 24)).astype(np.float32)[None, :]
    vals, idx, st = oracle.topk(x, k, dtype=FP32, sorted=1)
    assert idx[0].tolist() == list(range(n - 1, n - 1 - k, -1))
    assert (vals[0] == x[0, n - 1:n - 1 - k:-1]).all()


# ---------------------------------------------------------------- workloads
def _numpy_reference_indices(x, dtype, L, k, sorted_mode):
    v = as_f64(x[:L], dtype)
    order = np.argsort(-v, kind="stable")[:k]     # -(+0) == -(-0): ties keep index order
    if sorted_mode != 1:
        order = np.sort(order)
    return order


@pytest.mark.parametrize("num,shape", [
    (1, {}),
    (2, {"batch": 6}),
    (3, {"batch": 6}),
    (4, {"batch": 300, "n_cols": 8192}),
    (5, {"batch": 2, "n_cols": 1 << 20}),
])
def test_workloads_vs_numpy_and_torch(num, shape):
    import torch
    w = workloads.workload(num, **shape)
    x, end = workloads.make_input(w, poison_tail=True)
    idx_t = np.int64 if w.index_dtype == "int64" else np.int32
    vals, idx, st = oracle.topk(x, w.k, dtype=w.dtype, n_cols=w.n_cols, end=end,
                                sorted=w.sorted, return_values=True, index_dtype=idx_t)
    assert (st == 0).all()
    for i in range(w.batch):
        L = w.n_cols if end is None else int(end[i])
        m = min(w.k, L)
        want = _numpy_reference_indices(x[i], w.dtype, L, w.k, w.sorted)
        got = idx[i, :m].astype(np.int64)
        if w.sorted == 0:
            got = np.sort(got)
        assert got.tolist() == want.tolist(), f"row {i}"
        check_row(x[i], L, w.k, w.dtype, w.sorted, vals[i], idx[i], st[i], f"row {i}")
        # value multiset against torch.topk (numeric, ties resolved any way)
        tv = torch.from_numpy(as_f64(x[i, :L], w.dtype))
        top = torch.topk(tv, m, sorted=True).values.numpy()
        mine = np.sort(as_f64(vals[i, :m], w.dtype))[::-1]
        assert np.array_equal(top, mine), f"row {i}"


def test_k1_is_first_argmax():
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.integers(-3, 4, size=(500, 33)).astype(np.float32)
    _, idx, _ = oracle.topk(x, 1, dtype=FP32)
    assert (idx[:, 0] == np.argmax(x, axis=1)).all()


def test_threads_do_not_change_result():
    w = workloads.workload(3, batch=16, n_cols=4096)
    x, _ = workloads.make_input(w)
    a = oracle.topk(x, w.k, dtype=w.dtype, sorted=1, n_threads=1)
    b = oracle.topk(x, w.k, dtype=w.dtype, sorted=1, n_threads=7)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
