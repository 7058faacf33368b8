"""Pin strength: plausible mistakes planted in copies of the oracle are caught.

Each mutant is an edited copy of ``oracle/topk_oracle.cpp`` compiled with g++
into a temporary directory (the real oracle is never touched).  A compact
battery built from the same independent pins as test_oracle.py -- the
hand-derived cases, brute-force rank counting and the invariants -- must reject
every mutant.  CPU only.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from tests.checks import as_f64, bits, brute_force_row, check_row
from tests.golden_cases import load_cases

SRC = os.path.join(os.path.dirname(oracle.__file__), "topk_oracle.cpp")

# (name, text to find, replacement) -- each a mistake someone could make
MUTANTS = [
    ("tie_to_higher_index",
     "std::iota(perm.begin(), perm.end(), int64_t{0});",
     "std::iota(perm.begin(), perm.end(), int64_t{0}); std::reverse(perm.begin(), perm.end());"),
    ("ascending_instead_of_descending",
     "return v[p] > v[q];", "return v[p] < v[q];"),
    ("nan_not_checked",
     "if (std::isnan(v[j])) has_nan = true;", ""),
    ("end_equal_to_n_cols_rejected",
     "if (L < 0 || L > a.n_cols) {", "if (L < 0 || L >= a.n_cols) {"),
    ("index_order_not_applied",
     "if (a.sorted != 1) std::sort(sel.begin(), sel.end());",
     "if (a.sorted == 0) std::sort(sel.begin(), sel.end());"),
    ("padding_value_nan",
     "fill_row(a, i, m, kNegInf);", "fill_row(a, i, m, kQNaN);"),
    ("minus_zero_below_plus_zero",
     "return static_cast<double>(f);",
     "return (f == 0.0f && std::signbit(f)) ? -1e-300 : static_cast<double>(f);"),
    ("one_too_few_selected",
     "const int64_t m = std::min<int64_t>(a.k, L);",
     "const int64_t m = std::min<int64_t>(a.k, L) - (L > 1 ? 1 : 0);"),
    ("value_from_slot_not_index",
     "put_value_bits(a, i, s, sel[s], 0);", "put_value_bits(a, i, s, s, 0);"),
    ("bf16_widened_wrong",
     "const uint32_t w = static_cast<uint32_t>(h) << 16;",
     "const uint32_t w = static_cast<uint32_t>(h) << 15;"),
    ("stride_ignored",
     "const int64_t off = i * a.row_stride + j;", "const int64_t off = i * a.n_cols + j;"),
    ("last_element_dropped",
     "for (int64_t j = 0; j < L; ++j) {", "for (int64_t j = 0; j + 1 < L; ++j) {"),
]


def _battery(lib):
    """Raises AssertionError if the library disagrees with an independent pin."""
    for c in load_cases():
        end = None if c["end"] is None else np.array([c["end"]], dtype=np.int32)
        vals, idx, st = oracle.topk(c["x"][None, :], c["k"], dtype=c["dtype"], end=end,
                                    sorted=c["sorted"], library=lib)
        assert st[0] == c["status"], c["name"]
        got = idx[0].astype(np.int64).tolist()
        want = c["idx"].tolist()
        assert (sorted(got) == sorted(want)) if c["sorted"] == 0 else (got == want), c["name"]
        if c["val"] is not None:
            assert bits(vals[0]).astype(np.uint32).tolist() == c["val"].tolist(), c["name"]
    rng = np.random.Generator(np.random.PCG64(5))
    for dtype in (0, 1):
        f = rng.integers(-3, 4, size=(40, 24)).astype(np.float32)
        f[rng.random(f.shape) < 0.2] = -0.0
        x = workloads.to_bf16_bits(f) if dtype else f
        # a wider stride whose padding is NaN: only [0, n_cols) may be read
        xs = np.full((40, 32), np.nan, dtype=np.float32)
        if dtype:
            xs = np.full((40, 32), 0x7FC0, dtype=np.uint16)
        xs[:, :24] = x
        end = rng.integers(0, 25, size=40).astype(np.int32)
        for sorted_mode in (0, 1, 2):
            for k in (1, 5, 24, 30):
                vals, idx, st = oracle.topk(xs, k, dtype=dtype, n_cols=24, end=end,
                                            sorted=sorted_mode, library=lib)
                for i in range(40):
                    L = int(end[i])
                    check_row(xs[i], L, k, dtype, sorted_mode, vals[i], idx[i], st[i])
                    want = brute_force_row(as_f64(x[i, :L], dtype), k, sorted_mode)
                    got = idx[i, :min(k, L)].astype(np.int64)
                    got = np.sort(got) if sorted_mode == 0 else got
                    assert got.tolist() == want.tolist()


def test_real_oracle_passes_battery():
    _battery(None)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[0])
def test_mutant_is_caught(mutant, tmp_path):
    name, find, repl = mutant
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"{name}.cpp"
    path.write_text(src.replace(find, repl))
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-pthread",
                           str(path), "-o", str(so)])
    lib = oracle.open_library(str(so))
    with pytest.raises(AssertionError):
        _battery(lib)
