"""Pins of the sampler-tail oracle (oracle/sampler.py) against what the
mathematics fixes, and mutants that each pin battery must reject.  CPU only.

The oracle follows the plainest reading of the step after the sampler's TopK
(narracomm.com, "DeepSeek releases DeepSelect, a TopK kernel for sparse
attention and sampling", motive paragraph: TopK selects the candidate tokens;
deepseek-v4-pro.uk, "Inside DeepSeek V4.1's New Open Inference Toolkit": the
generation settings include temperature and top-p).  Its pins are
independent of its own code: closed forms, scipy's softmax, brute-force
prefix search and a Monte Carlo frequency check.
"""
from __future__ import annotations

import math
import types

import numpy as np
import pytest
from scipy.special import softmax

import oracle.sampler as S

SRC = S.__file__


def _row(rng, k, dup=False):
    v = np.sort(rng.standard_normal(k).astype(np.float32))[::-1].copy()
    if dup:
        v = np.round(v * 2) / 2
        v = np.sort(v)[::-1].copy()
    idx = rng.permutation(10 * k)[:k].astype(np.int64)
    return v, idx


def _battery(mod):
    """Every pin below, as one function a mutant must fail."""
    rng = np.random.Generator(np.random.PCG64(5))
    # 1. equal values: uniform over all m, draw position floor(u * m)
    for m in (1, 3, 8):
        v = np.full(m, 0.25, dtype=np.float32)
        idx = np.arange(100, 100 + m)
        for u in (0.0, 0.12, 0.5, 0.97):
            tok, K, p = mod.sample_row(v, idx, 0, 0.8, 1.0, u)
            assert K == m and tok == 100 + min(int(u * m), m - 1) and abs(p - 1.0 / m) < 1e-12
    # 2. greedy
    v, idx = _row(rng, 16)
    assert mod.sample_row(v, idx, 0, 0.0, 0.9, 0.7) == (int(idx[0]), 1, 1.0)
    # 3. two candidates, closed form
    for a, b, tau in ((1.0, 0.0, 1.0), (2.0, 1.5, 0.25), (0.0, -3.0, 2.0)):
        p0 = 1.0 / (1.0 + math.exp((b - a) / tau))
        v = np.array([a, b], dtype=np.float32)
        idx = np.array([7, 3])
        assert mod.sample_row(v, idx, 0, tau, p0 * 0.99, 0.999)[:2] == (7, 1)
        assert mod.sample_row(v, idx, 0, tau, min(1.0, p0 * 1.01 + 1e-9), p0 * 0.98)[:2] == (7, 2)
        tok, K, p = mod.sample_row(v, idx, 0, tau, 1.0, min(p0 * 1.02 + 1e-9, 0.999999))
        assert (tok, K) == (3, 2) and abs(p - (1 - p0)) < 1e-9
    # 4. scipy softmax and brute-force nucleus on random rows
    for trial in range(40):
        k = int(rng.integers(1, 40))
        v, idx = _row(rng, k, dup=trial % 3 == 0)
        tau = float(rng.uniform(0.05, 3.0))
        top_p = float(rng.uniform(0.05, 1.0))
        u = float(rng.random())
        sm = softmax(v.astype(np.float64) / tau)
        K = next(K for K in range(1, k + 1) if sum(sm[:K]) >= top_p * (1 - 1e-12)) if top_p < 1 else k
        tok, Kg, p = mod.sample_row(v, idx, 0, tau, top_p, u)
        kept = sm[:Kg] / sum(sm[:Kg])
        assert Kg == K, (Kg, K)
        j = int(np.flatnonzero(idx == tok)[0])
        assert abs(p - kept[j]) < 1e-9
        cum = np.cumsum(kept)
        assert (j == 0 or cum[j - 1] <= u + 1e-12) and u < cum[j] + 1e-12
    # 5. padding and status
    v, idx = _row(rng, 8)
    idx[5:] = -1
    for u in (0.0, 0.5, 0.999):
        tok, K, _ = mod.sample_row(v, idx, 0, 50.0, 1.0, u)
        assert tok in set(idx[:5].tolist()) and K == 5
    tok, K, p = mod.sample_row(v, idx, 1, 1.0, 1.0, 0.3)
    assert tok == -1 and K == 0 and math.isnan(p)
    assert mod.sample_row(v, np.full(8, -1), 0, 1.0, 1.0, 0.3)[0] == -1
    # 6. infinities: +inf candidates share the mass; -inf ones get none
    v = np.array([np.inf, np.inf, 3.0, -np.inf], dtype=np.float32)
    idx = np.array([4, 9, 1, 2])
    assert mod.sample_row(v, idx, 0, 1.0, 1.0, 0.25)[:2] == (4, 2)
    assert mod.sample_row(v, idx, 0, 1.0, 1.0, 0.75)[:2] == (9, 2)
    v = np.array([1.0, -np.inf, -np.inf], dtype=np.float32)
    assert mod.sample_row(v, np.array([5, 6, 7]), 0, 1.0, 1.0, 0.999)[0] == 5
    # 7. bf16 decoding: 0x3F80 is 1.0, 0x4000 is 2.0
    tok, K, p = mod.sample_row(np.array([0x4000, 0x3F80], dtype=np.uint16), np.array([1, 2]), 0,
                               1.0, 1.0, 0.0, bf16=True)
    assert tok == 1 and abs(p - 1.0 / (1.0 + math.exp(-1.0))) < 1e-9


def test_oracle_pins():
    _battery(S)


def test_monte_carlo_frequencies():
    """Drawing with many uniforms reproduces the kept, renormalised softmax."""
    v = np.array([2.0, 1.5, 1.5, 0.0, -1.0, -4.0], dtype=np.float32)
    idx = np.arange(6) + 10
    tau, top_p = 0.7, 0.9
    sm = softmax(v.astype(np.float64) / tau)
    K = next(K for K in range(1, 7) if sum(sm[:K]) >= top_p)
    p = sm[:K] / sum(sm[:K])
    n = 100_000
    us = np.random.Generator(np.random.PCG64(9)).random(n)
    toks = np.array([S.sample_row(v, idx, 0, tau, top_p, u)[0] for u in us])
    for j in range(6):
        f = np.mean(toks == 10 + j)
        want = p[j] if j < K else 0.0
        assert abs(f - want) <= 4 * math.sqrt(max(want * (1 - want), 1e-12) / n) + 1e-9, (j, f, want)


def test_batch_matches_rows():
    rng = np.random.Generator(np.random.PCG64(2))
    vals = np.stack([_row(rng, 32)[0] for _ in range(6)])
    idx = np.stack([_row(rng, 32)[1] for _ in range(6)])
    st = np.array([0, 0, 1, 0, 0, 0], dtype=np.int32)
    us = rng.random(6)
    t, K, p = S.sample(vals, idx, st, 0.9, 0.8, us)
    for r in range(6):
        assert (t[r], K[r]) == S.sample_row(vals[r], idx[r], int(st[r]), 0.9, 0.8, us[r])[:2]


MUTANTS = [
    ("nucleus_strict_vs_inclusive", "c[K - 1] < top_p * S", "c[K - 1] <= top_p * S"),
    ("temperature_multiplies", "        w = np.exp((v - top) / float(temperature))",
     "        w = np.exp((v - top) * float(temperature))"),
    ("prob_not_renormalised", "float(w[j] / CK)", "float(w[j] / S)"),
    ("draw_against_total_mass", "c[j] > uu * CK", "c[j] > uu * S"),
    ("draw_inclusive", "not (c[j] > uu * CK)", "not (c[j] >= uu * CK)"),
    ("padding_counted", "m = int(np.sum(idx >= 0))\n    if status", "m = len(idx)\n    if status"),
    ("status_ignored", "if status != 0 or m == 0:", "if m == 0:"),
    ("greedy_takes_last", "return int(idx[0]), 1, 1.0", "return int(idx[m - 1]), 1, 1.0"),
    ("inf_not_special", "if math.isinf(top):\n        w = (v == top)", "if False:\n        w = (v == top)"),
    ("bf16_low_half", "values.astype(np.uint32) << 16", "values.astype(np.uint32)"),
]


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, name
    mod = types.ModuleType(f"mutant_{name}")
    exec(compile(src.replace(find, repl), f"<mutant {name}>", "exec"), mod.__dict__)
    with pytest.raises(Exception):
        _battery(mod)
