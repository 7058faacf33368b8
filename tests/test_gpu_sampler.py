"""GPU parity of the sampler tail (ds_sampler_tail) with the CPU oracle.

The GPU path runs ds_topk and then ds_sampler_tail through the C ABI; the
oracle side runs the CPU top-k oracle and then oracle/sampler.py (float64) on
the same seeded inputs and uniforms.

The draw and the nucleus size are integers decided by floating point: the
kernel sums fp32 weights in a fixed order, the oracle float64 ones.  A draw
is compared exactly; where the two differ, the GPU's draw must be one that a
cumulative sum within EPS (relative to the row's total weight) of the exact
one would give, and such rows must be rare.  EPS bounds the fp32 error of a
prefix sum of at most 4096 weights in [0, 1] plus expf's: 4096 * 2^-24 plus
a few ulp, about 2.5e-4.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.sampler as S
import workloads
from tests.gpu_util import BF16, FP32, oracle_topk, say, to_device

pytestmark = pytest.mark.gpu
EPS = 3e-4


def _gpu(x_np, dtype, k, index_dtype, end, temps, uniforms):
    import torch
    import row_wise_topk_amd as rt
    xt = to_device(x_np, dtype)
    endt = None if end is None else torch.from_numpy(np.asarray(end, dtype=np.int32)).cuda()
    it = torch.int64 if index_dtype == "int64" else torch.int32
    vals, idx, st = rt.topk(xt, k, end=endt, sorted=1, return_values=True, index_dtype=it)
    u = torch.from_numpy(np.asarray(uniforms, dtype=np.float32)).cuda()
    out = []
    for tau, top_p in temps:
        tok, prob = rt.sample_from_topk(vals, idx, st, temperature=tau, top_p=top_p, uniforms=u)
        out.append((tok, prob))
    torch.cuda.synchronize()
    return [(t.cpu().numpy(), p.cpu().numpy()) for t, p in out]


def _valid_draw(vals, idx, tau, top_p, u, j, bf16):
    """Is position j a draw some cumulative sum within EPS of the exact one gives?"""
    c = S.cumulative(vals, idx, tau, bf16)
    tot = c[-1]
    m = len(c)
    k_lo = next((K for K in range(1, m + 1) if c[K - 1] >= (top_p - EPS) * tot), m)
    k_hi = next((K for K in range(1, m + 1) if c[K - 1] >= (top_p + EPS) * tot), m)
    uu = min(max(u, 0.0), 1.0)
    for K in range(k_lo, k_hi + 1):
        if j >= K:
            continue
        ck = c[K - 1]
        lo = c[j - 1] if j > 0 else 0.0
        if lo <= uu * ck + EPS * tot and c[j] >= uu * ck - EPS * tot:
            return True
    return False


def _compare(x_np, dtype, k, index_dtype, end, temps, uniforms, name, max_near=None):
    bf16 = dtype == BF16
    n_cols = x_np.shape[1]
    wv, wi, ws = oracle_topk(x_np, dtype, n_cols, k, 1, True, index_dtype, end)
    if not bf16:
        wv = wv.view(np.float32)   # the oracle returns bit patterns
    got = _gpu(x_np, dtype, k, index_dtype, end, temps, uniforms)
    batch = wi.shape[0]
    for (tau, top_p), (gt, gp) in zip(temps, got):
        tok, K, prob = S.sample(wv, wi, ws, tau, top_p, uniforms, bf16)
        near = 0
        for r in range(batch):
            if gt[r] == tok[r]:
                if tok[r] >= 0:
                    assert abs(gp[r] - prob[r]) <= 1e-4 * prob[r] + 1e-6, (name, tau, top_p, r, gp[r], prob[r])
                else:
                    assert np.isnan(gp[r])
                continue
            assert tok[r] >= 0 and gt[r] >= 0 and tau > 0, (name, tau, top_p, r, gt[r], tok[r])
            j = int(np.flatnonzero(wi[r] == gt[r])[0])
            assert _valid_draw(wv[r], wi[r], tau, top_p, float(uniforms[r]), j, bf16), \
                (name, tau, top_p, r, gt[r], tok[r])
            near += 1
        limit = max(1, batch // 32) if max_near is None else max_near
        assert near <= limit, (name, tau, top_p, near)
        say(f"{name} tau={tau} top_p={top_p}: {batch} rows, {near} draws at a rounding boundary")


def test_sampler_workload_full_size():
    w = workloads.workload(2)
    x, end = workloads.make_input(w)
    us = np.random.Generator(np.random.PCG64(21)).random(w.batch)
    temps = [(1.0, 1.0), (0.7, 0.9), (1.3, 0.5), (0.5, 0.05), (0.0, 0.9)]
    say(f"sampler tail on {w.name}")
    _compare(x, w.dtype, w.k, w.index_dtype, end, temps, us, w.name)


# k = 512 and k = 2500: two and ten candidates per lane.
@pytest.mark.parametrize("k", [512, 2500])
@pytest.mark.parametrize("dtype,index_dtype", [(FP32, "int32"), (BF16, "int64"), (BF16, "int32")])
def test_edge_rows(dtype, index_dtype, k):
    """Padding (end < k), an empty row, a NaN row, -inf and +inf candidates,
    all-equal rows, and uniforms at 0, 1 and just below 1."""
    rng = np.random.Generator(np.random.PCG64(31 + dtype))
    n = 3000
    f = (2.0 * rng.standard_normal((10, n))).astype(np.float32)
    f[3, 77] = np.nan
    f[4, :] = -np.inf
    f[4, 10:20] = 1.0
    f[5, :] = -np.inf
    f[6, [5, 900, 2000]] = np.inf
    f[7, :] = 0.25
    end = np.array([n, 100, 0, n, n, n, n, n, 600, 511], dtype=np.int32)
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    us = np.array([0.3, 0.0, 0.5, 0.5, 0.999, 0.2, 0.7, 0.61, 1.0, np.nextafter(1.0, 0.0)])
    temps = [(1.0, 1.0), (0.8, 0.9), (0.0, 0.5), (0.3, 0.2)]
    _compare(x, dtype, k, index_dtype, end, temps, us, f"edge rows {dtype} {index_dtype} k={k}", max_near=1)


def test_same_draw_on_every_call():
    import torch
    import row_wise_topk_amd as rt
    w = workloads.workload(2, batch=16)
    x, _ = workloads.make_input(w)
    xt = to_device(x, w.dtype)
    vals, idx, st = rt.topk(xt, w.k, sorted=1, index_dtype=torch.int64)
    u = torch.from_numpy(np.random.Generator(np.random.PCG64(4)).random(16).astype(np.float32)).cuda()
    first = rt.sample_from_topk(vals, idx, st, temperature=0.8, top_p=0.95, uniforms=u)
    for _ in range(20):
        t, p = rt.sample_from_topk(vals, idx, st, temperature=0.8, top_p=0.95, uniforms=u)
        assert torch.equal(t, first[0]) and torch.equal(p, first[1])
