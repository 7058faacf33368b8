"""Helpers shared by the GPU tests: run the HIP path through the binding and
compare with the oracle element by element."""
from __future__ import annotations

import numpy as np

import oracle
from tests.build_util import ensure_built

FP32, BF16 = 0, 1
# Values per chunk of the chunk kernels: eight 16-byte loads per lane of a
# 512-lane workgroup (split rows and whole rows alike).
CHUNK_ELEMS = {FP32: 16384, BF16: 32768}
CHUNK_ELEMS_ROW = {FP32: 16384, BF16: 32768}


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def to_device(x_np: np.ndarray, dtype: int):
    import torch
    if dtype == BF16:
        return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x_np)).cuda()


def gpu_topk(x_np, dtype, n_cols, k, sorted_mode, return_values=True, index_dtype="int32",
             end=None, plan=None, xt=None):
    """Run the HIP path; returns numpy (values bits or None, indices int64, status)."""
    import torch
    ensure_built()
    import row_wise_topk_amd as rt
    if xt is None:
        xt = to_device(x_np, dtype)
    xv = xt[:, :n_cols]
    endt = None if end is None else torch.from_numpy(np.asarray(end, dtype=np.int32)).cuda()
    it = torch.int64 if index_dtype == "int64" else torch.int32
    vals, idx, st = rt.topk(xv, k, end=endt, sorted=sorted_mode, return_values=return_values,
                            index_dtype=it, plan=plan)
    torch.cuda.synchronize()
    assert idx.dtype == it
    v = None
    if return_values:
        v = vals.view(torch.int16 if dtype == BF16 else torch.int32).cpu().numpy()
        v = v.view(np.uint16 if dtype == BF16 else np.uint32)
    return v, idx.cpu().numpy().astype(np.int64), st.cpu().numpy()


def oracle_topk(x_np, dtype, n_cols, k, sorted_mode, return_values=True, index_dtype="int32",
                end=None):
    vals, idx, st = oracle.topk(x_np, k, dtype=dtype, n_cols=n_cols, end=end,
                                sorted=sorted_mode, return_values=True,
                                index_dtype=np.int64 if index_dtype == "int64" else np.int32)
    vb = vals.view(np.uint16 if dtype == BF16 else np.uint32)
    return (vb if return_values else None), idx.astype(np.int64), st


def assert_same(want, got, sorted_mode, where=""):
    """Bit-exact comparison; for unsorted output the rows are compared as sets
    (each GPU row is put in index order first, values carried along)."""
    wv, wi, ws = want
    gv, gi, gs = got
    bad = np.flatnonzero(ws != gs)
    assert bad.size == 0, f"{where}: status differs in rows {bad[:8]} ({ws[bad[:4]]} vs {gs[bad[:4]]})"
    if sorted_mode == 0:
        order = np.argsort(np.where(gi < 0, np.iinfo(np.int64).max, gi), axis=1, kind="stable")
        gi = np.take_along_axis(gi, order, axis=1)
        if gv is not None:
            gv = np.take_along_axis(gv, order, axis=1)
        worder = np.argsort(np.where(wi < 0, np.iinfo(np.int64).max, wi), axis=1, kind="stable")
        wi = np.take_along_axis(wi, worder, axis=1)
        if wv is not None:
            wv = np.take_along_axis(wv, worder, axis=1)
    rows = np.flatnonzero((wi != gi).any(axis=1))
    if rows.size:
        r = rows[0]
        j = np.flatnonzero(wi[r] != gi[r])[:6]
        raise AssertionError(f"{where}: indices differ in {rows.size} rows; row {r} slots {j}: "
                             f"want {wi[r, j]} got {gi[r, j]}")
    if wv is not None:
        assert gv is not None
        rows = np.flatnonzero((wv != gv).any(axis=1))
        if rows.size:
            r = rows[0]
            j = np.flatnonzero(wv[r] != gv[r])[:6]
            raise AssertionError(f"{where}: value bits differ in {rows.size} rows; row {r} "
                                 f"slots {j}: want {wv[r, j]} got {gv[r, j]}")


def check_case(x_np, dtype, n_cols, k, sorted_mode, return_values=True, index_dtype="int32",
               end=None, plan=None, name="", xt=None):
    say(f"{name}: dtype={'bf16' if dtype else 'fp32'} shape={x_np.shape} n_cols={n_cols} "
        f"k={k} sorted={sorted_mode} values={return_values} idx={index_dtype} "
        f"end={'yes' if end is not None else 'no'} plan={plan}")
    got = gpu_topk(x_np, dtype, n_cols, k, sorted_mode, return_values, index_dtype, end, plan, xt)
    want = oracle_topk(x_np, dtype, n_cols, k, sorted_mode, return_values, index_dtype, end)
    assert_same(want, got, sorted_mode, name)
    return got
