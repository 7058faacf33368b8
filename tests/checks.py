"""Independent checks of a TopK result, written from the definition alone.

Used to pin the oracle (brute force on tiny rows, invariants on any row) and to
check GPU outputs for properties that hold at any size.  Nothing here calls the
oracle or the HIP library.

Definition (narracomm.com, "DeepSeek releases DeepSelect...", method and API
paragraphs; xhh.club Q&A on stable results): the result of a row is the k
largest valid elements; among equal values the lower index wins; NaN rows and
rows with an out-of-range end are flagged instead of answered.
"""
from __future__ import annotations

import numpy as np

FP32, BF16 = 0, 1
QNAN32, NEGINF32 = 0x7FC00000, 0xFF800000


def as_f64(row_bits_or_f32: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of fp32 values / bf16 bit patterns to float64."""
    if dtype == FP32:
        return np.asarray(row_bits_or_f32, dtype=np.float32).astype(np.float64)
    w = np.asarray(row_bits_or_f32, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a.view(np.uint16)


def brute_force_row(v: np.ndarray, k: int, sorted_mode: int):
    """Rank counting, O(L^2): rank(a) = #{b : b precedes a}."""
    L = len(v)
    if L == 0:
        return np.zeros(0, dtype=np.int64)
    a = np.arange(L)
    gt = v[None, :] > v[:, None]                       # gt[a, b]: v[b] > v[a]
    eq_lower = (v[None, :] == v[:, None]) & (a[None, :] < a[:, None])
    rank = (gt | eq_lower).sum(axis=1)
    sel = np.flatnonzero(rank < k)
    if sorted_mode == 1:
        return sel[np.argsort(rank[sel])]
    return np.sort(sel)


def check_row(x_row, L: int, k: int, dtype: int, sorted_mode: int, values_row, idx_row,
              status: int, where: str = ""):
    """Invariants of one output row against its input row (any size)."""
    v = as_f64(x_row[:L], dtype)
    if np.isnan(v).any():
        assert status == 1, f"{where}: NaN row not flagged"
        assert (np.asarray(idx_row) == -1).all(), f"{where}: NaN row indices"
        if values_row is not None:
            vb = bits(values_row).astype(np.uint32)
            want = QNAN32 if dtype == FP32 else QNAN32 >> 16
            assert (vb == want).all(), f"{where}: NaN row values"
        return
    assert status == 0, f"{where}: status {status} on a clean row"
    m = min(k, L)
    idx = np.asarray(idx_row, dtype=np.int64)
    sel, pad = idx[:m], idx[m:]
    assert (pad == -1).all(), f"{where}: padding indices"
    assert ((sel >= 0) & (sel < L)).all(), f"{where}: index out of [0, end)"
    assert len(np.unique(sel)) == m, f"{where}: duplicate indices"
    if values_row is not None:
        vb = bits(values_row)
        xb = bits(np.asarray(x_row))
        assert (vb[:m] == xb[sel]).all(), f"{where}: values are not bit copies"
        neg = NEGINF32 if dtype == FP32 else NEGINF32 >> 16
        assert (vb[m:].astype(np.uint32) == neg).all(), f"{where}: padding values"
    # min selected >= max non-selected; ties at the boundary go to lower indices
    mask = np.zeros(L, dtype=bool)
    mask[sel] = True
    if m < L:
        kth = v[sel].min()
        rest = v[~mask]
        assert kth >= rest.max(), f"{where}: a larger value was left out"
        tied_sel = np.flatnonzero(mask & (v == kth))
        tied_rest = np.flatnonzero(~mask & (v == kth))
        if len(tied_rest):
            assert tied_sel.max() < tied_rest.min(), f"{where}: tie-break by lower index"
    if sorted_mode == 1 and m > 1:
        sv = v[sel]
        ok = (sv[:-1] > sv[1:]) | ((sv[:-1] == sv[1:]) & (sel[:-1] < sel[1:]))
        assert ok.all(), f"{where}: not in value order"
    if sorted_mode == 2 and m > 1:
        assert (np.diff(sel) > 0).all(), f"{where}: not in index order"
