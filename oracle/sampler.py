"""CPU oracle for the sampler tail after TopK -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The HIP library never calls it and it
shares no code with the HIP library.

What it computes.  narracomm.com, "DeepSeek releases DeepSelect, a TopK
kernel for sparse attention and sampling" (motive paragraph) says that
during sampling TopK selects the candidate tokens from a large vocabulary;
the generation settings around it include a temperature and a top-p
(deepseek-v4-pro.uk, "Inside DeepSeek V4.1's New Open Inference Toolkit",
the recipe section that lists the generation settings).  The pages stop
there; this oracle takes the plainest reading of the step that follows the
TopK, written out in float64 on one row at a time:

  1. The candidates are the row's top-k output in order: values v[0..m) sorted
     by value (larger first, ties by lower index) and their indices; entries
     whose index is negative (the padding of a row shorter than k) are not
     candidates.  A row with a status bit set (a NaN row) draws nothing.
  2. Temperature tau > 0: weight w_j = exp((v_j - v_0) / tau), v_0 the largest
     value.  If v_0 is infinite, w_j = 1 where v_j == v_0, else 0 (the limit of
     the same formula).  tau <= 0 means greedy: the first candidate.
  3. Top-p (nucleus): with c_j = w_0 + ... + w_j and S = c_{m-1}, keep the
     smallest prefix of K candidates with c_{K-1} >= top_p * S (K >= 1;
     top_p >= 1 keeps every candidate of non-zero weight).
  4. Draw with a caller-supplied uniform u in [0, 1): the first j < K with
     c_j > u * c_{K-1}.  The token is index[j]; its probability after the
     cut is w_j / c_{K-1}.

Outputs per row: token (int64; -1 when the row draws nothing), the kept count
K (0 when nothing is drawn), and the probability (NaN when nothing is drawn).
"""
from __future__ import annotations

import math

import numpy as np


def _row_values(values: np.ndarray, bf16: bool) -> np.ndarray:
    """Values of a row as float64 (bf16 given as uint16 bit patterns)."""
    if bf16:
        return (values.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(values, dtype=np.float32).astype(np.float64)


def sample_row(values, indices, status: int, temperature: float, top_p: float, u: float,
               bf16: bool = False):
    """One row of the sampler tail: (token, kept count K, probability)."""
    idx = np.asarray(indices, dtype=np.int64)
    v = _row_values(np.asarray(values), bf16)
    m = int(np.sum(idx >= 0))
    if status != 0 or m == 0:
        return -1, 0, math.nan
    v = v[:m]
    if temperature <= 0.0:
        return int(idx[0]), 1, 1.0
    top = v[0]
    if math.isinf(top):
        w = (v == top).astype(np.float64)
    else:
        w = np.exp((v - top) / float(temperature))
    c = np.cumsum(w)
    S = c[-1]
    K = 1
    while K < m and c[K - 1] < top_p * S:
        K += 1
    CK = c[K - 1]
    uu = min(max(float(u), 0.0), 1.0)
    j = 0
    while j < K - 1 and not (c[j] > uu * CK):
        j += 1
    return int(idx[j]), K, float(w[j] / CK)


def sample(values, indices, status, temperature: float, top_p: float, uniforms,
           bf16: bool = False):
    """The sampler tail over a batch: arrays (tokens int64, kept int32, probs float64)."""
    values = np.asarray(values)
    indices = np.asarray(indices)
    batch = indices.shape[0]
    status = np.zeros(batch, dtype=np.int32) if status is None else np.asarray(status)
    tokens = np.empty(batch, dtype=np.int64)
    kept = np.empty(batch, dtype=np.int32)
    probs = np.empty(batch, dtype=np.float64)
    for r in range(batch):
        tokens[r], kept[r], probs[r] = sample_row(values[r], indices[r], int(status[r]),
                                                  temperature, top_p, float(uniforms[r]), bf16)
    return tokens, kept, probs


def cumulative(values, indices, temperature: float, bf16: bool = False) -> np.ndarray:
    """c_j of step 3 for one row (float64), for tests that check a draw lying
    within rounding distance of a boundary."""
    idx = np.asarray(indices, dtype=np.int64)
    m = int(np.sum(idx >= 0))
    v = _row_values(np.asarray(values), bf16)[:m]
    top = v[0]
    w = (v == top).astype(np.float64) if math.isinf(top) else np.exp((v - top) / float(temperature))
    return np.cumsum(w)
