"""Seeded synthetic inputs shaped like the pages' TopK workloads.

This module holds input generation only -- none of the selection arithmetic --
so that the CPU oracle, the GPU parity tests and the benchmark all draw the
same rows from the same seeds.  Every generator uses numpy's
``Generator(PCG64(seed))``; bf16 rows are produced from fp32 by
round-to-nearest-even (torch's ``.to(torch.bfloat16)``) and carried as uint16
bit patterns on the host.

The five workloads (sizes, value distributions, k and options) follow the
pages' two use cases: the sampler path (fp32 logits over a vocabulary of
129,280 -- narracomm.com, "DeepSeek releases DeepSelect...", coverage
paragraph) and the Lightning Indexer path (bf16 scores, k tuned for 512, per-row
``end`` for variable-length rows -- aifluxnews.com, section
"PyTorch 接口与 CUDA 环境要求"), plus a small fp32 case and an adversarial
ascending-by-index case for the randomised block order (narracomm.com, method
paragraph).  A sixth is the pages' torch.topk pathology case: the top 1000 of
a billion floats in one row (xhh.club, "DeepSeek开源DeepSelect", section
"torch.topk 的性能痛点与版本波动"); its values are i.i.d. N(0, 1), the
plainest reading of an unstated distribution.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, replace

import numpy as np

FP32, BF16 = 0, 1


@dataclass(frozen=True)
class Workload:
    num: int              # 1..6
    name: str
    dtype: int            # FP32 / BF16
    batch: int
    n_cols: int
    row_stride: int
    k: int
    sorted: int           # 1 by value, 2 by index, 0 unsorted
    return_values: bool
    index_dtype: str      # "int32" / "int64"
    ragged: bool          # per-row end

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == FP32 else 2


WORKLOADS = {
    1: Workload(1, "fp32 4x8192 k=64", FP32, 4, 8192, 8192, 64, 1, True, "int32", False),
    2: Workload(2, "sampler fp32 64x129280 k=1024", FP32, 64, 129280, 129280, 1024, 1, True,
                "int64", False),
    3: Workload(3, "indexer decode bf16 128x131072 k=512", BF16, 128, 131072, 131072, 512, 0,
                False, "int32", False),
    4: Workload(4, "indexer prefill bf16 4096x65536 end-ramp k=2048", BF16, 4096, 65536, 65536,
                2048, 1, True, "int32", True),
    5: Workload(5, "ascending fp32 8x16777216 k=4096", FP32, 8, 16777216, 16777216, 4096, 1,
                True, "int32", False),
    6: Workload(6, "huge row fp32 1x1000000000 k=1000", FP32, 1, 1_000_000_000, 1_000_000_000,
                1000, 1, True, "int64", False),
}


def workload(num: int, **overrides) -> Workload:
    """The named workload, optionally with smaller ``batch`` / ``n_cols``."""
    w = WORKLOADS[num]
    if "n_cols" in overrides and "row_stride" not in overrides:
        n = overrides["n_cols"]
        step = 16 // w.elem_bytes
        overrides["row_stride"] = (n + step - 1) // step * step
    return replace(w, **overrides)


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) as uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def end_ramp(batch: int, n_cols: int) -> np.ndarray:
    """Causal-prefill row lengths: end[i] = min(n_cols, 512 + 16 i)."""
    return np.minimum(n_cols, 512 + 16 * np.arange(batch, dtype=np.int64)).astype(np.int32)


def make_input(w: Workload, seed: int | None = None, poison_tail: bool = False):
    """Return ``(x, end)``: host array ``[batch, row_stride]`` and int32 ends or None.

    Columns past ``n_cols`` (stride padding) are filled with NaN bit patterns,
    and with ``poison_tail`` so are columns past ``end[i]``: a correct
    implementation never reads or flags them.
    """
    rng = np.random.Generator(np.random.PCG64(w.num if seed is None else seed))
    b, n = w.batch, w.n_cols
    if w.num == 1:
        v = rng.random((b, n), dtype=np.float32) * np.float32(2) - np.float32(1)
    elif w.num == 2:
        v = np.float32(3) * rng.standard_normal((b, n), dtype=np.float32)
        spikes = min(32, n)
        for i in range(b):
            pos = rng.choice(n, spikes, replace=False)
            v[i, pos] = (12 + rng.standard_normal(spikes)).astype(np.float32)
    elif w.num == 3:
        v = rng.standard_normal((b, n), dtype=np.float32)
    elif w.num == 4:
        z = rng.standard_normal((b, n), dtype=np.float32)
        u = rng.random((b, n), dtype=np.float32) + np.float32(0.5)
        v = np.maximum(z, np.float32(0)) * u
        del z, u
    elif w.num == 5:
        ramp = (np.arange(n, dtype=np.float64) / float(1 << 24)).astype(np.float32)
        noise = np.float32(1e-3) * rng.random((b, n), dtype=np.float32)
        v = ramp[None, :] + noise
        del noise
    elif w.num == 6:
        v = rng.standard_normal((b, n), dtype=np.float32)
    else:
        raise ValueError(w.num)

    if w.dtype == BF16:
        bits = to_bf16_bits(v)
        nan_bits = np.uint16(0x7FC0)
        out = np.full((b, w.row_stride), nan_bits, dtype=np.uint16)
        out[:, :n] = bits
    elif w.row_stride == n:   # no padding: the rows as drawn (a 4 GB row is not copied)
        out = v
    else:
        out = np.full((b, w.row_stride), np.float32(np.nan), dtype=np.float32)
        out[:, :n] = v
    del v
    end = end_ramp(b, n) if w.ragged else None
    if end is not None and poison_tail:
        cols = np.arange(n)[None, :]
        mask = cols >= end[:, None]
        if w.dtype == BF16:
            out[:, :n][mask] = np.uint16(0x7FC0)
        else:
            out[:, :n][mask] = np.float32(np.nan)
    return out, end


def digest(x: np.ndarray, end=None) -> str:
    """SHA-256 of an input (and its ends), for reproducibility records."""
    h = hashlib.sha256(np.ascontiguousarray(x).view(np.uint8).reshape(-1))
    if end is not None:
        h.update(np.ascontiguousarray(end, dtype=np.int32).tobytes())
    return h.hexdigest()


def algorithmic_bytes(w: Workload, end=None) -> int:
    """Bytes the method must read: every valid element once."""
    if end is None:
        return w.batch * w.n_cols * w.elem_bytes
    return int(np.minimum(np.asarray(end, dtype=np.int64), w.n_cols).clip(min=0).sum()) * w.elem_bytes


def output_bytes(w: Workload) -> int:
    idx = 4 if w.index_dtype == "int32" else 8
    return w.batch * w.k * (idx + (w.elem_bytes if w.return_values else 0))
