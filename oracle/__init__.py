"""CPU oracle for row-wise TopK -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and it
shares no code with the HIP library.

``topk(x, k, ...)`` runs ``topk_oracle.cpp`` (a stable sort per row on host
memory, see that file's header for the definition and the pages it follows)
through ctypes on numpy arrays.  The shared object is built with g++ on first
use, or by :func:`build`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "topk_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

FP32, BF16 = 0, 1
ROW_NAN, ROW_BAD_END = 1, 2


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with g++ (plain C++17 + std::thread)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def open_library(path: str):
    """ctypes handle on an oracle shared object (the default one, or a variant
    compiled from an edited copy of the source by the pin-strength tests)."""
    lib = ctypes.CDLL(path)
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = open_library(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def topk(x: np.ndarray, k: int, *, dtype: int, n_cols: int | None = None, end=None,
         sorted: int = 1, return_values: bool = True, index_dtype=np.int32,
         n_threads: int = 0, library=None):
    """Top-k of every row of ``x`` (host array, shape ``[batch, row_stride]``).

    ``x`` is float32 for ``dtype=FP32`` and uint16 (bf16 bit patterns) for
    ``dtype=BF16``.  Columns ``[0, n_cols)`` are the row (``n_cols`` defaults to
    the row stride); ``end`` (int32, per row) narrows each row further.

    Returns ``(values, indices, row_status)``; ``values`` is None when
    ``return_values`` is false, else it has ``x``'s dtype and holds bit copies.
    """
    x = np.ascontiguousarray(x)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [batch, row_stride]")
    want = np.float32 if dtype == FP32 else np.uint16
    if x.dtype != want:
        raise TypeError(f"x must be {np.dtype(want).name} for dtype={dtype}")
    batch, row_stride = x.shape
    n_cols = row_stride if n_cols is None else int(n_cols)
    idx_t = np.dtype(index_dtype)
    if idx_t not in (np.dtype(np.int32), np.dtype(np.int64)):
        raise TypeError("index_dtype must be int32 or int64")
    end_a = None if end is None else np.ascontiguousarray(end, dtype=np.int32)
    if end_a is not None and end_a.shape != (batch,):
        raise ValueError("end must have shape [batch]")
    indices = np.empty((batch, k), dtype=idx_t)
    values = np.empty((batch, k), dtype=want) if return_values else None
    status = np.empty((batch,), dtype=np.int32)
    lib = _load() if library is None else library
    rc = lib.oracle_topk(
        _ptr(x), dtype, batch, n_cols, row_stride, _ptr(end_a), int(k), int(sorted),
        int(bool(return_values)), 0 if idx_t == np.dtype(np.int32) else 1,
        _ptr(values), _ptr(indices), _ptr(status), int(n_threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return values, indices, status
