"""Parser for ``tests/golden/hand_cases.txt`` (hand-derived TopK cases)."""
from __future__ import annotations

import os
import struct

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.txt")


def _f32(tok: str) -> float:
    return float(tok)


def load_cases():
    cases, cur = [], {}
    with open(PATH) as f:
        for raw in f:
            line = raw.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    cases.append(cur)
                    cur = {}
                continue
            key, _, val = line.partition(":")
            cur[key.strip()] = val.strip()
    if cur:
        cases.append(cur)
    out = []
    for c in cases:
        dtype = 0 if c["dtype"] == "fp32" else 1
        toks = c["x"].split()
        if dtype == 0:
            x = np.array([_f32(t) for t in toks], dtype=np.float32)
        else:
            x = np.array([int(t, 16) for t in toks], dtype=np.uint16)
        n = len(x)
        end = int(c["end"]) if "end" in c else None
        idx = np.array([int(t) for t in c["idx"].split()], dtype=np.int64)
        val = None
        if "val" in c:
            val = np.array([int(t, 16) for t in c["val"].split()], dtype=np.uint32)
        out.append(dict(name=c["name"], dtype=dtype, x=x, n=n, end=end, k=int(c["k"]),
                        sorted=int(c["sorted"]), idx=idx, val=val, status=int(c["status"])))
    return out


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]
