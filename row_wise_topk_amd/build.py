"""Build ``libdstopk.so`` (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdstopk.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed fp32 instructions disabled.  No fast-math
# and no denormal-flush option: the kernels compare values as floats, and
# subnormals must order exactly (the default keeps them).
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    extra = list(extra or [])
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    k_obj = os.path.join(bdir, "topk_kernels.o")
    c_obj = os.path.join(bdir, "chunk_kernels_row.o")
    c2_obj = os.path.join(bdir, "chunk_kernels_split.o")
    a_obj = os.path.join(bdir, "topk_api.o")
    n_obj = os.path.join(bdir, "noalloc.o")
    _run([HIPCC, *COMMON, *DEVICE, *extra, "-c", os.path.join(CSRC, "topk_kernels.hip"),
          "-o", k_obj], verbose)
    # The chunk kernels twice: whole rows and split rows.
    _run([HIPCC, *COMMON, *DEVICE, *extra, "-DCHUNK_SPLIT=0", "-c",
          os.path.join(CSRC, "chunk_kernels.hip"), "-o", c_obj], verbose)
    _run([HIPCC, *COMMON, *DEVICE, *extra, "-DCHUNK_SPLIT=1", "-c",
          os.path.join(CSRC, "chunk_kernels.hip"), "-o", c2_obj], verbose)
    _run([HIPCC, *COMMON, *DEVICE, *extra, "-x", "hip", "-c", os.path.join(CSRC, "topk_api.cpp"),
          "-o", a_obj], verbose)
    _run([HIPCC, *COMMON, *DEVICE, *extra, "-c", os.path.join(CSRC, "noalloc.hip"), "-o", n_obj],
         verbose)
    s_obj = os.path.join(bdir, "sampler_tail.o")
    _run([HIPCC, *COMMON, *DEVICE, *extra, "-c", os.path.join(CSRC, "sampler_tail.hip"), "-o", s_obj],
         verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", k_obj, c_obj, c2_obj, a_obj, n_obj, s_obj, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
