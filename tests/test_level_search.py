"""The radix-select level arithmetic of the streaming kernel's cuts, on the CPU.

The kernel's two level loops (the key search of a cut and its column search)
narrow a 32-bit range with RangeLevel (row_wise_topk_amd/csrc/level_search.h).
The C++ driver under tests/cpp checks, with g++, that a loop driven by real
histograms finds the right value within three levels, and that a loop fed
counts no buffer can produce (the case that could once spin forever) still
ends within three levels without leaving its range.
"""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_level_search_terminates_and_finds(tmp_path):
    exe = tmp_path / "level_search_test"
    subprocess.check_call(["g++", "-O2", "-std=c++17",
                           "-I" + os.path.join(ROOT, "row_wise_topk_amd", "csrc"),
                           os.path.join(ROOT, "tests", "cpp", "level_search_test.cpp"),
                           "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "level search: ok" in out.stdout
