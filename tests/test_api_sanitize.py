"""The C ABI's host side under AddressSanitizer and UBSan, on the CPU.

tests/cpp/api_sanitize_test.cpp builds row_wise_topk_amd/csrc/topk_api.cpp
with g++ -fsanitize=address,undefined (host code only: the kernel launchers
are stubs) and drives ds_topk_validate, ds_topk_ex, ds_read_ceiling and the
workspace-size calls with 20,000 argument sets, half near their limits and
half valid for every shape class.  The stubs check that every workspace
pointer handed to a kernel lies inside the workspace the caller sized, that
validation and the call agree, and that a workspace one byte short is
refused.
"""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_api_under_sanitizers(tmp_path):
    exe = tmp_path / "api_sanitize_test"
    subprocess.check_call([
        "g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
        "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "row_wise_topk_amd", "csrc"),
        os.path.join(ROOT, "row_wise_topk_amd", "csrc", "topk_api.cpp"),
        os.path.join(ROOT, "tests", "cpp", "api_sanitize_test.cpp"), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    assert "api sanitize: ok" in out.stdout
