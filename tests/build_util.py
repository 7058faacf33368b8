"""Build the HIP library for the tests only when nothing is built yet."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "row_wise_topk_amd", "libdstopk.so")


def ensure_built():
    if os.path.exists(LIB):
        return
    spec = importlib.util.spec_from_file_location(
        "_dstopk_build", os.path.join(ROOT, "row_wise_topk_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build()
