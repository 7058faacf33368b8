"""Benchmark: row-wise TopK on one MI355X, one JSON line on stdout.

A step is one ds_topk call (one kernel launch: stream, cut, merge, epilogue)
over one batch of the sampler workload (fp32 logits 64 x 129,280, k = 1024,
sorted by value, values and int64 indices).  Inputs are resident in HBM before
timing starts and rotate over enough copies that every call reads cold from
HBM rather than from the 256 MB Infinity Cache.

value        effective GB/s = valid input bytes / (timed wall time / steps),
             the pages' metric (effective memory bandwidth).
roofline     the kernel's own average duration from HIP events around every
             launch, against MI355X's 8 TB/s HBM peak; traffic (FETCH_SIZE /
             WRITE_SIZE per launch) comes from the committed rocprofv3 counter
             summary when the kernel source still matches it.
cpu_baseline the CPU oracle (full stable sort per row) on the host cores.
read_ceiling the same input bytes read by a kernel with the same grid, block
             order and loads that does nothing else (ds_read_ceiling): the
             achievable ceiling of this access pattern, and value's fraction
             of it.
return_values_ab
             µs per call with and without the values output (the pages note
             that skipping the values is faster).

  python bench.py [--steps K] [--warmup W] [--config N] [--no-cpu]
  python bench.py --calibrate-copy ...        also run a plain 256 MiB copy first
                                              (the counter calibration kernel)
  python bench.py --traffic-from FETCH_DIR WRITE_DIR [--config N]
                                              write profiles/traffic.json from two
                                              rocprofv3 --pmc runs (no GPU needed)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s and µs/call for row-wise TopK (bf16 k=512, fp32 k=1024)"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
KERNEL_SRCS = [os.path.join(ROOT, "row_wise_topk_amd", "csrc", f)
               for f in ("topk_kernels.hip", "topk_api.cpp", "topk_internal.h")]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_ELEMS = 64 << 20          # calibration copy: 64 Mi fp32 = 256 MiB read, 256 MiB written


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2, help="workload number (2 = sampler)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-torch", action="store_true", help="skip the torch.topk context timing")
    p.add_argument("--segments", type=int, default=0,
                   help="workgroups per row (0 = the library's automatic plan)")
    p.add_argument("--kernel", type=int, default=0,
                   help="0 automatic, 1 the streaming kernel, 2 the chunk kernels")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run a plain elementwise copy of known size before the TopK calls")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc output folders into profiles/traffic.json")
    return p.parse_args()


def _kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def _traffic(workload_name: str):
    """Per-launch HBM bytes from the committed counter summary, if current."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        data = json.load(open(TRAFFIC_JSON))
        rec = data.get(workload_name)
        if not rec or rec.get("kernel_sha256_16") != _kernel_hash():
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def _pmc_rows(folder: str, counter: str):
    """(kernel name, value in KiB) for every dispatch in a rocprofv3 --pmc CSV."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {folder}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def _write_traffic(args):
    """FETCH_SIZE / WRITE_SIZE per TopK launch, scaled by the copy kernel's reading."""
    import workloads
    w = workloads.workload(args.config)
    copy_bytes = COPY_ELEMS * 4
    out = {}
    for counter, folder in (("FETCH_SIZE", args.traffic_from[0]), ("WRITE_SIZE", args.traffic_from[1])):
        rows = _pmc_rows(folder, counter)
        cp = [v for n, v in rows if "neg" in n.lower()]
        tk = [v for n, v in rows if "topk_kernel" in n]
        if not cp or not tk:
            raise SystemExit(f"{counter}: copy dispatches {len(cp)}, topk dispatches {len(tk)}")
        cp_kib = sorted(cp)[len(cp) // 2]
        tk_kib = sum(tk) / len(tk)
        factor = copy_bytes / (cp_kib * 1024.0)
        out[counter] = {"topk_kib_per_dispatch": round(tk_kib, 1), "topk_dispatches": len(tk),
                        "copy_kib_per_dispatch": round(cp_kib, 1), "copy_bytes": copy_bytes,
                        "scale": round(factor, 4), "bytes_per_launch": int(tk_kib * 1024.0 * factor)}
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    fetch, write = out["FETCH_SIZE"]["bytes_per_launch"], out["WRITE_SIZE"]["bytes_per_launch"]
    data[w.name] = {
        "kernel_sha256_16": _kernel_hash(),
        "bytes_per_launch": fetch + write,
        "fetch_bytes": fetch,
        "write_bytes": write,
        "algorithmic_input_bytes": workloads.algorithmic_bytes(w, workloads.end_ramp(w.batch, w.n_cols) if w.ragged else None),
        "output_bytes": workloads.output_bytes(w),
        "counters": out,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -- python3 bench.py --config {w.num} --steps 5 --warmup 2 --no-cpu --no-torch --calibrate-copy",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -- python3 bench.py --config {w.num} --steps 5 --warmup 2 --no-cpu --no-torch --calibrate-copy",
            f"python3 bench.py --config {w.num} --traffic-from <FETCH_DIR> <WRITE_DIR>",
        ],
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[w.name]))


def main():
    args = _parse()
    if args.traffic_from:
        _write_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows shard across GPUs without any exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from tests.build_util import ensure_built
    ensure_built()
    import row_wise_topk_amd as rt

    w = workloads.workload(args.config)
    x_np, end_np = workloads.make_input(w)
    alg_bytes = workloads.algorithmic_bytes(w, end_np)
    out_bytes = workloads.output_bytes(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    copy_bytes = x_np.nbytes
    n_copies = max(2, math.ceil(2 * MALL_BYTES / copy_bytes))
    if w.dtype == workloads.BF16:
        base = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        base = torch.from_numpy(x_np).to(dev)
    copies = [base] + [base.clone() for _ in range(n_copies - 1)]
    views = [c[:, : w.n_cols] for c in copies]
    end_t = None if end_np is None else torch.from_numpy(end_np).to(dev)
    it = torch.int64 if w.index_dtype == "int64" else torch.int32
    values = torch.empty((w.batch, w.k), dtype=base.dtype, device=dev) if w.return_values else None
    indices = torch.empty((w.batch, w.k), dtype=it, device=dev)
    status = torch.empty((w.batch,), dtype=torch.int32, device=dev)
    out = (values, indices, status)

    plan = (rt.Plan(segments=args.segments, perm_seed=0x5EED, kernel=args.kernel)
            if (args.segments or args.kernel) else None)

    def call(i):
        rt.topk(views[i % n_copies], w.k, end=end_t, sorted=w.sorted,
                return_values=w.return_values, index_dtype=it, out=out, plan=plan)

    if args.calibrate_copy:
        src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    assert int(status.abs().sum().item()) == 0, "row status set on clean input"

    # Whole-job timing: K back-to-back calls, synchronised on both sides.
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        call(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # Kernel duration: events around every launch, on the launch stream.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        call(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    kernel_ms = sum(per) / len(per)
    kernel_med_ms = per[len(per) // 2]

    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = _traffic(w.name)

    def timed(fn, reps):
        for i in range(min(args.warmup, 5)):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    # Read ceiling: the same bytes, blocks, workgroups and loads, and nothing else.
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    ceil_us = timed(lambda i: rt.read_ceiling(views[i % n_copies], w.k, end=end_t, plan=plan,
                                              sink=sink), args.steps)
    ceil_gbps = alg_bytes / (ceil_us * 1e-6) / 1e9

    # The same calls with the values output switched the other way.
    alt = not w.return_values
    alt_vals = torch.empty((w.batch, w.k), dtype=base.dtype, device=dev) if alt else None
    alt_us = timed(lambda i: rt.topk(views[i % n_copies], w.k, end=end_t, sorted=w.sorted,
                                     return_values=alt, index_dtype=it,
                                     out=(alt_vals, indices, status), plan=plan), args.steps)
    us_call = ms_per_step * 1e3
    ab = {"with_values_us": round(alt_us if alt else us_call, 3),
          "without_values_us": round(us_call if alt else alt_us, 3)}

    torch_us = None
    if not args.no_torch:
        xs = views[0]
        for _ in range(3):
            torch.topk(xs, w.k, dim=1, sorted=True)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        a.record(stream)
        for i in range(reps):
            torch.topk(views[i % n_copies], w.k, dim=1, sorted=True)
        b.record(stream)
        torch.cuda.synchronize()
        torch_us = a.elapsed_time(b) * 1e3 / reps

    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        used = min(cores, w.batch)
        idx_np = np.int64 if w.index_dtype == "int64" else np.int32
        # The oracle sorts every row whole: a row longer than 2^24 elements is
        # timed on its first 2^24 columns instead (a bounded sample).
        cols = min(w.n_cols, 1 << 24)
        s_bytes = alg_bytes if cols == w.n_cols else w.batch * cols * w.elem_bytes
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.topk(x_np, w.k, dtype=w.dtype, n_cols=cols, end=end_np, sorted=w.sorted,
                        return_values=w.return_values, index_dtype=idx_np, n_threads=used)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or reps >= 1000:
                break
        what = (f"the full workload ({w.batch} rows)" if cols == w.n_cols
                else f"the first {cols} columns of each of the {w.batch} rows")
        cpu = {"value": round(s_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": used,
               "kind": "oracle",
               "sample": f"{what}, {reps} repetitions in "
                         f"{el:.1f} s, {used} threads, one row per thread at a time"}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == workloads.FP32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_cols": w.n_cols,
                   "row_stride": w.row_stride, "k": w.k, "sorted": w.sorted,
                   "return_values": w.return_values, "index_dtype": w.index_dtype,
                   "input_copies": n_copies, "input_sha256": workloads.digest(x_np, end_np)[:16],
                   "segments": args.segments or "auto"},
        "us_per_call": round(ms_per_step * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel_us_mean": round(kernel_ms * 1e3, 3),
                     "kernel_us_median": round(kernel_med_ms * 1e3, 3),
                     "algorithmic_bytes": alg_bytes},
        "read_ceiling": {"us_per_call": round(ceil_us, 3), "GBps": round(ceil_gbps, 2),
                         "frac_of_ceiling": round(value / ceil_gbps, 4)},
        "return_values_ab": ab,
        "effective_GBps_with_outputs": round((alg_bytes + out_bytes) / (ms_per_step * 1e-3) / 1e9, 2),
        "torch_topk_us": None if torch_us is None else round(torch_us, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
