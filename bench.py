"""Benchmark: row-wise TopK on one MI355X, one JSON line on stdout.

A step is one ds_topk call on each of the two workloads the metric is quoted
on, back to back on one stream:

  sampler          fp32 logits 64 x 129,280, k = 1024, sorted by value,
                   values and int64 indices;
  indexer decode   bf16 scores 128 x 131,072, k = 512, unsorted, int32
                   indices only.

Inputs are resident in HBM before timing starts and rotate over enough copies
that every call reads cold from HBM rather than from the 256 MB Infinity
Cache.  The K timed steps are captured once into a HIP graph and replayed, so
the figures are the GPU's, not Python's launch overhead (the eager per-call
times are reported beside them).  Every replay's outputs are checked against
the eager call's.

value        effective GB/s of a step = valid input bytes of both workloads /
             (timed time / steps), the pages' metric (effective bandwidth).
workloads    per workload: µs per call, effective GB/s, its kernel's roofline
             and read ceiling.
roofline     the dominant kernel (the workload whose call takes longer):
             algorithmic bytes per launch / its average duration (a graph of
             K launches of that workload alone, timed with HIP events on the
             launch stream), against MI355X's 8 TB/s HBM peak; traffic
             (FETCH_SIZE + WRITE_SIZE per launch) comes from the committed
             rocprofv3 counter summary when the kernel sources still match it.
cpu_baseline the CPU oracle (full stable sort per row) on the host cores, on a
             bounded sample of each workload.
read_ceiling the same input bytes read by a kernel with the same grid, chunk
             order and loads that does nothing else (ds_read_ceiling).
sampler_tail the sampling step after the sampler's TopK (ds_sampler_tail:
             temperature softmax, nucleus cut, draw) on that call's outputs.

  python bench.py [--steps K] [--warmup W] [--config N] [--no-cpu]
       --config 0 (default) both workloads; N alone: that workload only
  python bench.py --calibrate-copy ...        also run a plain 256 MiB copy first
                                              (the counter calibration kernel)
  python bench.py --traffic-from FETCH_DIR WRITE_DIR --config N
                                              write profiles/traffic.json from two
                                              rocprofv3 --pmc runs (no GPU needed)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s and µs/call for row-wise TopK (bf16 k=512, fp32 k=1024)"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
HEADLINE = (2, 3)              # sampler fp32 k=1024, indexer decode bf16 k=512
KERNEL_SRCS = [os.path.join(ROOT, "row_wise_topk_amd", "csrc", f)
               for f in ("topk_kernels.hip", "chunk_kernels.hip", "topk_api.cpp",
                         "topk_internal.h", "level_search.h")]
# Names of the selection kernels in a profile (the read-ceiling kernels,
# chunk_read_kernel and read_kernel, are not among them).
TOPK_KERNEL_NAMES = ("topk_kernel", "chunk_split_kernel", "chunk_row_kernel")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_ELEMS = 64 << 20          # calibration copy: 64 Mi fp32 = 256 MiB read, 256 MiB written


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=0,
                   help="workload number; 0 = the sampler and indexer-decode workloads together")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="CPU-oracle seconds per workload")
    p.add_argument("--no-torch", action="store_true", help="skip the torch.topk context timing")
    p.add_argument("--no-graph", action="store_true",
                   help="time eager launches only (for profilers that do not follow graphs)")
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
    if not args.config:
        raise SystemExit("--traffic-from needs --config N (one workload per pair of runs)")
    w = workloads.workload(args.config)
    copy_bytes = COPY_ELEMS * 4
    out = {}
    names = set()
    for counter, folder in (("FETCH_SIZE", args.traffic_from[0]), ("WRITE_SIZE", args.traffic_from[1])):
        rows = _pmc_rows(folder, counter)
        cp = [v for n, v in rows if "neg" in n.lower()]
        tk = [(n, v) for n, v in rows if any(s in n for s in TOPK_KERNEL_NAMES)]
        if not cp or not tk:
            raise SystemExit(f"{counter}: copy dispatches {len(cp)}, topk dispatches {len(tk)}")
        names.update(n for n, _ in tk)
        cp_kib = sorted(cp)[len(cp) // 2]
        tk_kib = sum(v for _, v in tk) / len(tk)
        factor = copy_bytes / (cp_kib * 1024.0)
        out[counter] = {"topk_kib_per_dispatch": round(tk_kib, 1), "topk_dispatches": len(tk),
                        "copy_kib_per_dispatch": round(cp_kib, 1), "copy_bytes": copy_bytes,
                        "scale": round(factor, 4), "bytes_per_launch": int(tk_kib * 1024.0 * factor)}
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    fetch, write = out["FETCH_SIZE"]["bytes_per_launch"], out["WRITE_SIZE"]["bytes_per_launch"]
    data[w.name] = {
        "kernel_sha256_16": _kernel_hash(),
        "kernels": sorted(names),
        "bytes_per_launch": fetch + write,
        "fetch_bytes": fetch,
        "write_bytes": write,
        "algorithmic_input_bytes": workloads.algorithmic_bytes(w, workloads.end_ramp(w.batch, w.n_cols) if w.ragged else None),
        "output_bytes": workloads.output_bytes(w),
        "counters": out,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -- python3 bench.py --config {w.num} --steps 5 --warmup 2 --no-cpu --no-torch --no-graph --calibrate-copy",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -- python3 bench.py --config {w.num} --steps 5 --warmup 2 --no-cpu --no-torch --no-graph --calibrate-copy",
            f"python3 bench.py --config {w.num} --traffic-from <FETCH_DIR> <WRITE_DIR>",
        ],
    }
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[w.name]))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class Case:
    """One workload's device buffers and its call."""

    def __init__(self, num, args, torch, np, workloads, rt, dev):
        self.w = w = workloads.workload(num)
        x_np, end_np = workloads.make_input(w)
        self.x_np, self.end_np = x_np, end_np
        self.alg_bytes = workloads.algorithmic_bytes(w, end_np)
        self.out_bytes = workloads.output_bytes(w)
        self.n_copies = max(2, math.ceil(2 * MALL_BYTES / x_np.nbytes))
        if w.dtype == workloads.BF16:
            base = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            base = torch.from_numpy(x_np).to(dev)
        self.copies = [base] + [base.clone() for _ in range(self.n_copies - 1)]
        self.views = [c[:, : w.n_cols] for c in self.copies]
        self.end_t = None if end_np is None else torch.from_numpy(end_np).to(dev)
        self.it = torch.int64 if w.index_dtype == "int64" else torch.int32
        values = torch.empty((w.batch, w.k), dtype=base.dtype, device=dev) if w.return_values else None
        indices = torch.empty((w.batch, w.k), dtype=self.it, device=dev)
        status = torch.empty((w.batch,), dtype=torch.int32, device=dev)
        self.out = (values, indices, status)
        self.plan = (rt.Plan(segments=args.segments, perm_seed=0x5EED, kernel=args.kernel)
                     if (args.segments or args.kernel) else None)
        self.rt = rt
        self.sink = torch.zeros((1,), dtype=torch.int32, device=dev)
        self.ref = None

    def call(self, i, return_values=None, out=None):
        w = self.w
        rv = w.return_values if return_values is None else return_values
        self.rt.topk(self.views[i % self.n_copies], w.k, end=self.end_t, sorted=w.sorted,
                     return_values=rv, index_dtype=self.it, out=out or self.out, plan=self.plan)

    def read(self, i):
        self.rt.read_ceiling(self.views[i % self.n_copies], self.w.k, end=self.end_t,
                             plan=self.plan, sink=self.sink)

    def snapshot(self):
        return [None if t is None else t.clone() for t in self.out]

    def check(self, what):
        """Outputs equal to the eager call's, bit for bit; unsorted rows (any
        order is valid) are compared in index order."""
        got, ref = list(self.out), list(self.ref)
        if self.w.sorted == 0:
            for o in (got, ref):
                idx, order = o[1].sort(dim=1)
                o[1] = idx
                if o[0] is not None:
                    o[0] = o[0].gather(1, order)
        for name, a, b in zip(("values", "indices", "row_status"), got, ref):
            if a is None:
                continue
            if not bool((a.view(torch_dtype_int(a)) == b.view(torch_dtype_int(b))).all()):
                raise SystemExit(f"{self.w.name}: {name} after {what} differ from the eager call")


def torch_dtype_int(t):
    import torch
    return {2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]


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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nums = HEADLINE if args.config == 0 else (args.config,)
    cases = [Case(n, args, torch, np, workloads, rt, dev) for n in nums]
    K, W = args.steps, args.warmup

    if args.calibrate_copy:
        src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # Everything below runs on one side stream, which the library's workspace
    # is keyed by; warm-up calls allocate that workspace outside any capture.
    stream = torch.cuda.Stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def step(i):
        for c in cases:
            c.call(i)

    with torch.cuda.stream(stream):
        for i in range(max(W, 1)):
            step(i)
            for c in cases:
                c.read(i)
        torch.cuda.synchronize()
        for c in cases:
            st = c.out[2]
            assert int(st.abs().sum().item()) == 0, f"{c.w.name}: row status set on clean input"
            c.ref = c.snapshot()

    def eager_time(fn, reps):
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record(stream)
            for i in range(reps):
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def graph_of(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(reps):
                    fn(i)
        torch.cuda.synchronize()
        return g

    def graph_time(g, reps, check_cases=()):
        """ms per rep of one replay; an eager call and a check of every
        replay's outputs sit between replays."""
        with torch.cuda.stream(stream):
            g.replay()                       # untimed replay, checked
            torch.cuda.synchronize()
            for c in check_cases:
                c.check("an untimed graph replay")
                c.call(0)                    # eager work between replays
            torch.cuda.synchronize()
            a, b = ev(), ev()
            t0 = time.perf_counter()
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            for c in check_cases:
                c.check("the timed graph replay")
        return a.elapsed_time(b) / reps, wall

    # Whole-job timing: K steps, synchronised on both sides.
    if args.no_graph:
        ms_per_step = eager_time(step, K)
        wall_s = None
        per_ms = {c.w.num: eager_time(c.call, K) for c in cases}
    else:
        g_step = graph_of(step, K)
        ms_per_step, wall_s = graph_time(g_step, K, cases)
        del g_step
        per_ms = {}
        for c in cases:
            g = graph_of(c.call, K)
            per_ms[c.w.num], _ = graph_time(g, K, (c,))
            del g
    eager_ms = {c.w.num: eager_time(c.call, K) for c in cases}
    for c in cases:
        c.check("the eager timing loop")

    # Read ceiling: the same bytes, chunks, workgroups and loads, and nothing else.
    ceil_ms = {}
    for c in cases:
        if args.no_graph:
            ceil_ms[c.w.num] = eager_time(c.read, K)
        else:
            g = graph_of(c.read, K)
            ceil_ms[c.w.num], _ = graph_time(g, K)
            del g

    # The sampler's calls with the values output switched off (the pages note
    # that skipping the values is faster).
    ab = None
    for c in cases:
        if c.w.return_values and not args.no_graph:
            alt_out = (None, c.out[1].clone(), c.out[2].clone())
            g = graph_of(lambda i, c=c, o=alt_out: c.call(i, return_values=False, out=o), K)
            alt_ms, _ = graph_time(g, K)
            del g
            ab = {"workload": c.w.name, "with_values_us": round(per_ms[c.w.num] * 1e3, 3),
                  "without_values_us": round(alt_ms * 1e3, 3)}
            break

    # The sampling step after the sampler's TopK (ds_sampler_tail), on that
    # call's outputs, timed the same way.
    tail = None
    for c in cases:
        if c.w.num == 2 and c.w.sorted == 1 and c.w.return_values and not args.no_graph:
            u = torch.rand(c.w.batch, generator=torch.Generator().manual_seed(7)).to(dev)
            vals, idx, st = c.out
            fn = lambda i, vals=vals, idx=idx, st=st, u=u: rt.sample_from_topk(  # noqa: E731
                vals, idx, st, temperature=0.8, top_p=0.95, uniforms=u)
            with torch.cuda.stream(stream):
                fn(0)
            g = graph_of(fn, K)
            tail_ms, _ = graph_time(g, K)
            del g
            tail = {"workload": c.w.name + " outputs", "temperature": 0.8, "top_p": 0.95,
                    "us_per_call": round(tail_ms * 1e3, 3)}

    torch_us = {}
    if not args.no_torch:
        for c in cases:
            with torch.cuda.stream(stream):
                for _ in range(3):
                    torch.topk(c.views[0], c.w.k, dim=1, sorted=bool(c.w.sorted))
            reps = 20
            torch_us[c.w.name] = round(eager_time(
                lambda i, c=c: torch.topk(c.views[i % c.n_copies], c.w.k, dim=1, sorted=bool(c.w.sorted)),
                reps) * 1e3, 2)

    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        parts, t_step, b_step = [], 0.0, 0
        used_max = 1
        for c in cases:
            w = c.w
            used = min(cores, w.batch)
            used_max = max(used_max, used)
            idx_np = np.int64 if w.index_dtype == "int64" else np.int32
            # The oracle sorts every row whole: a row longer than 2^24 elements is
            # timed on its first 2^24 columns instead (a bounded sample).
            cols = min(w.n_cols, 1 << 24)
            s_bytes = c.alg_bytes if cols == w.n_cols else w.batch * cols * w.elem_bytes
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.topk(c.x_np, w.k, dtype=w.dtype, n_cols=cols, end=c.end_np, sorted=w.sorted,
                            return_values=w.return_values, index_dtype=idx_np, n_threads=used)
                reps += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds or reps >= 1000:
                    break
            t_step += el / reps
            b_step += s_bytes
            what = (f"{w.name}: the full batch ({w.batch} rows)" if cols == w.n_cols
                    else f"{w.name}: the first {cols} columns of each of the {w.batch} rows")
            parts.append(f"{what}, {reps} repetitions in {el:.1f} s on {used} threads "
                         f"({s_bytes / (el / reps) / 1e9:.3f} GB/s)")
        cpu = {"value": round(b_step / t_step / 1e9, 4), "unit": "GB/s", "cores": used_max,
               "kind": "oracle", "cpu_model": _cpu_model(),
               "sample": "; ".join(parts) + "; value = both workloads' bytes / the sum of "
                         "their times per call, one row per thread at a time"}

    total_bytes = sum(c.alg_bytes for c in cases)
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    rows = []
    for c in cases:
        w, n = c.w, c.w.num
        k_ms = per_ms[n]
        achieved = c.alg_bytes / (k_ms * 1e-3) / 1e9
        ceil_gbps = c.alg_bytes / (ceil_ms[n] * 1e-3) / 1e9
        rows.append({
            "workload": w.name, "batch": w.batch, "n_cols": w.n_cols, "row_stride": w.row_stride,
            "k": w.k, "sorted": w.sorted, "return_values": w.return_values,
            "index_dtype": w.index_dtype, "input_dtype": "f32" if w.dtype == workloads.FP32 else "bf16",
            "input_copies": c.n_copies, "input_sha256": workloads.digest(c.x_np, c.end_np)[:16],
            "us_per_call": round(k_ms * 1e3, 3),
            "eager_us_per_call": round(eager_ms[n] * 1e3, 3),
            "GBps": round(achieved, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "traffic": _traffic(w.name), "algorithmic_bytes": c.alg_bytes},
            "read_ceiling": {"us_per_call": round(ceil_ms[n] * 1e3, 3), "GBps": round(ceil_gbps, 2),
                             "frac_of_ceiling": round(achieved / ceil_gbps, 4)},
            "effective_GBps_with_outputs": round((c.alg_bytes + c.out_bytes) / (k_ms * 1e-3) / 1e9, 2),
        })
    dom = max(rows, key=lambda r: r["us_per_call"])
    roof = dict(dom["roofline"], workload=dom["workload"], kernel_us_mean=dom["us_per_call"])

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": " + ".join(r["workload"] for r in rows),
                   "timing": "eager launches" if args.no_graph else "HIP graph of the K steps",
                   "segments": args.segments or "auto", "kernel": args.kernel or "auto"},
        "us_per_step": round(ms_per_step * 1e3, 3),
        "wall_s_timed_region": None if wall_s is None else round(wall_s, 6),
        "workloads": rows,
        "roofline": roof,
        "return_values_ab": ab,
        "sampler_tail": tail,
        "torch_topk_us": torch_us or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
