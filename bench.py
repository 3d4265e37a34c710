#!/usr/bin/env python3
"""Benchmark of the fused sum + residual + RMSNorm + FP8 quant epilogue on one GPU.

A step is one ``arnfp8_run`` call over the prefill workload (P = 8 bf16 slabs
[8192, 7168] ~ N(0, 0.5) with 0.1 % outliers x100, bf16 residual ~ N(0, 1),
gamma ~ U(0.8, 1.2), eps 1e-6, scale_ub 64), all inputs resident in HBM before
the timed region.  Each call writes the next of several output buffer sets,
together larger than twice the 256 MB Infinity Cache, so no call finds its
outputs in cache.  Prints ONE JSON line:

  value       algorithmic HBM bytes per step / wall time per step   (GB/s)
  roofline    the kernel's algorithmic bytes / its average duration from HIP
              events on the launch stream, against the 8 TB/s HBM peak; the
              measured HBM traffic (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
              by a plain copy of known size) when a committed counter summary
              matches the current kernel source
  cpu_baseline the CPU oracle on the same bytes (rows of the same workload)
  latency_us_per_call  graph-replayed microseconds per call for the decode
              shapes (P = 4 [32, 7168], P = 8 [128, 8192], P = 2 [4, 256]) and of
              the sum alone (P = 4 [64, 4096]), the
              same buffers every call (cache-warm); latency_us_per_call_cold
              the same with every call reading its own inputs, > 512 MB in all

Other modes (not the JSON contract): ``--workload NAME`` times another
workload; ``--pmc-calib`` first runs one plain copy of known size (the P = 1
sum kernel; it scales the HBM counters); ``--summarize-pmc DIR`` turns rocprofv3 counter CSVs into the
committed summary; ``--summarize-ktrace DIR`` does the same for a
``rocprofv3 --kernel-trace --stats`` run.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import itertools
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
DEFAULT_WORKLOAD = "prefill_p8_8192x7168"
DECODE_WORKLOADS = ["decode_p4_32x7168", "unit_offset_p8_128x8192", "tiny_p2_4x256",
                    "sum_p4_64x4096"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "arnfp8_row_kernel_prefill_p8_8192x7168_hbm_traffic.md")
# The device code, the host code that picks its launch shape and cache
# policy, the ABI header whose constants both use, and the build flags: the
# committed HBM-counter summary applies only while their code (comments
# aside) is unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8_kernels.hpp"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8_tables.hpp"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8.hip"),
                  os.path.join(ROOT, "include", "arnfp8.h"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "build.py")]


def _code_only(path: str) -> bytes:
    """The file with comments and blank space removed, so that an edit of a
    comment does not retire the counters taken on the code."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    if path.endswith(".py"):
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split()).encode()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(_code_only(p))
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------- GPU side --

# Outputs rotate over enough buffer sets that together they exceed twice the
# 256 MB Infinity Cache: every call then writes buffers that are not cache-
# resident, as in a model, where other work runs between two calls.
CACHE_FLUSH_BYTES = 512 << 20
MAX_OUT_SETS = 8


def out_sets_for(w) -> int:
    per = w.numel * (2 if w.sum_only else 1 + (2 if w.residual_std is not None else 0))
    return max(1, min(MAX_OUT_SETS, -(-CACHE_FLUSH_BYTES // max(1, per))))


def alloc_workload(w, torch, dev, out_sets: int = 1, seed=None):
    """Inputs of workload `w` on `dev`, and `out_sets` sets of output buffers
    (d["outs"]; d["out"], d["scales"], d["res_out"], d["sum_out"] are set 0)."""
    from all_reduce_rmsnorm_amd import synth

    d = synth.make_inputs(w, device=dev, seed=seed)
    rows, cols = w.rows, w.cols
    d["outs"] = []
    for _ in range(out_sets):
        o = {"out": None, "scales": None, "res_out": None, "sum_out": None}
        if w.sum_only:
            o["sum_out"] = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
        else:
            o["out"] = torch.empty((rows, cols), dtype=torch.float8_e4m3fn, device=dev)
            o["scales"] = torch.empty((rows,), dtype=torch.float32, device=dev)
            if d["residual"] is not None:
                o["res_out"] = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
        d["outs"].append(o)
    d.update(d["outs"][0])
    return d


def input_sha256(d, torch) -> str:
    """SHA-256 over the bytes of every input tensor (slabs in rank order, the
    residual if any, gamma), so a run records exactly what it measured."""
    h = hashlib.sha256()
    ts = list(d["inputs"]) + ([d["residual"]] if d["residual"] is not None else []) + [d["gamma"]]
    for t in ts:
        flat = t.reshape(-1).view(torch.uint8)
        step = 64 << 20
        for i in range(0, flat.numel(), step):
            h.update(flat[i:i + step].cpu().numpy().tobytes())
    return h.hexdigest()


def rotating(fns):
    """One callable that calls fns[0], fns[1], ... in turn."""
    it = itertools.cycle(fns)
    return lambda: next(it)()


def step_fn(w, d, arn):
    """One step of workload `w`, each call writing the next output set."""
    def one(o):
        if w.sum_only:
            return lambda: arn.arn_sum_bf16(d["inputs"], o["sum_out"])
        return lambda: arn.arnfp8_run(d["inputs"], d["residual"], o["res_out"], o["out"],
                                      o["scales"], d["gamma"], w.eps, w.weight_offset, w.scale_ub)
    return rotating([one(o) for o in d["outs"]])


def time_steps(torch, fn, steps, warmup):
    """Exactly `steps` calls, synchronised on both sides: (wall ms per step,
    ms per launch from one HIP event pair on the launch stream around the
    same `steps` launches, which run back to back)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps * 1e3, a.elapsed_time(b) / steps


def graph_us_per_call_cold(torch, w, arn, dev, min_bytes=600 << 20, max_sets=400):
    """Microseconds per call with every call in the captured graph reading its
    own input set, the sets together larger than the 256 MB Infinity Cache."""
    from all_reduce_rmsnorm_amd import synth

    per = w.algorithmic_bytes()
    nsets = int(min(max_sets, -(-min_bytes // per)))
    if nsets * per < min_bytes:
        return None, nsets
    base = alloc_workload(w, torch, dev)
    sets = []
    for k in range(nsets):
        dk = dict(base)
        dk["inputs"] = [x.clone() for x in base["inputs"]]
        o = {key: (None if t is None else torch.empty_like(t)) for key, t in base["outs"][0].items()}
        if base["residual"] is not None:
            dk["residual"] = base["residual"].clone()
            o["res_out"] = dk["residual"]  # in place, as the decode workloads update it
        dk["outs"] = [o]
        sets.append(step_fn(w, dk, arn))
    us = graph_us_per_call(torch, lambda: [f() for f in sets], calls=1, reps=5) / nsets
    del sets, base
    torch.cuda.empty_cache()
    return us, nsets


def graph_us_per_call(torch, fn, calls=100, reps=5):
    """Microseconds per call with `calls` calls captured in one graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        best.append(a.elapsed_time(b) * 1e3 / calls)
    best.sort()
    return best[len(best) // 2]


# -------------------------------------------------------------- CPU side ---

def cpu_baseline(w, d, torch, min_seconds=10.0, max_passes=3):
    """The oracle over every row of the workload (same bytes as the GPU),
    repeated until at least `min_seconds` of CPU work (at most `max_passes`)."""
    import oracle
    from all_reduce_rmsnorm_amd import synth

    block = 1024
    gamma = synth.bf16_bits(d["gamma"])
    times, total_t = [], 0.0
    while len(times) < max_passes and (not times or total_t < min_seconds):
        pass_t = 0.0
        for r0 in range(0, w.rows, block):
            r1 = min(w.rows, r0 + block)
            xs = [synth.bf16_bits(x[r0:r1]) for x in d["inputs"]]
            res = None if d["residual"] is None else synth.bf16_bits(d["residual"][r0:r1])
            t = time.perf_counter()
            if w.sum_only:
                oracle.sum_bf16(xs)
            else:
                oracle.arnfp8(xs, gamma, w.eps, w.weight_offset, w.scale_ub, residual_in=res)
            pass_t += time.perf_counter() - t
        times.append(pass_t)
        total_t += pass_t
    per_pass = sorted(times)[len(times) // 2]
    return {
        "value": round(w.algorithmic_bytes() / per_pass / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"every row of {w.name} ({w.rows} rows), median of {len(times)} pass(es), "
                  f"{per_pass * 1e3:.1f} ms per pass; single-threaded C oracle",
        "ms_per_step": round(per_pass * 1e3, 3),
    }


def cpu_oracle_latency(names, runs=20):
    """Median microseconds per call of the single-threaded oracle on the small
    workloads (host bytes drawn by the same recipe), next to the GPU's."""
    import oracle
    from all_reduce_rmsnorm_amd import synth

    out = {}
    for name in names:
        w = synth.WORKLOADS[name]
        d = synth.make_inputs(w, device="cpu")
        xs = [synth.bf16_bits(x) for x in d["inputs"]]
        res = None if d["residual"] is None else synth.bf16_bits(d["residual"])
        gamma = synth.bf16_bits(d["gamma"])
        ts = []
        for _ in range(runs):
            t = time.perf_counter()
            if w.sum_only:
                oracle.sum_bf16(xs)
            else:
                oracle.arnfp8(xs, gamma, w.eps, w.weight_offset, w.scale_ub, residual_in=res)
            ts.append(time.perf_counter() - t)
        out[name] = round(sorted(ts)[len(ts) // 2] * 1e6, 1)
    return out


def host_cpu():
    """Model name and the CPUs this process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "usable_cpus": len(os.sched_getaffinity(0))}


def cpu_oracle_threaded(w, d, torch, passes=3, max_threads=16):
    """The same oracle, unchanged, with the workload's rows split into blocks
    that a thread pool hands to it (the C calls run without the interpreter
    lock).  A second CPU figure beside the single-threaded baseline."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from all_reduce_rmsnorm_amd import synth

    threads = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    block = max(1, -(-w.rows // (4 * threads)))
    gamma = synth.bf16_bits(d["gamma"])
    blocks = []
    for r0 in range(0, w.rows, block):
        r1 = min(w.rows, r0 + block)
        xs = [synth.bf16_bits(x[r0:r1]) for x in d["inputs"]]
        res = None if d["residual"] is None else synth.bf16_bits(d["residual"][r0:r1])
        blocks.append((xs, res))

    def one(b):
        xs, res = b
        if w.sum_only:
            oracle.sum_bf16(xs)
        else:
            oracle.arnfp8(xs, gamma, w.eps, w.weight_offset, w.scale_ub, residual_in=res)

    times = []
    with ThreadPoolExecutor(threads) as pool:
        for _ in range(passes):
            t = time.perf_counter()
            list(pool.map(one, blocks))
            times.append(time.perf_counter() - t)
    per_pass = sorted(times)[len(times) // 2]
    return {"value": round(w.algorithmic_bytes() / per_pass / 1e9, 4), "unit": "GB/s",
            "threads": threads, "ms_per_step": round(per_pass * 1e3, 3),
            "sample": f"every row of {w.name} in {len(blocks)} blocks, median of {passes} passes",
            "host_cpu": host_cpu()}


# ------------------------------------------------------- HBM counters ------

def read_traffic(kernel_hash: str):
    """(bytes per launch, note) from the committed counter summary, or None
    when it is missing or was taken on different kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash:
        return None
    return int(m_bytes.group(1))


def summarize_pmc(directory: str, out_path: str, workload: str):
    """Build the counter summary from rocprofv3 --pmc CSV output under `directory`:
    one run with FETCH_SIZE, one with WRITE_SIZE, each holding the fused kernel's
    dispatches and one plain copy of known size (``--pmc-calib``)."""
    import csv

    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS[workload]
    per = {}  # counter -> {"kernel": [kib...], "copy": [kib...]}
    files = sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    for f in files:
        for row in csv.DictReader(open(f)):
            name = row.get("Kernel_Name", "")
            ctr = row.get("Counter_Name", "")
            val = float(row.get("Counter_Value", "nan"))
            kind = "kernel" if "arnfp8_row_kernel" in name else (
                "copy" if "arn_sum_kernel<1" in name else None)
            if kind is None or ctr not in ("FETCH_SIZE", "WRITE_SIZE"):
                continue
            per.setdefault(ctr, {}).setdefault(kind, []).append(val)
    calib_bytes = int(os.environ.get("ARNFP8_CALIB_BYTES", str(1 << 30)))
    lines = []
    total = 0.0
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        k = per.get(ctr, {}).get("kernel", [])
        c = per.get(ctr, {}).get("copy", [])
        if not k or not c:
            raise SystemExit(f"missing {ctr} samples (kernel {len(k)}, copy {len(c)})")
        k_kib = sum(k) / len(k)
        c_kib = max(c)
        factor = calib_bytes / (c_kib * 1024.0)
        scaled = k_kib * 1024.0 * factor
        total += scaled
        lines.append(f"| {ctr} | {k_kib:.0f} KiB ({len(k)} dispatches) | {c_kib:.0f} KiB | "
                     f"{factor:.4f} | {scaled / 1e6:.2f} MB |")
    alg = w.algorithmic_bytes()
    text = "\n".join([
        f"# HBM traffic of the fused row kernel on {w.name}",
        "",
        "Counters from two `rocprofv3 --pmc` runs (FETCH_SIZE, then WRITE_SIZE), per",
        "dispatch, scaled by what the same counter reads for a plain copy of",
        f"{calib_bytes} bytes (read {calib_bytes} B, write {calib_bytes} B).",
        "Commands (from the repository root, on one MI355X):",
        "",
        f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {directory}/pmc_fetch -o fetch -- "
        "python -u bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-latency --pmc-calib",
        f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {directory}/pmc_write -o write -- "
        "python -u bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-latency --pmc-calib",
        f"    python bench.py --summarize-pmc {directory}",
        "",
        "| counter | fused kernel (mean per dispatch) | copy kernel | scale factor | scaled bytes |",
        "|---|---|---|---|---|",
        *lines,
        "",
        f"kernel_source_hash: {kernel_source_hash()}",
        f"traffic_bytes_per_launch: {int(round(total))}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic / algorithmic: {total / alg:.4f}",
        "",
    ])
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


def _short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def summarize_ktrace(directory: str, out_path: str, command: str):
    """Summarise a rocprofv3 --kernel-trace --stats CSV run: the library's
    kernels, split by launch shape (grid, workgroup), with mean durations."""
    import csv
    from collections import defaultdict

    traces = sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True))
    stats = sorted(glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True))
    if not traces:
        raise SystemExit(f"no kernel_trace.csv under {directory}")
    shapes = defaultdict(list)
    for f in traces:
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            if "arnfp8_" not in name and "arn_sum_kernel" not in name:
                continue
            key = (_short_name(name),
                   int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            shapes[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [f"# Kernel trace: {os.path.basename(out_path)[:-3]}", "",
             "Command (from the repository root, on one MI355X):", "",
             f"    {command}", "",
             "Per launch shape (grid = total lanes), from the kernel trace:", "",
             "| kernel | grid lanes | workgroup | calls | mean us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid, wg), v in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {grid} | {wg} | {len(v)} | {sum(v) / len(v) / 1e3:.3f} | "
                     f"{min(v) / 1e3:.3f} | {max(v) / 1e3:.3f} |")
    if stats:
        lines += ["", "rocprofv3 --stats summary (all kernels of the run, every shape pooled):", "",
                  "| kernel | calls | mean us | share % |", "|---|---|---|---|"]
        for r in csv.DictReader(open(stats[0])):
            nm = _short_name(r["Name"])
            if len(nm) > 90:
                nm = nm[:87] + "..."
            lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                         f"{float(r['Percentage']):.2f} |")
    lines.append("")
    text = "\n".join(lines)
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


# -------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=None,
                    help="input seed (default: the workload's own, 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="first run one plain device copy of 1 GiB (scales the HBM counters)")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--pmc-out", default=PMC_SUMMARY)
    ap.add_argument("--summarize-ktrace", metavar="DIR")
    ap.add_argument("--ktrace-out")
    ap.add_argument("--ktrace-command", default="")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.pmc_out, args.workload)
        return 0
    if args.summarize_ktrace:
        summarize_ktrace(args.summarize_ktrace, args.ktrace_out, args.ktrace_command)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange is out of scope; run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import all_reduce_rmsnorm_amd as arn
    from all_reduce_rmsnorm_amd import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    arn.library()

    if args.pmc_calib:
        # A plain copy of known size: the rank-order sum with P = 1 reads one
        # bf16 tensor and writes it back unchanged (1 GiB each way).
        src = torch.ones((65536, 8192), dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        arn.arn_sum_bf16([src], dst)
        torch.cuda.synchronize()
        log(f"pmc calibration copy: {src.numel() * 2} bytes read, {dst.numel() * 2} bytes written")
        del src, dst

    w = synth.WORKLOADS[args.workload]
    log(f"bench: workload {w.name}, steps {args.steps}, warmup {args.warmup}")
    n_out = out_sets_for(w)
    d = alloc_workload(w, torch, dev, out_sets=n_out, seed=args.seed)
    torch.cuda.synchronize()
    fn = step_fn(w, d, arn)
    ms_per_step, kern_ms = time_steps(torch, fn, args.steps, args.warmup)
    alg = w.algorithmic_bytes()
    value = alg / (ms_per_step * 1e-3) / 1e9
    achieved = alg / (kern_ms * 1e-3) / 1e9
    log(f"bench: {ms_per_step * 1e3:.2f} us/step wall, {kern_ms * 1e3:.2f} us/launch (events)")

    khash = kernel_source_hash()
    traffic = read_traffic(khash) if w.name == DEFAULT_WORKLOAD else None
    result = {
        "metric": "fused sum+RMSNorm+FP8 quant: achieved HBM GB/s (% of peak) and us/call",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtypes": "bf16 in, bf16 residual out, e4m3fn + f32 scales out" if not w.sum_only else "bf16 in, bf16 out",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "output_sets": n_out,
        "config": {"workload": w.name, "seed": w.seed if args.seed is None else args.seed,
                   "P": w.P, "rows": w.rows, "cols": w.cols,
                   "residual": w.residual_std is not None, "eps": w.eps,
                   "weight_offset": w.weight_offset, "scale_ub": w.scale_ub,
                   "algorithmic_bytes_per_step": alg, "input_sha256": input_sha256(d, torch)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us": round(kern_ms * 1e3, 3),
                     "kernel_source_hash": khash},
    }
    if not w.sum_only and not args.no_latency:
        # The unfused chain the fusion removes: the sum is written to HBM as
        # bf16 and read back by a second launch (the fused kernel with P = 1).
        s_bufs = [torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=dev)
                  for _ in d["outs"]]

        def unfused_one(o, s_buf):
            return lambda: (arn.arn_sum_bf16(d["inputs"], s_buf),
                            arn.arnfp8_run([s_buf], d["residual"], o["res_out"], o["out"],
                                           o["scales"], d["gamma"], w.eps, w.weight_offset,
                                           w.scale_ub))
        unfused = rotating([unfused_one(o, sb) for o, sb in zip(d["outs"], s_bufs)])
        un_ms, _ = time_steps(torch, unfused, max(5, args.steps // 2), 3)
        result["unfused_two_launch"] = {
            "us_per_call": round(un_ms * 1e3, 2),
            "extra_bytes_per_step": 4 * w.numel,
            "fused_speedup": round(un_ms / ms_per_step, 3),
        }
        log(f"bench: unfused two-launch chain {un_ms * 1e3:.2f} us/step")
        # The other output formats on the same workload and bytes (the MX
        # block scales replace the per-row scales: rows * cols / 32 bytes).
        fmt_out = {}
        mx_scales = [torch.empty((w.rows, w.cols // 32), dtype=torch.uint8, device=dev)
                     for _ in d["outs"]]

        def fmt_one(o, sc, fmt):
            return lambda: arn.arnfp8_run_fmt(d["inputs"], d["residual"], o["res_out"], o["out"],
                                              sc, d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                                              out_format=fmt)
        for name, fmt in (("e5m2", arn.FMT_E5M2), ("mxfp8", arn.FMT_MXFP8)):
            scs = mx_scales if fmt == arn.FMT_MXFP8 else [o["scales"] for o in d["outs"]]
            f = rotating([fmt_one(o, sc, fmt) for o, sc in zip(d["outs"], scs)])
            _, f_k = time_steps(torch, f, max(10, args.steps // 2), 3)
            fmt_out[f"{name}_us_per_call"] = round(f_k * 1e3, 2)
        result["formats"] = fmt_out
        del mx_scales
        # The residual updated in place (residual_out == residual_in), as a
        # transformer's residual stream is: each output set carries its own
        # residual copy, so the rotation still keeps every call out of cache.
        if d["residual"] is not None:
            res_sets = [d["residual"].clone() for _ in d["outs"]]

            def in_place_one(o, r):
                return lambda: arn.arnfp8_run(d["inputs"], r, r, o["out"], o["scales"], d["gamma"],
                                              w.eps, w.weight_offset, w.scale_ub)
            _, ip_k = time_steps(torch, rotating([in_place_one(o, r) for o, r in
                                                  zip(d["outs"], res_sets)]),
                                 max(10, args.steps // 2), 3)
            result["in_place_residual"] = {
                "us_per_call": round(ip_k * 1e3, 2),
                "gbs": round(alg / (ip_k * 1e-3) / 1e9, 1),
            }
            del res_sets
        # One rank's share of the two-stage layout (8 ranks): the single-GPU
        # half of the large-payload path, at its real shape.
        ngpus = 8
        stg = torch.empty((arn.arnfp8_stage_bytes(w.rows, w.cols, ngpus),), dtype=torch.uint8,
                          device=dev)
        share_rows = -(-w.rows // ngpus)

        # The ranks' shares in turn: each call reads other rows and writes
        # another staging slot, so no call finds its inputs in cache.
        def share_one(rank):
            return lambda: arn.arnfp8_run_share(
                d["inputs"], d["residual"], d["res_out"], stg, d["gamma"], w.eps,
                w.weight_offset, w.scale_ub, ngpus=ngpus, rank=rank)
        sh_ms, sh_k = time_steps(torch, rotating([share_one(r) for r in range(ngpus)]),
                                 max(16, args.steps), 3)
        share_bytes = (2 * w.P + 4 + 1) * share_rows * w.cols + 4 * share_rows + 2 * w.cols
        result["two_stage_share"] = {
            "ngpus": ngpus, "rank": "0-7 in turn", "rows": share_rows,
            "us_per_call": round(sh_k * 1e3, 2),
            "gbs": round(share_bytes / (sh_k * 1e-3) / 1e9, 1),
        }
        del stg
        # Achievable-bandwidth references on the same device: a plain copy
        # (the P = 1 sum kernel, 1 GiB each way) and the P-slab sum alone.
        src = torch.ones((65536, 8192), dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        cp_ms, cp_k = time_steps(torch, lambda: arn.arn_sum_bf16([src], dst), 10, 3)
        del src, dst
        sm_ms, sm_k = time_steps(torch, rotating([(lambda sb=sb: arn.arn_sum_bf16(d["inputs"], sb))
                                                  for sb in s_bufs]), 10, 3)
        del s_bufs
        result["reference_kernels"] = {
            "copy_1GiB_gbs": round(2 * (1 << 30) / (cp_k * 1e-3) / 1e9, 1),
            "sum_only_same_slabs_gbs": round((2 * w.P + 2) * w.numel / (sm_k * 1e-3) / 1e9, 1),
        }
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "hbm_gib": round(props.total_memory / 2**30, 1)}
    if not args.no_latency:
        lat = {}
        for name in DECODE_WORKLOADS:
            wd = synth.WORKLOADS[name]
            dd = alloc_workload(wd, torch, dev)
            lat[name] = round(graph_us_per_call(torch, step_fn(wd, dd, arn)), 3)
            del dd
        result["latency_us_per_call"] = lat
        log(f"bench: graph-replayed latency {lat}")
        cold = {}
        for name in DECODE_WORKLOADS:
            us, nsets = graph_us_per_call_cold(torch, synth.WORKLOADS[name], arn, dev)
            if us is not None:
                cold[name] = round(us, 3)
        result["latency_us_per_call_cold"] = cold
        log(f"bench: graph-replayed latency, inputs not in cache {cold}")
        # The same figures as algorithmic bytes per second (latency-bound
        # shapes: these are far below the HBM peak by nature).
        result["latency_gbs"] = {
            kind: {n: round(synth.WORKLOADS[n].algorithmic_bytes() / (us * 1e-6) / 1e9, 1)
                   for n, us in table.items()}
            for kind, table in (("warm", lat), ("cold", cold))}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, d, torch)
        log(f"bench: cpu baseline {result['cpu_baseline']}")
        result["cpu_oracle_threaded"] = cpu_oracle_threaded(w, d, torch)
        log(f"bench: oracle on a thread pool {result['cpu_oracle_threaded']}")
        result["cpu_oracle_us_per_call"] = cpu_oracle_latency(DECODE_WORKLOADS)
        log(f"bench: oracle per call on the small workloads {result['cpu_oracle_us_per_call']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
