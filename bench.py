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
              events on the launch stream (also the median of 5 equal
              segments of the timed steps), against the 8 TB/s HBM peak; the
              measured HBM traffic (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
              by a plain copy of known size) when a committed counter summary
              matches the current kernel source
  cpu_baseline the CPU oracle on the same bytes (rows of the same workload)
  two_stage_share  the 8 ranks' 1024-row shares of the same inputs, replayed
              from a captured graph (no host launch cost), with its roofline;
              the same with the residual updated in place; and the reference
              kernels (read-only, traffic twin) at the share's shape, timed
              the same way
  latency     per small workload (decode, unit offset, one token, tiny, sum):
              graph-replayed microseconds per call with the same buffers every
              call (cache-warm) and with every call on its own inputs after a
              1 GiB cache flush (cold), the single-call graph latency, and the
              kernel-only duration from the committed kernel trace
  reference_kernels  a plain copy, the sum alone, and the fused kernel's byte
              mix without its arithmetic (read-only, write-only, traffic twin)

Other modes (not the JSON contract): ``--profile-workload NAME`` runs only that
workload's calls (for rocprofv3); ``--pmc-calib`` first runs one plain copy of
known size (the P = 1 sum kernel; it scales the HBM counters);
``--summarize-pmc DIR`` and ``--summarize-ktrace DIR`` turn rocprofv3 output
into the committed summaries under profiles/.
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
SHARE_WORKLOAD = "prefill_share_p8_1024x7168"
SHARE_NGPUS = 8
LATENCY_WORKLOADS = ["decode_p4_32x7168", "unit_offset_p8_128x8192", "token_p4_1x7168",
                     "token_p8_1x8192", "tiny_p2_4x256", "sum_p4_64x4096"]
PROFILES = os.path.join(ROOT, "profiles")
# The device code, the host code that picks its launch shape and cache
# policy, the ABI header whose constants both use, and the build flags: a
# committed profile summary applies only while their code (comments aside)
# is unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8_kernels.hpp"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8_tables.hpp"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8.hip"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "csrc", "arnfp8_split.hip"),
                  os.path.join(ROOT, "include", "arnfp8.h"),
                  os.path.join(ROOT, "all_reduce_rmsnorm_amd", "build.py")]


def kernel_name_of(workload, split=False) -> str:
    """The kernel a workload times: the sum kernel for the sum-only workload,
    the split-row kernel for its arnfp8_run_split calls, else the fused row
    kernel."""
    from all_reduce_rmsnorm_amd import synth

    if split:
        return "arnfp8_split_kernel"
    return "arn_sum_kernel" if synth.WORKLOADS[workload].sum_only else "arnfp8_row_kernel"


# Small workloads whose arnfp8_run_split calls are profiled too (residual out
# of place, rows well under one per compute unit).
SPLIT_PROFILE_WORKLOADS = ["token_p8_1x8192", "unit_offset_p8_128x8192"]


def profile_path(workload: str, kind: str, split=False) -> str:
    """profiles/<kernel>_<workload>_<kind>.md, kind "hbm_traffic" or "kernel_trace"."""
    return os.path.join(PROFILES, f"{kernel_name_of(workload, split)}_{workload}_{kind}.md")


PMC_SUMMARY = os.path.join(PROFILES, "arnfp8_row_kernel_prefill_p8_8192x7168_hbm_traffic.md")


def _code_only(path: str) -> bytes:
    """The file with comments and blank space removed, so that an edit of a
    comment does not retire the profiles taken on the code."""
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


# ------------------------------------------------------ committed profiles --

def read_profile(path: str, key: str, kernel_hash: str):
    """The number after ``key:`` in a committed profile summary, or None when
    the summary is missing or was taken on different kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_val = re.search(rf"(?m)^{re.escape(key)}:\s*([0-9.eE+-]+)\s*$", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_hash:
        return None
    v = float(m_val.group(1))
    return int(v) if v.is_integer() else v


def read_traffic(kernel_hash: str, path: str | None = None):
    """HBM bytes per launch from a committed counter summary (None if stale)."""
    return read_profile(PMC_SUMMARY if path is None else path, "traffic_bytes_per_launch",
                        kernel_hash)


# --------------------------------------------------------------- GPU side --

# Outputs rotate over enough buffer sets that together they exceed twice the
# 256 MB Infinity Cache: every call then writes buffers that are not cache-
# resident, as in a model, where other work runs between two calls.
CACHE_FLUSH_BYTES = 512 << 20
MAX_OUT_SETS = 8


def out_sets_for(w) -> int:
    per = w.numel * (2 if w.sum_only else 1 + (2 if w.residual_std is not None else 0))
    return max(1, min(MAX_OUT_SETS, -(-CACHE_FLUSH_BYTES // max(1, per))))


def _outputs(w, torch, dev, rows):
    o = {"out": None, "scales": None, "res_out": None, "sum_out": None}
    if w.sum_only:
        o["sum_out"] = torch.empty((rows, w.cols), dtype=torch.bfloat16, device=dev)
    else:
        o["out"] = torch.empty((rows, w.cols), dtype=torch.float8_e4m3fn, device=dev)
        o["scales"] = torch.empty((rows,), dtype=torch.float32, device=dev)
        if w.residual_std is not None:
            o["res_out"] = torch.empty((rows, w.cols), dtype=torch.bfloat16, device=dev)
    return o


def alloc_workload(w, torch, dev, out_sets: int = 1, seed=None):
    """Inputs of workload `w` on `dev`, and `out_sets` sets of output buffers
    (d["outs"]; d["out"], d["scales"], d["res_out"], d["sum_out"] are set 0).
    The residual is written out of place, so that every step is identical."""
    from all_reduce_rmsnorm_amd import synth

    d = synth.make_inputs(w, device=dev, seed=seed)
    d["outs"] = [_outputs(w, torch, dev, w.rows) for _ in range(out_sets)]
    d.update(d["outs"][0])
    return d


def alloc_windows(w, torch, dev, nwin: int):
    """`nwin` disjoint copies ("windows") of workload `w`'s inputs and outputs,
    cut from one tensor set of nwin * rows rows drawn by the same recipe: a
    call on window k touches bytes no other window touches.  A workload whose
    residual is updated in place writes it back into its own window."""
    from all_reduce_rmsnorm_amd import synth

    big = synth.make_inputs(w, device=dev, rows=nwin * w.rows)
    outs = _outputs(w, torch, dev, nwin * w.rows)
    wins = []
    for k in range(nwin):
        sl = slice(k * w.rows, (k + 1) * w.rows)
        d = {"inputs": [x[sl] for x in big["inputs"]], "gamma": big["gamma"],
             "residual": None if big["residual"] is None else big["residual"][sl]}
        for key, t in outs.items():
            d[key] = None if t is None else t[sl]
        if w.in_place and d["residual"] is not None:
            d["res_out"] = d["residual"]
        wins.append(d)
    return wins


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


def call_on(w, d, arn, launch=None):
    """One call of workload `w` on the buffers of `d` (d["out"] etc.)."""
    if w.sum_only:
        return lambda: arn.arn_sum_bf16(d["inputs"], d["sum_out"])
    if launch is not None:
        return lambda: arn.arnfp8_run_ex(d["inputs"], d["residual"], d["res_out"], d["out"],
                                         d["scales"], d["gamma"], w.eps, w.weight_offset,
                                         w.scale_ub, launch=launch)
    return lambda: arn.arnfp8_run(d["inputs"], d["residual"], d["res_out"], d["out"],
                                  d["scales"], d["gamma"], w.eps, w.weight_offset, w.scale_ub)


def split_call_on(w, d, arn, workspace):
    """One arnfp8_run_split call of workload `w` on the buffers of `d` (the
    automatic number of parts), trading statistics through `workspace`."""
    return lambda: arn.arnfp8_run_split(d["inputs"], d["residual"], d["res_out"], d["out"],
                                        d["scales"], d["gamma"], w.eps, w.weight_offset,
                                        w.scale_ub, workspace=workspace)


def split_parts(w, arn):
    """The parts per row arnfp8_run_split picks for workload `w` (for the record)."""
    return arn.arnfp8_split_parts(w.rows, w.cols)


def step_fn(w, d, arn):
    """One step of workload `w`, each call writing the next output set."""
    return rotating([call_on(w, dict(d, **o), arn) for o in d["outs"]])


def share_calls(w, d, arn, staging, residual=None):
    """The SHARE_NGPUS ranks' two-stage shares of the prefill inputs `d`, each
    into its own staging slot, the residual rows written into d["res_out"]
    (or, with `residual`, read from and written back into that tensor)."""
    res_in = d["residual"] if residual is None else residual
    res_out = d["res_out"] if residual is None else residual
    return [(lambda r=r: arn.arnfp8_run_share(d["inputs"], res_in, res_out, staging[r],
                                              d["gamma"], w.eps, w.weight_offset, w.scale_ub,
                                              ngpus=SHARE_NGPUS, rank=r))
            for r in range(SHARE_NGPUS)]


def share_reference(w, d, torch, dev):
    """The bench's reference kernels at one share's shape, timed as the share
    is (the 8 ranks' row ranges in turn, four rounds in one graph): reading
    the share's 9 streams, and the traffic twin (the same reads plus 16 + 8
    bytes written per 16-byte chunk, no arithmetic)."""
    import ctypes

    L = ref_library()
    S = -(-w.rows // SHARE_NGPUS)
    streams = list(d["inputs"]) + [d["residual"]]
    arrs = [(ctypes.c_void_p * len(streams))(*[t[r * S:(r + 1) * S].data_ptr() for t in streams])
            for r in range(SHARE_NGPUS)]
    sink = torch.empty((S, 16), dtype=torch.uint8, device=dev)
    tw16 = [torch.empty((S, w.cols), dtype=torch.bfloat16, device=dev) for _ in range(SHARE_NGPUS)]
    tw8 = [torch.empty((S, w.cols), dtype=torch.uint8, device=dev) for _ in range(SHARE_NGPUS)]

    def checked(st):
        if st != 0:
            raise RuntimeError(f"reference kernel launch failed with status {st}")

    def stream():
        return torch.cuda.current_stream().cuda_stream

    read = [(lambda r=r: checked(L.arnref_read(arrs[r], len(streams), sink.data_ptr(), S,
                                               2 * w.cols, 0, 0, stream())))
            for r in range(SHARE_NGPUS)]
    twin = [(lambda r=r: checked(L.arnref_twin(arrs[r], len(streams), tw16[r].data_ptr(),
                                               tw8[r].data_ptr(), S, 2 * w.cols, 0, 0, stream())))
            for r in range(SHARE_NGPUS)]
    rd_us = graph_us_per_call(torch, read * 4, reps=7)
    tw_us = graph_us_per_call(torch, twin * 4, reps=7)
    rd_bytes = len(streams) * 2 * S * w.cols
    tw_bytes = rd_bytes + 3 * S * w.cols
    return {"read_only_us": round(rd_us, 3),
            "read_only_frac": round(rd_bytes / (rd_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic_twin_us": round(tw_us, 3),
            "traffic_twin_frac": round(tw_bytes / (tw_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def share_bytes(w) -> int:
    """Algorithmic bytes of one rank's share of workload `w` (all its rows'
    traffic; the slot holds the share's fp8 rows and scales)."""
    rows = -(-w.rows // SHARE_NGPUS)
    return (2 * w.P + 4 + 1) * rows * w.cols + 4 * rows + 2 * w.cols


def time_steps(torch, fn, steps, warmup, segments=1):
    """Exactly `steps` calls, synchronised on both sides: (wall ms per step,
    ms per launch from a HIP event pair on the launch stream around the same
    `steps` launches, which run back to back, [ms per launch of each of
    `segments` equal segments of them, from events between the segments])."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    bounds = [round(i * steps / segments) for i in range(segments + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(segments):
        for _ in range(bounds[i + 1] - bounds[i]):
            fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    segs = [ev[i].elapsed_time(ev[i + 1]) / max(1, bounds[i + 1] - bounds[i])
            for i in range(segments)]
    return wall / steps * 1e3, ev[0].elapsed_time(ev[-1]) / steps, segs


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def graph_us_per_call(torch, fns, reps=7, flush=None):
    """Median microseconds per call of the calls `fns`, captured in order in
    one graph and replayed `reps` times; each replay is timed alone by a HIP
    event pair.  With `flush` (a device buffer), the buffer is overwritten
    and the device synchronised before every replay, so the replay starts
    with no input in any cache."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns[:3]:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(0x5A)
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3 / len(fns))
    del g
    return median(times)


def latency_figures(w, torch, arn, dev, flush, khash, calls=100, nwin=64):
    """Graph-replayed microseconds per call of small workload `w`."""
    wins = alloc_windows(w, torch, dev, nwin)
    fs = [call_on(w, d, arn) for d in wins]
    alg = w.algorithmic_bytes()
    r = {"warm_us_per_call": graph_us_per_call(torch, [fs[0]] * calls),
         "cold_us_per_call": graph_us_per_call(torch, fs, flush=flush),
         "single_call_graph_us_warm": graph_us_per_call(torch, [fs[0]], reps=21),
         "single_call_graph_us_cold": graph_us_per_call(torch, [fs[1]], reps=21, flush=flush)}
    r = {k: round(v, 3) for k, v in r.items()}
    r["algorithmic_bytes"] = alg
    r["gbs_warm"] = round(alg / (r["warm_us_per_call"] * 1e-6) / 1e9, 1)
    r["gbs_cold"] = round(alg / (r["cold_us_per_call"] * 1e-6) / 1e9, 1)
    r["residual"] = ("in place" if w.in_place else "out of place") if w.residual_std else None
    k_us = read_profile(profile_path(w.name, "kernel_trace"), "mean_us", khash)
    traffic = read_profile(profile_path(w.name, "hbm_traffic"), "traffic_bytes_per_launch", khash)
    r["kernel_us_trace"] = k_us
    r["frac_kernel_trace"] = (round(alg / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                              if k_us else None)
    r["traffic"] = traffic
    if not w.sum_only and w.rows == 1:
        # One token: the automatic launch shape against one chunk per lane
        # (a workgroup of up to 1024 lanes), both cold.
        fs1 = [call_on(w, d, arn, launch={"vpt": 1}) for d in wins]
        r["one_chunk_per_lane_cold_us_per_call"] = round(
            graph_us_per_call(torch, fs1, flush=flush), 3)
    if not w.sum_only and not w.in_place:
        # The same calls with each row split across workgroups that trade
        # their statistics (arnfp8_run_split; not for an in-place residual).
        ws = torch.zeros((arn.arnfp8_split_workspace_bytes(w.rows) // 8,), dtype=torch.int64,
                         device=dev)
        fsp = [split_call_on(w, d, arn, ws) for d in wins]
        r["split_parts"] = split_parts(w, arn)
        r["split_warm_us_per_call"] = round(graph_us_per_call(torch, [fsp[0]] * calls), 3)
        r["split_cold_us_per_call"] = round(graph_us_per_call(torch, fsp, flush=flush), 3)
        sk_us = read_profile(profile_path(w.name, "kernel_trace", True), "mean_us", khash)
        r["split_kernel_us_trace"] = sk_us
        r["split_frac_kernel_trace"] = (round(alg / (sk_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                        if sk_us else None)
        r["split_traffic"] = read_profile(profile_path(w.name, "hbm_traffic", True),
                                          "traffic_bytes_per_launch", khash)
        del ws, fsp
    del wins, fs
    torch.cuda.empty_cache()
    return r


# -------------------------------------------------- reference kernels ------

_ref = None


def ref_library():
    """libarnfp8_ref.so: the benchmark's achievable-bandwidth reference kernels."""
    global _ref
    if _ref is None:
        import ctypes

        path = os.path.join(ROOT, "all_reduce_rmsnorm_amd", "libarnfp8_ref.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run `python -m all_reduce_rmsnorm_amd.build`")
        L = ctypes.CDLL(path)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.arnref_read.argtypes = [ctypes.POINTER(vp), ci, vp, i64, i64, ci, ci, vp]
        L.arnref_write.argtypes = [ctypes.POINTER(vp), ci, i64, i64, ci, ci, vp]
        L.arnref_twin.argtypes = [ctypes.POINTER(vp), ci, vp, vp, i64, i64, ci, ci, vp]
        L.arnref_empty.argtypes = [i64, ci, vp]
        L.arnref_exchange.argtypes = [vp, ci, ci, ci, vp, vp]
        for f in (L.arnref_read, L.arnref_write, L.arnref_twin, L.arnref_empty,
                  L.arnref_exchange):
            f.restype = ci
        _ref = L
    return _ref


def reference_kernels(w, d, torch, arn, dev, s_bufs, steps=20):
    """Bandwidth of kernels that move the fused kernel's bytes, on the same
    device, inputs and launch pattern (one workgroup per row)."""
    import ctypes

    L = ref_library()
    stream = torch.cuda.current_stream().cuda_stream
    row_bytes = 2 * w.cols
    arr = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])

    def checked(st):
        if st != 0:
            raise RuntimeError(f"reference kernel launch failed with status {st}")

    out = {}
    src = torch.ones((65536, 8192), dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    _, cp_k, _ = time_steps(torch, lambda: arn.arn_sum_bf16([src], dst), 10, 3)
    out["copy_1GiB_gbs"] = round(2 * (1 << 30) / (cp_k * 1e-3) / 1e9, 1)
    del src, dst
    _, sm_k, _ = time_steps(torch, rotating([(lambda sb=sb: arn.arn_sum_bf16(d["inputs"], sb))
                                             for sb in s_bufs]), 10, 3)
    out["sum_only_same_slabs_gbs"] = round((2 * w.P + 2) * w.numel / (sm_k * 1e-3) / 1e9, 1)
    streams = list(d["inputs"]) + [d["residual"]]
    sink = torch.empty((w.rows, 16), dtype=torch.uint8, device=dev)
    rd = arr(streams)
    _, rd_k, _ = time_steps(torch, lambda: checked(L.arnref_read(rd, len(streams), sink.data_ptr(),
                                                                 w.rows, row_bytes, 0, 0, stream)),
                            steps, 3)
    rd_bytes = len(streams) * w.numel * 2
    out["read_only_streams"] = len(streams)
    out["read_only_gbs"] = round(rd_bytes / (rd_k * 1e-3) / 1e9, 1)
    wsets = [torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=dev) for _ in range(8)]
    wptrs = [arr([t]) for t in wsets]
    _, wr_k, _ = time_steps(torch, rotating([(lambda p=p: checked(L.arnref_write(
        p, 1, w.rows, row_bytes, 0, 0, stream))) for p in wptrs]), steps, 3)
    out["write_only_gbs"] = round(w.numel * 2 / (wr_k * 1e-3) / 1e9, 1)
    del wsets
    # The twin: the same 9 read streams, 16 + 8 bytes written per 16-byte
    # chunk into the fused step's own rotating output sets.
    tw = [(lambda o=o: checked(L.arnref_twin(rd, len(streams), o["res_out"].data_ptr(),
                                             o["out"].data_ptr(), w.rows, row_bytes, 0, 0,
                                             stream))) for o in d["outs"]]
    _, tw_k, _ = time_steps(torch, rotating(tw), steps, 3)
    tw_bytes = rd_bytes + 3 * w.numel
    out["traffic_twin_us"] = round(tw_k * 1e3, 2)
    out["traffic_twin_gbs"] = round(tw_bytes / (tw_k * 1e-3) / 1e9, 1)
    out["note"] = ("read/write kernels of libarnfp8_ref.so: one workgroup per row, 16-byte "
                   "non-temporal loads and stores, no arithmetic; twin = the fused kernel's "
                   "byte mix (9 read streams, 16 + 8 bytes written per chunk)")
    return out


# The launch shape the library picks for these workloads (one chunk per lane
# for eight slabs up to one row per CU, else 512 lanes of two chunks), used by
# every kernel of the breakdown below.
BREAKDOWN = {"decode_p4_32x7168": (512, 2), "unit_offset_p8_128x8192": (1024, 1),
             "token_p8_1x8192": (1024, 1)}


def decode_breakdown(w, torch, arn, dev, flush, nwin=64):
    """Where a small workload's time goes: graph-replayed microseconds per
    call (cold: every call on its own inputs after a 1 GiB flush; warm: the
    same inputs every call) of kernels on the same grid that do successively
    more of the fused kernel's work: nothing (the launch), the loads of the
    slabs and residual, the loads and the stores (the traffic twin), and the
    fused kernel itself (adds the row reduction and the row scalars)."""
    import ctypes

    L = ref_library()
    threads, vpt = BREAKDOWN[w.name]
    wins = alloc_windows(w, torch, dev, nwin)
    sink = torch.empty((8 * w.rows, 16), dtype=torch.uint8, device=dev)
    # The twin writes its bytes into buffers of its own (never the inputs).
    tw16 = torch.empty((nwin * w.rows, w.cols), dtype=torch.bfloat16, device=dev)
    tw8 = torch.empty((nwin * w.rows, w.cols), dtype=torch.uint8, device=dev)
    arrs = [(ctypes.c_void_p * (w.P + 1))(*[t.data_ptr() for t in d["inputs"] + [d["residual"]]])
            for d in wins]
    cur = lambda: torch.cuda.current_stream().cuda_stream
    launch = {"threads": threads, "vpt": vpt}

    def checked(st):
        if st != 0:
            raise RuntimeError(f"reference kernel launch failed with status {st}")

    kinds = {
        "empty": lambda k: (lambda: checked(L.arnref_empty(w.rows, threads, cur()))),
        "loads": lambda k: (lambda: checked(L.arnref_read(arrs[k], w.P + 1, sink.data_ptr(), w.rows,
                                                          2 * w.cols, threads, vpt, cur()))),
        "loads_and_stores": lambda k: (lambda: checked(L.arnref_twin(
            arrs[k], w.P + 1, tw16[k * w.rows].data_ptr(), tw8[k * w.rows].data_ptr(), w.rows,
            2 * w.cols, threads, vpt, cur()))),
        "fused": lambda k: call_on(w, wins[k], arn, launch=launch),
    }
    if not w.in_place:
        ws = torch.zeros((arn.arnfp8_split_workspace_bytes(w.rows) // 8,), dtype=torch.int64,
                         device=dev)
        kinds["fused_split_rows"] = lambda k: split_call_on(w, wins[k], arn, ws)
    # The same bytes spread over `parts` times as many workgroups, each
    # reading (and writing) 1/parts of a row: what splitting rows across
    # workgroups could save on the memory side, before the cost of exchanging
    # the row statistics between them.
    parts = max(1, min(8, 256 // w.rows))
    if parts > 1 and (w.cols // 8) % parts == 0:
        sub_c16 = w.cols // 8 // parts
        sub_threads = max(64, -(-sub_c16 // 64) * 64)
        kinds[f"loads_over_{parts * w.rows}_workgroups"] = lambda k: (lambda: checked(L.arnref_read(
            arrs[k], w.P + 1, sink.data_ptr(), parts * w.rows, 16 * sub_c16, sub_threads, 1,
            cur())))
        kinds[f"loads_and_stores_over_{parts * w.rows}_workgroups"] = lambda k: (
            lambda: checked(L.arnref_twin(arrs[k], w.P + 1, tw16[k * w.rows].data_ptr(),
                                          tw8[k * w.rows].data_ptr(), parts * w.rows,
                                          16 * sub_c16, sub_threads, 1, cur())))
    out = {"launch": f"{w.rows} workgroups x {threads} lanes, {vpt} chunk(s) per lane"}
    for name, mk in kinds.items():
        fs = [mk(k) for k in range(nwin)]
        out[name] = {"warm_us_per_call": round(graph_us_per_call(torch, [fs[0]] * 100), 3),
                     "cold_us_per_call": round(graph_us_per_call(torch, fs, flush=flush), 3)}
    del wins, arrs, tw16, tw8
    torch.cuda.empty_cache()
    return out


def exchange_cost(torch, dev, nwg=256, calls=64):
    """Graph-replayed microseconds per launch of 256 one-wave workgroups that
    do nothing, and of the same grid exchanging one 64-bit word within groups
    of 2 and 8 workgroups (consecutive ids, or ids equal modulo 8, which
    share an XCD): the price of the cross-workgroup step a split row needs."""
    L = ref_library()
    cur = lambda: torch.cuda.current_stream().cuda_stream
    words = torch.zeros((nwg,), dtype=torch.int64, device=dev)
    timeouts = torch.zeros((1,), dtype=torch.int32, device=dev)

    def checked(st):
        if st != 0:
            raise RuntimeError(f"reference kernel launch failed with status {st}")

    out = {"workgroups": nwg, "empty_us_per_call": round(graph_us_per_call(
        torch, [lambda: checked(L.arnref_empty(nwg, 64, cur()))] * calls), 3)}
    for S in (2, 8):
        for stride, where in ((1, "consecutive"), (8, "same_xcd")):
            f = lambda S=S, stride=stride: checked(L.arnref_exchange(
                words.data_ptr(), nwg, S, stride, timeouts.data_ptr(), cur()))
            out[f"groups_of_{S}_{where}_us_per_call"] = round(graph_us_per_call(
                torch, [f] * calls), 3)
    torch.cuda.synchronize()
    out["timeouts"] = int(timeouts.item())
    return out


def latency_scaling(torch, arn, dev, flush, rows_list=(1, 8, 32, 64, 128, 256, 512, 1024)):
    """Graph-replayed microseconds per call (cold) of the unit-offset
    workload's laws (P = 8, 8192 columns) at growing row counts: a fixed
    latency plus a bandwidth term."""
    import dataclasses

    from all_reduce_rmsnorm_amd import synth

    base = synth.WORKLOADS["unit_offset_p8_128x8192"]
    out = {}
    for r in rows_list:
        w = dataclasses.replace(base, name=f"unit_offset_p8_{r}x8192", rows=r)
        wins = alloc_windows(w, torch, dev, min(64, max(8, 8192 // r)))
        us = graph_us_per_call(torch, [call_on(w, d, arn) for d in wins], flush=flush)
        out[str(r)] = {"cold_us_per_call": round(us, 3),
                       "gbs": round(w.algorithmic_bytes() / (us * 1e-6) / 1e9, 1)}
        del wins
        torch.cuda.empty_cache()
    return out


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

def _kernel_filter(workload, split=False):
    """A predicate on rocprofv3 kernel names: the kernel `workload` times
    (the e4m3fn row kernel with its P, the sum kernel with its P, or the
    split-row kernel with its P)."""
    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS[workload]
    if split:
        want = f"arnfp8_split_kernel<{w.P},"
    else:
        want = f"arn_sum_kernel<{w.P}," if w.sum_only else f"arnfp8_row_kernel<0, {w.P},"
    return lambda name: want in name.replace("(anonymous namespace)::", "")


def summarize_pmc(directory: str, out_path: str, workload: str, command: str = "", split=False):
    """Build the counter summary from rocprofv3 --pmc CSV output under
    `directory` (or under each of a comma-separated list of directories): one
    run with FETCH_SIZE, one with WRITE_SIZE, each holding the workload's
    kernel dispatches and one plain copy of known size (``--pmc-calib``)."""
    import csv

    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS[workload]
    is_kernel = _kernel_filter(workload, split)
    per = {}  # counter -> {"kernel": [kib...], "copy": [kib...]}
    dirs = directory.split(",")
    files = sorted(f for d in dirs for f in
                   glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    for f in files:
        for row in csv.DictReader(open(f)):
            name = row.get("Kernel_Name", "")
            ctr = row.get("Counter_Name", "")
            val = float(row.get("Counter_Value", "nan"))
            kind = "kernel" if is_kernel(name) else ("copy" if "arn_sum_kernel<1, 4>" in name else None)
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
        lines.append(f"| {ctr} | {k_kib:.1f} KiB ({len(k)} dispatches) | {c_kib:.0f} KiB | "
                     f"{factor:.4f} | {scaled / 1e6:.3f} MB |")
    alg = w.algorithmic_bytes()
    if not command:
        command = (f"python -u bench.py --profile-workload {workload} --pmc-calib"
                   + (" --split" if split else ""))
    fetch_dir, write_dir = (dirs + dirs)[:2] if len(dirs) > 1 else (f"{directory}/pmc_fetch",
                                                                  f"{directory}/pmc_write")
    text = "\n".join([
        f"# HBM traffic of `{kernel_name_of(workload, split)}` on {workload}",
        "",
        "Counters from two `rocprofv3 --pmc` runs (FETCH_SIZE, then WRITE_SIZE), per",
        "dispatch, scaled by what the same counter reads for a plain copy of",
        f"{calib_bytes} bytes (read {calib_bytes} B, write {calib_bytes} B): the P = 1 sum kernel.",
        "Every profiled dispatch reads inputs that no earlier dispatch touched since a",
        "1 GiB cache flush.  Commands (from the repository root, on one MI355X):",
        "",
        f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o fetch -- {command}",
        f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o write -- {command}",
        f"    python bench.py --summarize-pmc {directory} --workload {workload}"
        + (" --split" if split else ""),
        "",
        "| counter | kernel (mean per dispatch) | copy kernel | scale factor | scaled bytes |",
        "|---|---|---|---|---|",
        *lines,
        "",
        f"workload: {workload}",
        f"kernel_source_hash: {kernel_source_hash()}",
        f"traffic_bytes_per_launch: {int(round(total))}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {total / alg:.4f}",
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


def summarize_ktrace(directory: str, out_path: str, command: str, workload: str, split=False):
    """Summarise a rocprofv3 --kernel-trace --stats CSV run: the library's
    kernels, split by launch shape (grid, workgroup), with mean durations;
    the workload's own kernel and launch shape get machine-readable lines."""
    import csv
    from collections import defaultdict

    from all_reduce_rmsnorm_amd import synth

    w = synth.WORKLOADS[workload]
    traces = sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True))
    stats = sorted(glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True))
    if not traces:
        raise SystemExit(f"no kernel_trace.csv under {directory}")
    shapes = defaultdict(list)
    for f in traces:
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"]
            if "arnfp8_" not in name and "arn_sum_kernel" not in name and "arnref" not in name:
                continue
            key = (_short_name(name), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            shapes[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = [f"# Kernel trace: `{kernel_name_of(workload, split)}` on {workload}", "",
             "Command (from the repository root, on one MI355X):", "",
             f"    {command}", "",
             "Per launch shape (grid = total lanes), from the kernel trace:", "",
             "| kernel | grid lanes | workgroup | calls | mean us | median us | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, grid, wg), v in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {grid} | {wg} | {len(v)} | {sum(v) / len(v) / 1e3:.3f} | "
                     f"{median(v) / 1e3:.3f} | {min(v) / 1e3:.3f} | {max(v) / 1e3:.3f} |")
    if stats:
        lines += ["", "rocprofv3 --stats summary (all kernels of the run, every shape pooled):", "",
                  "| kernel | calls | mean us | share % |", "|---|---|---|---|"]
        for r in csv.DictReader(open(stats[0])):
            nm = _short_name(r["Name"])
            if len(nm) > 90:
                nm = nm[:87] + "..."
            lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                         f"{float(r['Percentage']):.2f} |")
    # The workload's kernel at its launch shape (grid = min(rows, 65536)
    # workgroups for the row kernel; the shape with the most calls otherwise).
    is_kernel = _kernel_filter(workload, split)
    mine = [(k, v) for k, v in shapes.items() if is_kernel(k[0])]
    if not w.sum_only and not split:
        wgs = min(w.rows, 65536)
        mine = [(k, v) for k, v in mine if k[1] == wgs * k[2]] or mine
    if not mine:
        raise SystemExit(f"no dispatch of the {workload} kernel in the trace")
    (name, grid, wg), v = max(mine, key=lambda kv: len(kv[1]))
    lines += ["", f"workload: {workload}", f"kernel_source_hash: {kernel_source_hash()}",
              f"kernel: {name}", f"launch: {grid // wg} workgroups x {wg} lanes",
              f"calls: {len(v)}", f"mean_us: {sum(v) / len(v) / 1e3:.3f}",
              f"median_us: {median(v) / 1e3:.3f}", ""]
    text = "\n".join(lines)
    with open(out_path, "w") as f:
        f.write(text)
    print(text)


# ------------------------------------------------------ profile workloads --

def profile_workload(name, torch, arn, dev, steps, split=False):
    """Only the calls of workload `name`, each on bytes that no earlier call
    touched since the last flush, for rocprofv3 (kernel trace or counters):
    the prefill step with rotating output sets, the share's ranks in turn,
    and the small workloads on disjoint windows (with `split`, through
    arnfp8_run_split)."""
    from all_reduce_rmsnorm_amd import synth

    if name == SHARE_WORKLOAD:
        # As the benchmark times it: the 8 ranks' calls in turn, four rounds
        # captured in one graph, replayed `steps` times.
        w = synth.WORKLOADS[DEFAULT_WORKLOAD]
        d = alloc_workload(w, torch, dev)
        stg = [torch.empty((arn.arnfp8_stage_bytes(w.rows, w.cols, SHARE_NGPUS),),
                           dtype=torch.uint8, device=dev) for _ in range(SHARE_NGPUS)]
        us = graph_us_per_call(torch, share_calls(w, d, arn, stg) * 4, reps=steps)
        log(f"profile workload {name}: {steps} graph replays of {4 * SHARE_NGPUS} calls, "
            f"{us:.3f} us per call")
        return
    elif name == DEFAULT_WORKLOAD:
        w = synth.WORKLOADS[name]
        fn = step_fn(w, alloc_workload(w, torch, dev, out_sets=out_sets_for(w)), arn)
    else:
        w = synth.WORKLOADS[name]
        wins = alloc_windows(w, torch, dev, max(steps, 8))
        if split:
            ws = torch.zeros((arn.arnfp8_split_workspace_bytes(w.rows) // 8,), dtype=torch.int64,
                             device=dev)
            fn = rotating([split_call_on(w, d, arn, ws) for d in wins])
        else:
            fn = rotating([call_on(w, d, arn) for d in wins])
    # The inputs were just written by the generator: flush them out of the
    # caches, so that every profiled call reads its bytes from HBM.
    flush = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    flush.fill_(0x5A)
    torch.cuda.synchronize()
    del flush
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    log(f"profile workload {name}: {steps} calls")


# -------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=None,
                    help="input seed (default: the workload's own, 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true",
                    help="time the headline step only (no share, formats, latency or references)")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="first run one plain device copy of 1 GiB (scales the HBM counters)")
    ap.add_argument("--profile-workload", metavar="NAME",
                    help="run only NAME's calls (--steps of them), for rocprofv3")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="the workload a --summarize-* run describes")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--summarize-ktrace", metavar="DIR")
    ap.add_argument("--command", default="", help="the profiled command, for the summary")
    ap.add_argument("--split", action="store_true",
                    help="with --profile-workload / --summarize-*: the arnfp8_run_split calls")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, profile_path(args.workload, "hbm_traffic", args.split),
                      args.workload, args.command, args.split)
        return 0
    if args.summarize_ktrace:
        summarize_ktrace(args.summarize_ktrace,
                         profile_path(args.workload, "kernel_trace", args.split), args.command,
                         args.workload, args.split)
        return 0
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
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
    if args.profile_workload:
        profile_workload(args.profile_workload, torch, arn, dev, args.steps, args.split)
        return 0

    w = synth.WORKLOADS[DEFAULT_WORKLOAD]
    log(f"bench: workload {w.name}, steps {args.steps}, warmup {args.warmup}")
    n_out = out_sets_for(w)
    d = alloc_workload(w, torch, dev, out_sets=n_out, seed=args.seed)
    torch.cuda.synchronize()
    fn = step_fn(w, d, arn)
    ms_per_step, kern_ms, seg_ms = time_steps(torch, fn, args.steps, args.warmup, segments=5)
    alg = w.algorithmic_bytes()
    value = alg / (ms_per_step * 1e-3) / 1e9
    achieved = alg / (kern_ms * 1e-3) / 1e9
    log(f"bench: {ms_per_step * 1e3:.2f} us/step wall, {kern_ms * 1e3:.2f} us/launch (events), "
        f"segments {[round(x * 1e3, 2) for x in seg_ms]}")

    khash = kernel_source_hash()
    traffic = read_traffic(khash)
    k_trace = read_profile(profile_path(w.name, "kernel_trace"), "mean_us", khash)
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
        "io_dtypes": "bf16 in, bf16 residual out, e4m3fn + f32 scales out",
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
                     "kernel_us_median_of_5_segments": round(median(seg_ms) * 1e3, 3),
                     "kernel_us_segments": [round(x * 1e3, 3) for x in seg_ms],
                     "kernel_us_trace": k_trace,
                     "kernel_source_hash": khash},
    }
    if not args.no_latency:
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
        un_ms, _, _ = time_steps(torch, unfused, max(5, args.steps // 2), 3)
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
            _, f_k, _ = time_steps(torch, f, max(10, args.steps // 2), 3)
            fmt_out[f"{name}_us_per_call"] = round(f_k * 1e3, 2)
        result["formats"] = fmt_out
        del mx_scales
        # The residual updated in place (residual_out == residual_in), as a
        # transformer's residual stream is: each output set carries its own
        # residual copy, so the rotation still keeps every call out of cache.
        res_sets = [d["residual"].clone() for _ in d["outs"]]

        def in_place_one(o, r):
            return lambda: arn.arnfp8_run(d["inputs"], r, r, o["out"], o["scales"], d["gamma"],
                                          w.eps, w.weight_offset, w.scale_ub)
        _, ip_k, _ = time_steps(torch, rotating([in_place_one(o, r) for o, r in
                                                 zip(d["outs"], res_sets)]),
                                max(10, args.steps // 2), 3)
        result["in_place_residual"] = {"us_per_call": round(ip_k * 1e3, 2),
                                       "gbs": round(alg / (ip_k * 1e-3) / 1e9, 1)}
        del res_sets
        # The two-stage share (8 ranks of 1024 rows, the single-GPU half of the
        # large-payload path at its real shape): the ranks' calls in turn, each
        # reading other rows and writing its own staging slot (1.2 GB of
        # inputs per round of 8, so every call runs out of cache).  Replayed
        # from a graph: eager launches from Python are host-bound at this size.
        stg = [torch.empty((arn.arnfp8_stage_bytes(w.rows, w.cols, SHARE_NGPUS),),
                           dtype=torch.uint8, device=dev) for _ in range(SHARE_NGPUS)]
        calls = share_calls(w, d, arn, stg)
        sh_graph = graph_us_per_call(torch, calls * 4, reps=7)
        _, sh_eager, _ = time_steps(torch, rotating(calls), 4 * SHARE_NGPUS, SHARE_NGPUS)
        sb = share_bytes(w)
        sh_trace = read_profile(profile_path(SHARE_WORKLOAD, "kernel_trace"), "mean_us", khash)
        result["two_stage_share"] = {
            "ngpus": SHARE_NGPUS, "rank": "0-7 in turn", "rows": -(-w.rows // SHARE_NGPUS),
            "algorithmic_bytes": sb,
            "graph_us_per_call": round(sh_graph, 3),
            "eager_us_per_call": round(sh_eager * 1e3, 3),
            "roofline": {
                "bound": "hbm", "achieved": round(sb / (sh_graph * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(sb / (sh_graph * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "kernel_us_trace": sh_trace,
                "frac_kernel_trace": (round(sb / (sh_trace * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                      if sh_trace else None),
                "traffic": read_profile(profile_path(SHARE_WORKLOAD, "hbm_traffic"),
                                        "traffic_bytes_per_launch", khash)},
        }
        # The same shares with the residual updated in place (a copy of the
        # residual, so that the other measurements keep their inputs).
        res_copy = d["residual"].clone()
        sh_in_place = graph_us_per_call(torch, share_calls(w, d, arn, stg, res_copy) * 4, reps=7)
        del res_copy
        result["two_stage_share"]["in_place_residual"] = {
            "graph_us_per_call": round(sh_in_place, 3),
            "frac": round(sb / (sh_in_place * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        result["two_stage_share"]["reference_kernels"] = share_reference(w, d, torch, dev)
        log(f"bench: two-stage share {result['two_stage_share']}")
        del stg, calls
        result["reference_kernels"] = reference_kernels(w, d, torch, arn, dev, s_bufs)
        result["reference_kernels"]["fused_kernel_us"] = round(kern_ms * 1e3, 2)
        log(f"bench: reference kernels {result['reference_kernels']}")
        del s_bufs
        torch.cuda.empty_cache()
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "hbm_gib": round(props.total_memory / 2**30, 1)}
    if not args.no_latency:
        flush = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
        lat = {}
        for name in LATENCY_WORKLOADS:
            lat[name] = latency_figures(synth.WORKLOADS[name], torch, arn, dev, flush, khash)
            log(f"bench: latency {name} {lat[name]}")
        result["latency"] = lat
        result["decode_breakdown"] = {n: decode_breakdown(synth.WORKLOADS[n], torch, arn, dev, flush)
                                      for n in BREAKDOWN}
        log(f"bench: decode breakdown {result['decode_breakdown']}")
        result["exchange_cost"] = exchange_cost(torch, dev)
        log(f"bench: exchange cost {result['exchange_cost']}")
        result["latency_scaling_unit_offset_laws"] = latency_scaling(torch, arn, dev, flush)
        log(f"bench: latency scaling {result['latency_scaling_unit_offset_laws']}")
        del flush
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, d, torch)
        log(f"bench: cpu baseline {result['cpu_baseline']}")
        result["cpu_oracle_threaded"] = cpu_oracle_threaded(w, d, torch)
        log(f"bench: oracle on a thread pool {result['cpu_oracle_threaded']}")
        result["cpu_oracle_us_per_call"] = cpu_oracle_latency(LATENCY_WORKLOADS)
        log(f"bench: oracle per call on the small workloads {result['cpu_oracle_us_per_call']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
