"""Benchmark of exact variable-length top-K selection on one MI355X.

Default workload: the long-row decode batch -- 1024 rows x 262144 fp32 logits,
top_k 2048, seq_lens U[131072, 262144] with 5 % of rows longer than the width
(clamped), spiky N(0,1) values, previous-step hint (workloads/synth.py,
"long").  One step = one topk_varlen call over the whole batch (prologue,
sampled threshold, streaming filter, selection, epilogue: the entire path).

Prints ONE JSON line:
  value       valid-logits GB/s of the timed steps (inputs resident in HBM):
              sum_r n_r * 4 bytes / (wall time per step)
  roofline    the top-k kernel against MI355X HBM peak (8 TB/s): algorithmic
              bytes per launch / mean kernel time from HIP events recorded on
              the launch stream over the timed region; `traffic` from the
              committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary when it was
              taken on the current kernel source, else null
  cold        per-call µs after a 512 MB cache flush (median, p10, p90)
  ceiling     a plain 16-byte streaming read of the same number of bytes
  cpu_baseline the CPU oracle timed on a bounded sample of the same batch
  others      µs/call of the other four workloads (smaller, latency-bound)

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 10]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
FLUSH_BYTES = 512 << 20  # larger than the 256 MB last-level cache plus the L2s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def valid_lengths(wl) -> np.ndarray:
    """Valid columns per row (measurement denominator)."""
    R = wl.rows
    if wl.kind == "varlen":
        r = np.arange(R)
        seq = wl.seq_lens.astype(np.int64)[r // wl.next_n]
        num = seq - wl.next_n + (r % wl.next_n) + 1
        n = np.where(num <= 0, 0, num // wl.compress_ratio)
        return np.minimum(n, wl.width)
    start = wl.row_starts.astype(np.int64)
    return np.clip(wl.lengths.astype(np.int64), 0, wl.width - start)


def _code_only(text: str) -> str:
    """Source text without comments and whitespace (a comment edit is not a kernel change)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


KERNEL_SOURCES = ("vts_device.hpp", "vts_internal.h", "vts_topk.hpp", "vts_kernels.hip")


def kernel_source_hash(csrc: str | None = None) -> str:
    """Hash of the code that defines the top-k kernel (comments and whitespace
    excluded; the host-side plan and argument checks are not part of it)."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "varlen_top_select_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def upload(wl, torch):
    dt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}[wl.dtype]
    raw = torch.from_numpy(wl.x.view(np.int32 if wl.dtype == 0 else np.int16)).cuda()
    return raw.view(dt)[:, : wl.width], dt


def make_step(wl, torch, vts, hint: bool = True, ragged: bool = False, page1: bool = False,
              tie: str | None = None):
    """Returns (step, workspace) for one call of the whole batch (with `tie`,
    the deterministic mode of the varlen selection)."""
    x, dt = upload(wl, torch)
    R, k = wl.rows, wl.k
    if wl.kind == "varlen":
        seq = torch.from_numpy(wl.seq_lens).cuda()
        idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
        vals = torch.empty((R, k), dtype=dt, device="cuda") if wl.return_values else None
        pre = torch.from_numpy(wl.pre_idx).cuda() if (hint and wl.pre_idx is not None) else None
        ws = vts.make_workspace(R, wl.width, k, dt, "cuda")

        def step():
            if tie is None:
                vts.topk_varlen(x, seq, k, pre_idx=pre, compress_ratio=wl.compress_ratio,
                                next_n=wl.next_n, return_values=wl.return_values, out_indices=idx,
                                out_values=vals, workspace=ws)
            else:
                vts.topk_varlen_ordered(x, seq, k, tie_break=tie, pre_idx=pre,
                                        compress_ratio=wl.compress_ratio, next_n=wl.next_n,
                                        return_values=wl.return_values, out_indices=idx,
                                        out_values=vals, workspace=ws)
        return step, ws
    L = torch.from_numpy(wl.lengths).cuda()
    rs = torch.from_numpy(wl.row_starts).cuda()
    if ragged:  # the same windows, each row's indices offset into a ragged KV buffer
        off = torch.from_numpy((np.arange(R, dtype=np.int64) * wl.width).astype(np.int32)).cuda()
        o = torch.empty((R, k), dtype=torch.int32, device="cuda")
        ws = vts.make_workspace(R, wl.width, k, dt, "cuda", transform=True)

        def rstep():
            vts.topk_transform_ragged(x, L, off, k, row_starts=rs, out=o, workspace=ws)
        return rstep, ws
    if page1:  # the same windows, one row per request, a page-size-1 table per request
        g = np.random.default_rng(7)
        pt1 = torch.from_numpy(g.integers(0, 1 << 30, size=(R, wl.width), dtype=np.int32)).cuda()
        cu = torch.arange(R + 1, dtype=torch.int32, device="cuda")
        o = torch.empty((R, k), dtype=torch.int32, device="cuda")
        ws = vts.make_workspace(R, wl.width, k, dt, "cuda", transform=True)

        def pstep():
            vts.topk_transform_page1(x, L, pt1, cu, k, row_starts=rs, out=o, workspace=ws)
        return pstep, ws
    pt = torch.from_numpy(wl.page_table).cuda()
    pr = torch.from_numpy(wl.page_table_row_starts).cuda()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    raw = torch.empty((R, k), dtype=torch.int32, device="cuda")
    ws = vts.make_workspace(R, wl.width, k, dt, "cuda", transform=True)

    def step():
        vts.topk_page_table_transform(x, L, pt, k, page_size=wl.page_size, row_starts=rs,
                                      page_table_row_starts=pr, out=out, out_raw_indices=raw,
                                      workspace=ws)
    return step, ws


def algorithmic_bytes(wl, n: np.ndarray) -> int:
    """Bytes the path must move per call: valid logits once, the outputs, the lengths."""
    isz = 4 if wl.dtype == 0 else 2
    b = int(n.sum()) * isz + wl.rows * wl.k * 4
    if wl.kind == "varlen":
        b += (wl.rows // wl.next_n) * 4
        if wl.return_values:
            b += wl.rows * wl.k * isz
    else:
        b += wl.rows * 4 * 3 + wl.rows * wl.k * 4  # lengths, starts, page starts; out_raw
    return b


class Flusher:
    """Evicts the caches by READING a 512 MB buffer (a write flush would leave
    dirty lines whose write-back lands inside the timed call)."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
        path = os.path.join(ROOT, "varlen_top_select_amd", "libvts_probe.so")
        self.lib = None
        if os.path.exists(path):
            self.lib = ctypes.CDLL(path)
            self.lib.vts_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                ctypes.c_void_p]

    def __call__(self):
        if self.lib is not None:
            self.lib.vts_probe_read(self.buf.data_ptr(), FLUSH_BYTES, self.sink.data_ptr(),
                                    self.torch.cuda.current_stream().cuda_stream)
        else:
            self.sink[0] = self.buf.sum()


def cold_times(step, torch, reps: int) -> np.ndarray:
    flush = Flusher(torch)
    ts = []
    for i in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1000.0)
    del flush
    return np.array(ts)


def read_ceiling(nbytes: int, torch) -> float | None:
    """GB/s of a plain 16-byte streaming read of nbytes (cold), median of 5."""
    path = os.path.join(ROOT, "varlen_top_select_amd", "libvts_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.vts_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = (nbytes // 16) * 16
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    flush = Flusher(torch)
    s = torch.cuda.current_stream().cuda_stream
    ts = []
    for i in range(6):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rc = lib.vts_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), s)
        b.record()
        torch.cuda.synchronize()
        if rc != 0:
            return None
        if i:
            ts.append(a.elapsed_time(b) * 1e-3)
    return nbytes / float(np.median(ts)) / 1e9


def launch_floor(torch, reps: int = 20) -> float | None:
    """Cold median µs of the smallest launch: one workgroup reading 16 bytes,
    timed like the workloads (read flush, one event pair around the call)."""
    path = os.path.join(ROOT, "varlen_top_select_amd", "libvts_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.vts_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    ts = cold_times(lambda: lib.vts_probe_read(buf.data_ptr(), 16, sink.data_ptr(), s), torch, reps)
    return float(np.median(ts))


def stored_traffic(src_hash: str):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", "topk_long_batch_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(wl, n: np.ndarray, budget_s: float = 12.0):
    """The CPU oracle as it stands on a bounded sample of rows (median of 3 runs)."""
    import oracle

    threads = oracle.default_threads()
    rows = 16
    base = np.zeros(wl.rows, np.int64)
    xb = wl.x[:, : wl.width]
    # grow the sample until one run costs about budget/3 seconds of wall time
    while True:
        sel = slice(0, rows)
        t0 = time.perf_counter()
        oracle.select(xb[sel], wl.dtype, base[sel], n[sel], wl.k, False, threads)
        dt = time.perf_counter() - t0
        if dt > budget_s / 6 or rows >= wl.rows:
            break
        rows = min(wl.rows, rows * 2)
    runs = [dt]
    for _ in range(2):
        t0 = time.perf_counter()
        oracle.select(xb[:rows], wl.dtype, base[:rows], n[:rows], wl.k, False, threads)
        runs.append(time.perf_counter() - t0)
    t = float(np.median(runs))
    isz = 4 if wl.dtype == 0 else 2
    vb = int(n[:rows].sum()) * isz
    return {"value": round(vb / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {wl.rows} rows ({vb / 1e6:.1f} MB valid logits), full sort per "
                      f"row, median of 3 runs, {t * 1e3:.0f} ms per run",
            "us_per_row": round(t / rows * 1e6, 1)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long",
                    choices=["small", "dsv32", "long", "dsv4_mtp", "page"])
    ap.add_argument("--no-hint", action="store_true", help="do not pass the workload's hint")
    ap.add_argument("--hint-rung", action="store_true",
                    help="bound the threshold by the hint too (diagnostic switch; off by default)")
    ap.add_argument("--cold-reps", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--only-steps", action="store_true",
                    help="time the steps only (for profiler runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="also run one plain copy of MB megabytes (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this selection path runs on a single MI355X; "
              "rows are independent, so a multi-GPU run would shard them by rows (balanced by "
              "valid length) with no exchange between GPUs.",
              file=sys.stderr)
        return 2

    import torch

    import varlen_top_select_amd as vts
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"generating workload {args.workload}")
    wl = workloads.make(args.workload, hint=not args.no_hint)
    n = valid_lengths(wl)
    isz = 4 if wl.dtype == 0 else 2
    valid = int(n.sum()) * isz
    alg = algorithmic_bytes(wl, n)
    if args.hint_rung:
        vts.set_tuning(vts.TUNE_HINT_RUNG, 1)
    step, ws = make_step(wl, torch, vts, hint=not args.no_hint)
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    vts.workspace_stats(ws)  # clear counters

    log(f"timing {args.steps} steps")
    # One event pair on the launch stream brackets the K back-to-back calls: an
    # event recorded between two launches holds the second back by several
    # microseconds.  The per-launch mean is the bracketed time over K, so any
    # gap between launches counts as kernel time (a bound from above).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stats = vts.workspace_stats(ws)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_us_mean = ev0.elapsed_time(ev1) * 1e3 / args.steps
    value = valid / (ms_per_step * 1e-3) / 1e9
    achieved = alg / (kern_us_mean * 1e-6) / 1e9
    src_hash = kernel_source_hash()
    traffic = stored_traffic(src_hash)

    line = {
        "metric": "µs/call and HBM GB/s (valid logits bytes) at N=262144,k=2048 vs roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "bf16", 2: "f16"}[wl.dtype],
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.rows}x{wl.width} "
                               f"{ {0: 'fp32', 1: 'bf16', 2: 'fp16'}[wl.dtype]}, top_k {wl.k}",
                   "rows": wl.rows, "width": wl.width, "top_k": wl.k,
                   "hint": ("passed, not read" if not args.hint_rung else "passed, hint rung on")
                           if (not args.no_hint) and wl.pre_idx is not None else False,
                   "valid_logits_bytes": valid, "parallelism": "1 GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "topk_kernel",
                     "algorithmic_bytes_per_launch": alg,
                     "kernel_us_mean": round(kern_us_mean, 2),
                     "valid_bytes_frac_of_peak": round(valid / (kern_us_mean * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "kernel_source_hash": src_hash},
        "events": {"refiltered_workgroups": stats[0], "whole_row_reselections": stats[1],
                   "spilled_rows": stats[2], "full_list_selections": stats[3]},
    }
    if args.calibrate_copy:
        nb = args.calibrate_copy << 20
        src = torch.ones(nb // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        plib = ctypes.CDLL(os.path.join(ROOT, "varlen_top_select_amd", "libvts_probe.so"))
        plib.vts_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
        Flusher(torch)()
        plib.vts_probe_copy(dst.data_ptr(), src.data_ptr(), nb,
                            torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = nb
        del src, dst
    if args.only_steps:
        print(json.dumps(line), flush=True)
        return 0

    log("cold protocol")
    ct = cold_times(step, torch, args.cold_reps)
    line["cold"] = {"us_median": round(float(np.median(ct)), 2),
                    "us_p10": round(float(np.percentile(ct, 10)), 2),
                    "us_p90": round(float(np.percentile(ct, 90)), 2),
                    "valid_GBps_median": round(valid / (np.median(ct) * 1e-6) / 1e9, 1),
                    "flush": f"read of {FLUSH_BYTES >> 20} MB before each call"}
    log("read ceiling")
    ceil = read_ceiling(valid, torch)
    if ceil:
        line["ceiling"] = {"plain_read_GBps": round(ceil, 1),
                           "kernel_frac_of_read_ceiling": round(achieved / ceil, 4)}
    del step, ws
    torch.cuda.empty_cache()
    if args.hint_rung:
        vts.set_tuning(vts.TUNE_HINT_RUNG, 0)

    if not args.no_others:
        others = {}
        for name in ("small", "dsv32", "long", "dsv4_mtp", "page", "page_ragged", "page_page1",
                     "long_ordered", "dsv4_mtp_ordered", "long_k16384"):
            if name == args.workload:
                continue
            log(f"workload {name}")
            base_name = name.split("_")[0] if name.startswith(("page", "long")) else name
            base_name = "dsv4_mtp" if name.startswith("dsv4_mtp") else base_name
            w2 = workloads.make(base_name)
            if name == "long_k16384":  # top_k at the end of radix_filter's range
                w2.k, w2.pre_idx = 16384, None
            n2 = valid_lengths(w2)
            s2, ws2 = make_step(w2, torch, vts, ragged=name.endswith("_ragged"),
                                page1=name.endswith("_page1"),
                                tie="small" if name.endswith("_ordered") else None)
            for _ in range(10):
                s2()
            ct2 = cold_times(s2, torch, args.cold_reps)
            vb2 = int(n2.sum()) * (4 if w2.dtype == 0 else 2)
            others[name] = {
                "us_median_cold": round(float(np.median(ct2)), 2),
                "valid_GBps": round(vb2 / (np.median(ct2) * 1e-6) / 1e9, 1),
                "valid_bytes": vb2}
            del s2, ws2
        lf = launch_floor(torch)
        if lf is not None:
            others["launch_floor"] = {"us_median_cold": round(lf, 2),
                                      "what": "one workgroup reading 16 bytes, same protocol"}
        line["others"] = others

    if not args.no_cpu:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(wl, n)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
