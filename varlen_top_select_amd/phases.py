"""Phase timing of the top-k kernel: where one call's time goes, per row unit.

Builds (``--build``, on any host with hipcc) a copy of the library compiled
with -DVTS_PHASE_STAMPS, ``libvts_phases.so``: thread 0 of every row unit
stamps the GPU's 100 MHz real-time counter at its start, when its window is
known, when its rungs are ready, when its stream has ended, when its final
selection starts, when that selection knows the k-th key, when its outputs
are written and when it took its split-row ticket.  Run (on the GPU) with
workload names (workloads.make): one untimed call, then a cold call (after a
512 MB read flush) and a warm call with stamps; prints percentiles of each
phase over the units, in microseconds from the first unit's start.

    python -m varlen_top_select_amd.phases --build
    python -m varlen_top_select_amd.phases long dsv32 dsv4_mtp page
    python -m varlen_top_select_amd.phases --tune resident=1 page   # a switch of vts_set_tuning
    python -m varlen_top_select_amd.phases --lib other/libvts_phases.so page  # another stamped build

The stamped kernel is not the product kernel (the stamps add a few stores);
the product build never defines the macro.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libvts_phases.so")
PER_UNIT = 16  # stamps per unit (slots 6 and 7: hardware id, row and length)


def build(out: str = LIB) -> str:
    # The stamps take registers: a stamped kernel may fit fewer waves per
    # SIMD than the product's (not refused here; its timings are then those
    # of a lower occupancy).
    from . import build as b
    saved = (b.FLAGS, b.OBJDIR, b.MIN_WAVES_PER_SIMD)
    b.FLAGS = saved[0] + ["-DVTS_PHASE_STAMPS"]
    b.OBJDIR = os.path.join(HERE, "_build_phases")
    b.MIN_WAVES_PER_SIMD = 1
    try:
        b._compile(b.SOURCES, out, verbose=True)
    finally:
        b.FLAGS, b.OBJDIR, b.MIN_WAVES_PER_SIMD = saved
    return out


def _pct(a) -> str:
    a = np.asarray(a, np.float64)
    a = a[np.isfinite(a)]
    if a.size == 0:
        return "-"
    q = np.percentile(a, [0, 10, 50, 90, 100])
    return "p0 %6.1f  p10 %6.1f  p50 %6.1f  p90 %6.1f  max %6.1f" % tuple(q)


def report(name: str, st: np.ndarray, event_us: float) -> None:
    st = st.reshape(-1, PER_UNIT).astype(np.int64)
    st = st[st[:, 0] > 0]
    t0 = st[:, 0].min()
    us = lambda i: np.where(st[:, i] > 0, (st[:, i] - t0) / 100.0, np.nan)  # 100 MHz ticks
    s = {i: us(i) for i in (0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 14, 15)}
    n = (st[:, 7] >> 32).astype(np.int64)
    print(f"== {name}: {st.shape[0]} units, kernel time by events {event_us:.1f} us")
    print("  unit start            ", _pct(s[0]))
    print("  window known          ", _pct(s[1]))
    print("  window -> rungs       ", _pct(s[2] - s[1]))
    print("    window -> sample in ", _pct(s[15] - s[1]))
    print("    sample in -> rungs  ", _pct(s[2] - s[15]))
    print("  rungs -> stream end   ", _pct(s[3] - s[2]))
    print("  stream end -> written ", _pct(s[4] - s[3]))
    print("    stream end -> select", _pct(s[8] - s[3]))
    print("    stream end -> publish", _pct(s[11] - s[3]))
    print("    publish -> stored   ", _pct(s[12] - s[11]))
    print("    stored -> ticket    ", _pct(s[5] - s[12]))
    print("    ticket -> counts    ", _pct(s[10] - s[5]))
    print("    counts -> select    ", _pct(s[8] - s[10]))
    print("    select -> k-th key  ", _pct(s[9] - s[8]))
    print("    k-th key -> written ", _pct(s[4] - s[9]))
    print("      k-th -> tickets   ", _pct(s[13] - s[9]))
    print("      tickets -> table  ", _pct(s[14] - s[13]))
    print("      table -> written  ", _pct(s[4] - s[14]))
    print("  rungs ready at        ", _pct(s[2]))
    print("  stream end at         ", _pct(s[3]))
    print("  ticket at             ", _pct(s[5]))
    print("  outputs written at    ", _pct(s[4]))
    short = np.isnan(s[2]) & np.isfinite(s[4])
    print(f"  units answered without a stream (short, direct or idle): {int(short.sum())}")
    big = np.isfinite(s[3]) & (n > 0)
    if big.any():
        print("  valid columns of streamed units", _pct(n[big]))


def main(argv) -> None:
    if argv and argv[0] == "--build":
        print(build())
        return
    lib_path = LIB
    if argv and argv[0] == "--lib":  # another stamped build of the library
        lib_path, argv = argv[1], argv[2:]
    tune = {}
    while argv and argv[0] == "--tune":
        key, val = argv[1].split("=")
        tune[key] = int(val)
        argv = argv[2:]
    sys.path.insert(0, ROOT)
    import torch

    import bench
    import varlen_top_select_amd as vts
    import workloads

    vts.LIB_PATH = lib_path
    lib = vts.library()
    lib.vts_phase_stamps.argtypes = [ctypes.c_void_p]
    for key, val in tune.items():
        vts.set_tuning(getattr(vts, "TUNE_" + key.upper()), val)
    for name in argv or ["long", "dsv32", "dsv4_mtp", "page"]:
        wl = workloads.make(name)
        step, ws = bench.make_step(wl, torch, vts)
        units = 1 << 16
        stamps = torch.zeros(units * PER_UNIT, dtype=torch.int64, device="cuda")
        step()
        torch.cuda.synchronize()
        flush = bench.Flusher(torch)
        for mode in ("cold", "warm"):
            if mode == "cold":
                flush()
            stamps.zero_()
            torch.cuda.synchronize()
            lib.vts_phase_stamps(stamps.data_ptr())
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            lib.vts_phase_stamps(None)
            label = " ".join([name, mode] + [f"{k}={v}" for k, v in tune.items()])
            report(label, stamps.cpu().numpy(), a.elapsed_time(b) * 1000.0)
        sys.stdout.flush()


if __name__ == "__main__":
    main(sys.argv[1:])
