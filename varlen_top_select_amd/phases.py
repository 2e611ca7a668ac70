"""Phase timing of the top-k kernel: where one call's time goes, per row unit.

Builds (``--build``, on any host with hipcc) a copy of the library compiled
with -DVTS_PHASE_STAMPS, ``libvts_phases.so``: thread 0 of every row unit
stamps the GPU's 100 MHz real-time counter at its start, when its window is
known, when its rungs are ready, when its stream has ended, when its outputs
are written and when it took its split-row ticket.  Run (on the GPU) with
workload names (workloads.make): one untimed call, then a cold call (after a
512 MB read flush) and a warm call with stamps; prints percentiles of each
phase over the units, in microseconds from the first unit's start.

    python -m varlen_top_select_amd.phases --build
    python -m varlen_top_select_amd.phases long dsv32 dsv4_mtp page
    python -m varlen_top_select_amd.phases --tune resident=1 page   # a switch of vts_set_tuning

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


def build() -> str:
    from . import build as b
    saved = (b.FLAGS, b.OBJDIR)
    b.FLAGS = saved[0] + ["-DVTS_PHASE_STAMPS"]
    b.OBJDIR = os.path.join(HERE, "_build_phases")
    try:
        b._compile(b.SOURCES, LIB, verbose=True)
    finally:
        b.FLAGS, b.OBJDIR = saved
    return LIB


def _pct(a) -> str:
    a = np.asarray(a, np.float64)
    a = a[np.isfinite(a)]
    if a.size == 0:
        return "-"
    q = np.percentile(a, [0, 10, 50, 90, 100])
    return "p0 %6.1f  p10 %6.1f  p50 %6.1f  p90 %6.1f  max %6.1f" % tuple(q)


def report(name: str, st: np.ndarray, event_us: float) -> None:
    st = st.reshape(-1, 8).astype(np.int64)
    st = st[st[:, 0] > 0]
    t0 = st[:, 0].min()
    us = lambda i: np.where(st[:, i] > 0, (st[:, i] - t0) / 100.0, np.nan)  # 100 MHz ticks
    s = {i: us(i) for i in range(6)}
    n = (st[:, 7] >> 32).astype(np.int64)
    print(f"== {name}: {st.shape[0]} units, kernel time by events {event_us:.1f} us")
    print("  unit start            ", _pct(s[0]))
    print("  window known          ", _pct(s[1]))
    print("  window -> rungs       ", _pct(s[2] - s[1]))
    print("  rungs -> stream end   ", _pct(s[3] - s[2]))
    print("  stream end -> written ", _pct(s[4] - s[3]))
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

    vts.LIB_PATH = LIB
    lib = vts.library()
    lib.vts_phase_stamps.argtypes = [ctypes.c_void_p]
    for key, val in tune.items():
        vts.set_tuning(getattr(vts, "TUNE_" + key.upper()), val)
    for name in argv or ["long", "dsv32", "dsv4_mtp", "page"]:
        wl = workloads.make(name)
        step, ws = bench.make_step(wl, torch, vts)
        units = 1 << 16
        stamps = torch.zeros(units * 8, dtype=torch.int64, device="cuda")
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
