"""Builds the HIP library libvts.so (gfx950) in-tree with hipcc."""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvts.so")
# compiled separately and in parallel, linked in this order (the first two are
# the kernels' code objects: any-order kernels, the deterministic mode, top_k
# above 2048)
SOURCES = ["vts_kernels.hip", "vts_kernels_ordered.hip", "vts_kernels_wide.hip",
           "vts_kernels_hint.hip", "vts_api.hip"]
PROBE_LIB = os.path.join(HERE, "libvts_probe.so")
PROBE_SOURCES = ["vts_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

OBJDIR = os.path.join(HERE, "_build")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The top-k kernels are sized for four workgroups of four waves per compute
# unit (every row of a 1024-row batch resident at once) and must not spill:
# the compiler's resource remarks are checked on every build.
MIN_WAVES_PER_SIMD = 4


def _check_resources(remarks: str, out: str) -> None:
    name = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        if name is None or "topk_kernel" not in name:
            continue
        m = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and int(m.group(1)) < MIN_WAVES_PER_SIMD:
            raise RuntimeError(f"{out}: {name} fits only {m.group(1)} waves per SIMD")
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            raise RuntimeError(f"{out}: {name} spills {m.group(1)} bytes per lane to scratch")


def _compile(sources, out, verbose):
    """Compiles each source to an object (all at once), checks the kernels'
    resource remarks, and links the objects into the shared library `out`."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = []
    for src in sources:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, obj, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
    failed = None
    for cmd, obj, proc in jobs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(err)
            failed = failed or subprocess.CalledProcessError(proc.returncode, cmd)
            continue
        _check_resources(err, out)
    if failed:
        raise failed
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _ in jobs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Builds libvts.so (the top-k library) and libvts_probe.so (measurement probes)."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
