"""Builds the HIP library libvts.so (gfx950) in-tree with hipcc."""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvts.so")
SOURCES = ["vts_kernels.hip", "vts_api.hip"]
PROBE_LIB = os.path.join(HERE, "libvts_probe.so")
PROBE_SOURCES = ["vts_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
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
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise subprocess.CalledProcessError(res.returncode, cmd)
    _check_resources(res.stderr, out)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Builds libvts.so (the top-k library) and libvts_probe.so (measurement probes)."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
