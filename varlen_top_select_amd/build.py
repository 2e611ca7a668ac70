"""Builds the HIP library libvts.so (gfx950) in-tree with hipcc."""
import os
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


def _compile(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
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
