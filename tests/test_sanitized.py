"""The CPU oracle and the C ABI's host side under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only: no GPU code is built with them).

tests/sanitize/oracle_battery.c drives oracle/vts_oracle.c (gcc); 
tests/sanitize/host_battery.cpp drives the argument checks, plans and
workspace sizing of varlen_top_select_amd/csrc/vts_api.hip (it holds no
kernels: its device side is the scratch array alone), with the sanitizers on
the host side only (after -Xarch_host) and stand-ins for the kernel launches.  Each must run clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_battery"
    b = _run(["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
              os.path.join(ROOT, "oracle", "vts_oracle.c"), os.path.join(SAN, "oracle_battery.c"),
              "-o", str(exe), "-lm"])
    assert b.returncode == 0, b.stderr
    r = _run([str(exe)], env=ENV, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "oracle battery clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_side_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_battery"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    b = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              os.path.join(ROOT, "varlen_top_select_amd", "csrc", "vts_api.hip"),
              os.path.join(SAN, "host_battery.cpp"), "-o", str(exe)])
    assert b.returncode == 0, b.stderr[-4000:]
    r = _run([str(exe)], env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "host battery clean" in r.stdout
