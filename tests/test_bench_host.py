"""Host-side pieces of bench.py (no GPU): the kernel source hash that decides
whether the stored HBM-traffic summary still describes the kernel."""
import os
import shutil

import bench


def _copy_csrc(tmp_path):
    src = os.path.join(bench.ROOT, "varlen_top_select_amd", "csrc")
    dst = tmp_path / "csrc"
    shutil.copytree(src, dst)
    return dst


def test_hash_ignores_comments_and_whitespace(tmp_path):
    d = _copy_csrc(tmp_path)
    h0 = bench.kernel_source_hash(str(d))
    p = d / "vts_kernels.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n" + text.replace("\n", "\n  ", 3) + "\n/* block\n comment */\n")
    assert bench.kernel_source_hash(str(d)) == h0


def test_hash_changes_with_code(tmp_path):
    d = _copy_csrc(tmp_path)
    h0 = bench.kernel_source_hash(str(d))
    p = d / "vts_device.hpp"
    text = p.read_text()
    assert "constexpr int NT = 256;" in text
    p.write_text(text.replace("constexpr int NT = 256;", "constexpr int NT = 512;"))
    assert bench.kernel_source_hash(str(d)) != h0


def test_hash_covers_every_kernel_file(tmp_path):
    d = _copy_csrc(tmp_path)
    h0 = bench.kernel_source_hash(str(d))
    for name in bench.KERNEL_SOURCES:
        p = d / name
        text = p.read_text()
        p.write_text(text + "\nstatic int hash_probe_extra_symbol;\n")
        assert bench.kernel_source_hash(str(d)) != h0, name
        p.write_text(text)
    assert bench.kernel_source_hash(str(d)) == h0


def test_stored_traffic_only_for_matching_hash():
    assert bench.stored_traffic("0000000000000000") is None
