"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/vts.h declares, and its host-side argument checks return the documented
status codes before any HIP call (fake pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import varlen_top_select_amd as vts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vts.h")

OK, WARN, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, -1, -2, -3, -4
A = 1 << 20  # fake, 16-byte aligned "device" addresses (never touched)


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vts.LIB_PATH):
        from varlen_top_select_amd import build
        build.build()
    return vts.library()


def test_header_declares_the_two_operations():
    names = declared_functions()
    for n in ("vts_topk_varlen", "vts_topk_page_table_transform", "topk_varlen",
              "topk_page_table_transform", "vts_topk_varlen_workspace_bytes",
              "vts_page_transform_workspace_bytes", "vts_workspace_init", "vts_status_string",
              "vts_workspace_stats", "vts_set_tuning"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", vts.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_probe_library_exports_its_header():
    probe_h = os.path.join(ROOT, "include", "vts_probe.h")
    path = os.path.join(ROOT, "varlen_top_select_amd", "libvts_probe.so")
    if not os.path.exists(path):
        from varlen_top_select_amd import build
        build.build()
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    names = declared_functions(probe_h)
    assert names == ["vts_probe_copy", "vts_probe_read"]
    for n in names:
        assert n in exported


def test_every_header_is_covered():
    heads = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert heads == ["vts.h", "vts_probe.h"]


def test_status_strings(lib):
    for s in (OK, WARN, INVALID, UNSUPPORTED, WORKSPACE, HIP):
        assert lib.vts_status_string(s)
    assert lib.vts_status_string(12345) == b"unknown status"


def test_workspace_size_is_a_pure_function_of_shape(lib):
    a = lib.vts_topk_varlen_workspace_bytes(1024, 262144, 2048, 0)
    b = lib.vts_topk_varlen_workspace_bytes(1024, 262144, 2048, 0)
    assert a == b and a >= 256 and a % 256 == 0
    assert lib.vts_topk_varlen_workspace_bytes(0, 10, 1, 0) == 256
    # more rows never need less
    assert lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0) <= \
        lib.vts_topk_varlen_workspace_bytes(128, 163840, 2048, 0)


def _varlen(lib, **kw):
    args = dict(logits=A, dtype=0, num_rows=8, width=4096, row_stride=4096, seq_lens=A,
                top_k=512, next_n=1, cr=1, pre_idx=None, out=A, vals=None, ws=A,
                ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return lib.vts_topk_varlen(args["logits"], args["dtype"], args["num_rows"], args["width"],
                               args["row_stride"], args["seq_lens"], args["top_k"], args["next_n"],
                               args["cr"], args["pre_idx"], args["out"], args["vals"], args["ws"],
                               args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=3), INVALID),
    (dict(dtype=-1), INVALID),
    (dict(num_rows=-1), INVALID),
    (dict(width=0), INVALID),
    (dict(row_stride=100), INVALID),
    (dict(top_k=0), INVALID),
    (dict(top_k=16385), UNSUPPORTED),
    (dict(width=1 << 31, row_stride=1 << 31), UNSUPPORTED),
    (dict(width=1 << 29, row_stride=1 << 29), UNSUPPORTED),   # 2^31 bytes of fp32
    (dict(dtype=1, width=1 << 30, row_stride=1 << 30), UNSUPPORTED),
    (dict(logits=None), INVALID),
    (dict(logits=A + 2), INVALID),          # not aligned to 4-byte fp32 elements
    (dict(seq_lens=None), INVALID),
    (dict(next_n=0), INVALID),
    (dict(next_n=3), INVALID),              # 8 rows not a multiple of 3
    (dict(cr=0), INVALID),
    (dict(out=None), INVALID),
    (dict(out=A + 4), INVALID),             # not 16-byte aligned
    (dict(vals=A + 8), INVALID),
    (dict(vals=A + 4096), INVALID),         # overlaps out_indices (8 x 512 x 4 bytes)
    (dict(ws=None), WORKSPACE),
    (dict(ws=A + 8), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE),
])
def test_varlen_argument_errors(lib, kw, want):
    assert _varlen(lib, **kw) == want


def test_varlen_zero_rows_is_a_no_op(lib):
    assert _varlen(lib, num_rows=0, logits=None, seq_lens=None, out=None, ws=None) == OK


def _transform(lib, **kw):
    args = dict(scores=A, dtype=2, num_rows=4, width=1024, row_stride=1040, lengths=A,
                row_starts=None, pt=A, pt_stride=32, pt_width=32, ptrs=None, page_size=64,
                top_k=256, out=A, raw=None, ws=A, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return lib.vts_topk_page_table_transform(
        args["scores"], args["dtype"], args["num_rows"], args["width"], args["row_stride"],
        args["lengths"], args["row_starts"], args["pt"], args["pt_stride"], args["pt_width"],
        args["ptrs"], args["page_size"], args["top_k"], args["out"], args["raw"], args["ws"],
        args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(page_size=0), INVALID),
    (dict(page_size=(1 << 30) + 1), INVALID),
    (dict(pt_width=0), INVALID),
    (dict(pt_stride=16), INVALID),
    (dict(row_starts=A), INVALID),          # page_size > 1 with row_starts needs ptrs
    (dict(lengths=None), INVALID),
    (dict(pt=None), INVALID),
    (dict(out=None), INVALID),
    (dict(raw=A + 8), INVALID),
    (dict(raw=A + 1024), INVALID),          # overlaps out (4 x 256 x 4 bytes)
    (dict(scores=A + 1), INVALID),          # not aligned to 2-byte fp16 elements
    (dict(top_k=16385), UNSUPPORTED),
    (dict(ws_bytes=0), WORKSPACE),
])
def test_transform_argument_errors(lib, kw, want):
    assert _transform(lib, **kw) == want


def test_workspace_second_workgroups(lib):
    """512 rows whose windows can hold 128 KB get two units per row in the
    workspace (the length-balanced placement cuts long rows into units of at
    least 128 KB, at most 1024 units in all); narrower rows, other row counts
    and the placement switched off keep one."""
    vb = lib.vts_topk_varlen_workspace_bytes
    two = vb(512, 65536, 1024, 1)      # bf16: 65536 columns are 128 KB
    narrow = vb(512, 65535, 1024, 1)
    assert two > narrow
    assert vb(512, 32768, 1024, 0) > vb(512, 32767, 1024, 0)  # fp32: 32768 columns
    assert vb(768, 262144, 1024, 1) == vb(768, 1024, 1024, 1)  # 768 rows: one unit each
    assert lib.vts_set_tuning(vts.TUNE_NO_BALANCE, 1) == OK
    try:
        assert vb(512, 65536, 1024, 1) < two
    finally:
        assert lib.vts_set_tuning(vts.TUNE_NO_BALANCE, 0) == OK


def test_tuning_switches(lib):
    assert lib.vts_set_tuning(99, 0) == INVALID
    assert lib.vts_set_tuning(vts.TUNE_NSPLIT, 33) == INVALID
    assert lib.vts_set_tuning(vts.TUNE_FORCE_PATH, 3) == INVALID
    assert lib.vts_set_tuning(vts.TUNE_LDS_SLOTS, 10) == INVALID
    assert lib.vts_set_tuning(vts.TUNE_LDS_SLOTS, 3841) == INVALID
    assert lib.vts_set_tuning(vts.TUNE_NO_BALANCE, 2) == INVALID
    assert lib.vts_set_tuning(vts.TUNE_HINT_RUNG, 2) == INVALID
    for key in (vts.TUNE_NSPLIT, vts.TUNE_FORCE_PATH, vts.TUNE_LDS_SLOTS, vts.TUNE_SPILL_SLOTS,
                vts.TUNE_SAMPLE_SIGMA, vts.TUNE_NO_BALANCE):
        assert lib.vts_set_tuning(key, 0) == OK
    # the forced split count changes the workspace size accordingly
    base = lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0)
    assert lib.vts_set_tuning(vts.TUNE_NSPLIT, 1) == OK
    one = lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0)
    assert lib.vts_set_tuning(vts.TUNE_NSPLIT, 0) == OK
    assert one < base


def test_valid_call_without_a_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; fake pointers must not reach a launch")
    assert _varlen(lib) == HIP


@pytest.mark.parametrize("tie", [0, 3, 4, 8, 5 | 8, -1])
def test_ordered_entry_points_reject_bad_tie_breaks(lib, tie):
    v = lib.vts_topk_varlen_ordered(A, 0, 8, 4096, 4096, A, 512, 1, 1, None, A, None, A, 1 << 40,
                                    None, tie)
    p = lib.vts_topk_page_table_transform_ordered(A, 2, 4, 1024, 1040, A, None, A, 32, 32, None,
                                                  64, 256, A, None, A, 1 << 40, None, tie)
    r = lib.vts_topk_transform_ragged_ordered(A, 2, 4, 1024, 1040, A, None, A, 256, A, None, A,
                                              1 << 40, None, tie)
    q = lib.vts_topk_transform_page1_ordered(A, 2, 4, 1024, 1040, A, None, A, 32, 32, A, 2, 256,
                                             A, None, A, 1 << 40, None, tie)
    assert v == p == r == q == INVALID


@pytest.mark.parametrize("tie", [1, 2, 1 | 4, 2 | 4])
def test_ordered_entry_points_accept_tie_breaks(lib, tie):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; fake pointers must not reach a launch")
    # every host check passes; the call then stops at the device query
    v = lib.vts_topk_varlen_ordered(A, 0, 8, 4096, 4096, A, 512, 1, 1, None, A, None, A, 1 << 40,
                                    None, tie)
    p = lib.vts_topk_page_table_transform_ordered(A, 2, 4, 1024, 1040, A, None, A, 32, 32, None,
                                                  64, 256, A, None, A, 1 << 40, None, tie)
    assert v == p == HIP


def test_noalloc_rejects_a_shape_beyond_its_scratch_on_the_host(lib):
    # 2048 rows of 262144 columns: more row units than the fixed scratch holds;
    # the check runs on the host before any device call (so also without a GPU)
    st = lib.vts_topk_varlen_noalloc(A, 0, 2048, 262144, 262144, A, 2048, 1, 1, None, A, None,
                                     None)
    assert st == -5
    assert b"scratch" in lib.vts_status_string(st)


def test_wide_top_k_limits_and_workspace(lib):
    # top_k above 2048 takes a larger workspace (candidate slots per unit
    # scale with top_k); the deterministic mode stops at 2048
    small = lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0)
    wide = lib.vts_topk_varlen_workspace_bytes(64, 163840, 16384, 0)
    assert wide > small
    assert lib.vts_topk_varlen_workspace_bytes(64, 163840, 4097, 0) == \
        lib.vts_topk_varlen_workspace_bytes(64, 163840, 8192, 0)
    assert lib.vts_page_transform_workspace_bytes(8, 4096, 16384, 2) > \
        lib.vts_page_transform_workspace_bytes(8, 4096, 512, 2)
    assert lib.vts_topk_varlen_ordered(A, 0, 8, 4096, 4096, A, 2049, 1, 1, None, A, None, A,
                                       1 << 40, None, 1) == UNSUPPORTED
    assert lib.vts_topk_page_table_transform_ordered(A, 2, 4, 1024, 1040, A, None, A, 32, 32, None,
                                                     64, 4096, A, None, A, 1 << 40, None,
                                                     2) == UNSUPPORTED
    # the workspace must match the wide size
    narrow8 = lib.vts_topk_varlen_workspace_bytes(8, 4096, 512, 0)
    assert _varlen(lib, top_k=8192, ws_bytes=narrow8) == WORKSPACE


def test_tuning_switches_belong_to_the_calling_thread(lib):
    import threading
    base = lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0)
    seen = {}

    def other():
        assert lib.vts_set_tuning(vts.TUNE_NSPLIT, 1) == OK
        seen["other"] = lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0)

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["other"] < base  # the switch took effect in its own thread ...
    assert lib.vts_topk_varlen_workspace_bytes(64, 163840, 2048, 0) == base  # ... only there
