"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Every case prints its name before its GPU step.  Outputs are compared with the
tie-aware checker (oracle/check.py): bit-exact up to interchangeable ties.
"""
import os
import subprocess
import sys
import zlib

import numpy as np
import pytest
import torch

import workloads
from workloads.synth import F16, F32, BF16, Workload, poison_outside, to_bf16_bits, to_f16_bits
from tests.gpu_util import (check_transform_wl, check_varlen, run_transform, run_varlen, say,
                            tuning)
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)


def _assert_ok(errs):
    assert errs == [], "\n".join(errs)


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the bench times
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["small", "dsv32", "long", "dsv4_mtp"])
def test_varlen_workload_full(name):
    wl = workloads.make(name)
    say(f"{name} full {wl.x.shape} k={wl.k} hint={wl.pre_idx is not None}")
    idx, vals, stats = run_varlen(wl)
    say(f"{name} stats {stats}")
    _assert_ok(check_varlen(wl, idx, vals))


@pytest.mark.parametrize("name", ["dsv32", "long"])
def test_hint_rung_full(name):
    """The hinted rung (a diagnostic switch; the default path does not read
    the hint) at full size, the long batch with the length-balanced placement."""
    wl = workloads.make(name)
    say(f"{name} full with the hint rung")
    with tuning(hint_rung=1):
        idx, vals, stats = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, vals))


def test_varlen_long_hint_free():
    wl = workloads.make("long", hint=False)
    say("long full, hint-free")
    idx, vals, stats = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, vals))


def test_transform_page_full():
    wl = workloads.make("page")
    say(f"page full {wl.x.shape}")
    out, raw, stats = run_transform(wl)
    _assert_ok(check_transform_wl(wl, out, raw))


# ---------------------------------------------------------------------------
# length-balanced placement of rows (256 * s rows, one workgroup per row):
# every row must be taken exactly once, with the placement on and off
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,rows,width", [("long", 512, 16384), ("long", 1024, 8192),
                                             ("dsv4_mtp", 768, 16384),
                                             ("page", 512, 8192), ("long", 4096, 4096)])
@pytest.mark.parametrize("balance", [True, False])
def test_balanced_placement(name, rows, width, balance):
    wl = workloads.make(name, rows=rows, width=width)
    say(f"{name} rows {rows} width {width} balance {balance}")
    with tuning(nsplit=1, no_balance=0 if balance else 1):
        if wl.kind == "varlen":
            idx, vals, stats = run_varlen(wl)
            errs = check_varlen(wl, idx, vals)
        else:
            out, raw, stats = run_transform(wl)
            errs = check_transform_wl(wl, out, raw)
    _assert_ok(errs)


# ---------------------------------------------------------------------------
# every internal path, forced, on reduced workloads
# ---------------------------------------------------------------------------

PATHS = {
    "normal": {},
    "careful": dict(force=1),
    "fallback": dict(force=2),
    "spill": dict(lds=64),
    "overflow": dict(lds=64, spill=64),
    "split8": dict(nsplit=8, min_chunk=1024),
    "split8_spill": dict(nsplit=8, min_chunk=1024, lds=64),
    "split8_careful": dict(nsplit=8, min_chunk=1024, force=1),
    "split3_fallback": dict(nsplit=3, min_chunk=4096, force=2),
    "split32": dict(nsplit=32, min_chunk=256),
    "tight_sigma": dict(sigma=1),
    "one_rung": dict(likely=55),
    "high_likely_rung": dict(likely=1, sigma=55),
    "split8_high_likely_rung": dict(nsplit=8, min_chunk=1024, likely=1),
    "split8_lo_overflow": dict(nsplit=8, min_chunk=1024, likely=1, spill=64),
}

REDUCED = {"small": dict(rows=4), "dsv32": dict(rows=8), "long": dict(rows=8, width=65536),
           "dsv4_mtp": dict(rows=32), "page": dict(rows=24)}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("name", ["small", "dsv32", "long", "dsv4_mtp", "page"])
def test_forced_paths(name, path):
    wl = workloads.make(name, **REDUCED[name])
    say(f"{name} reduced {wl.x.shape} path {path}")
    with tuning(**PATHS[path]):
        if wl.kind == "varlen":
            idx, vals, stats = run_varlen(wl)
            errs = check_varlen(wl, idx, vals)
        else:
            out, raw, stats = run_transform(wl)
            errs = check_transform_wl(wl, out, raw)
    _assert_ok(errs)
    if path in ("careful", "normal", "spill") or path.startswith("split8"):
        assert stats[1] == 0 or path.endswith("fallback")
    if path == "overflow":
        assert stats[0] > 0, "the overflow path was not exercised"


# ---------------------------------------------------------------------------
# hand-built rows
# ---------------------------------------------------------------------------

def _varlen_wl(values_f32: np.ndarray, seq_lens, k, dtype=F32, next_n=1, cr=1, stride=None,
               return_values=True, pre_idx=None, raw_bits=None) -> Workload:
    R, W = values_f32.shape if raw_bits is None else raw_bits.shape
    S = stride or W
    if raw_bits is None:
        if dtype == F32:
            bits = values_f32.astype(np.float32).view(np.uint32)
        elif dtype == BF16:
            bits = to_bf16_bits(values_f32)
        else:
            bits = to_f16_bits(values_f32)
    else:
        bits = raw_bits
    x = np.zeros((R, S), bits.dtype)
    x[:, :W] = bits
    return Workload(name="custom", kind="varlen", dtype=dtype, x=x, width=W, k=k,
                    seq_lens=np.asarray(seq_lens, np.int32), next_n=next_n, compress_ratio=cr,
                    pre_idx=pre_idx, return_values=return_values)


def _rows_of(n_list, W, rng, law="normal"):
    R = len(n_list)
    if law == "normal":
        return rng.standard_normal((R, W)).astype(np.float32)
    if law == "ints":
        return rng.integers(-3, 4, size=(R, W)).astype(np.float32)
    if law == "relu":
        return np.maximum(rng.standard_normal((R, W)), 0).astype(np.float32)
    if law == "ascending":
        return np.tile(np.arange(W, dtype=np.float32), (R, 1))
    if law == "descending":
        return np.tile(np.arange(W, 0, -1, dtype=np.float32), (R, 1))
    if law == "constant":
        return np.full((R, W), 0.75, np.float32)
    if law == "neginf":
        return np.full((R, W), -np.inf, np.float32)
    if law == "specials":
        choice = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1e-40, 3e38, -3e38, 1.0],
                          np.float32)
        return rng.choice(choice, size=(R, W))
    if law == "spike_cluster":  # the largest values sit in one short run the sample misses
        x = rng.standard_normal((R, W)).astype(np.float32)
        x[:, 100:100 + 3000] += 10.0
        return x
    raise ValueError(law)


N_EDGES = [0, 1, 511, 512, 513, 1024, 4095, 4096, 4097, 5000, 16383, 16384, 16385, 40000, 70000]


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("law", ["normal", "ints", "relu", "ascending", "descending", "constant",
                                 "neginf", "specials", "spike_cluster"])
def test_edge_lengths_and_values(law, dtype):
    rng = np.random.default_rng(zlib.crc32(f"{law}/{dtype}".encode()))
    W, k = 70000, 512
    vals = _rows_of(N_EDGES, W, rng, law)
    if dtype == F16:
        vals = np.clip(vals, -60000, 60000) if law not in ("neginf", "specials") else vals
    wl = _varlen_wl(vals, N_EDGES, k, dtype=dtype)
    say(f"edge lengths law={law} dtype={dtype}")
    idx, v, stats = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("k", [1, 7, 2048])
def test_k_extremes(k):
    rng = np.random.default_rng(k)
    n_list = [0, 1, k, k + 1, 2 * k + 3, 9000, 65536]
    W = 65536
    vals = _rows_of(n_list, W, rng, "ints")
    wl = _varlen_wl(vals, n_list, k)
    say(f"k={k}")
    idx, v, _ = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("offset", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("dtype", [F32, BF16])
def test_misaligned_base_and_odd_stride(dtype, offset):
    rng = np.random.default_rng(offset)
    n_list = [3, 600, 4099, 20001, 33333, 50001]
    W, S = 50001, 50013
    vals = _rows_of(n_list, W, rng, "normal")
    wl = _varlen_wl(vals, n_list, 512, dtype=dtype, stride=S)
    say(f"misaligned offset={offset} dtype={dtype}")
    with tuning(nsplit=4, min_chunk=4096):
        idx, v, _ = run_varlen(wl, offset=offset)
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("next_n,cr", [(1, 1), (2, 1), (3, 1), (4, 1), (1, 4), (2, 4), (3, 4),
                                       (4, 4)])
def test_mtp_grouping_and_compression(next_n, cr):
    rng = np.random.default_rng(next_n * 10 + cr)
    W, k = 20000, 1024
    reqs = 12
    seq = np.array([0, 1, next_n - 1, next_n, 2, 4100, 4 * k + 7, cr * W, cr * W + 999, -5,
                    2**31 - 1, -2**31], np.int64)
    seq = np.clip(seq, -2**31, 2**31 - 1).astype(np.int32)
    vals = rng.standard_normal((reqs * next_n, W)).astype(np.float32)
    wl = _varlen_wl(vals, seq, k, next_n=next_n, cr=cr)
    say(f"next_n={next_n} cr={cr}")
    idx, v, _ = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


def test_poisoned_columns_are_never_selected():
    wl = workloads.make("dsv32", rows=8)
    base, n = oracle.varlen_rows(wl.seq_lens, wl.rows, wl.next_n, wl.compress_ratio, wl.width)
    poison_outside(wl, base, n)
    say("poisoned columns")
    idx, v, _ = run_varlen(wl, return_values=True)
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("rung", [0, 1])
def test_degenerate_hints(rung):
    wl = workloads.make("dsv32", rows=8)
    R, k = wl.rows, wl.k
    for name, h in {
        "zeros": np.zeros((R, k), np.int32),
        "same": np.full((R, k), 7, np.int32),
        "max": np.full((R, k), 2**31 - 1, np.int32),
        "neg": np.full((R, k), -1, np.int32),
        "dup_half": np.concatenate([wl.pre_idx[:, : k // 2]] * 2, axis=1),
        "random": np.random.default_rng(0).integers(-10, 2 * wl.width, size=(R, k)).astype(np.int32),
    }.items():
        wl.pre_idx = h
        say(f"hint {name} hint rung {rung}")
        with tuning(hint_rung=rung):
            idx, v, _ = run_varlen(wl)
        _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_hint_rung_on_cluster_rows(dtype):
    """The top values sit in one run of 3000 columns; the hint is the previous
    step's top k (here: the current one shifted left by a column, as if the
    row had grown by one), so the hint rung is about the k-th largest value.
    Hinted and hint-free runs are both exact, and the hinted one never needs
    the whole-row re-selection (its rung is a lower bound of the k-th
    largest by construction)."""
    rng = np.random.default_rng(77 + dtype)
    n_list = [70000, 65536, 40000, 20000]
    W, k = 70000, 2048
    vals = _rows_of(n_list, W, rng, "spike_cluster")
    ref, _, _ = oracle.topk_varlen(vals, F32, np.array(n_list, np.int32), k)
    hint = np.where(ref > 0, ref - 1, ref).astype(np.int32)
    wl = _varlen_wl(vals, n_list, k, dtype=dtype, pre_idx=hint)
    say(f"cluster rows with hint dtype={dtype}")
    with tuning(hint_rung=1):
        idx, v, st_hint = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))
    say(f"cluster rows without hint dtype={dtype}")
    idx, v, st_free = run_varlen(wl, use_hint=False)
    _assert_ok(check_varlen(wl, idx, v))
    say(f"stats with hint {st_hint}, without {st_free}")
    assert st_hint[1] == 0


# NaN patterns per dtype: sign clear (quiet, payload, signalling), sign set
NAN_BITS = {F32: [0x7FC00000, 0x7FC00001, 0x7F800001, 0xFFC00000, 0xFFC00001],
            BF16: [0x7FC0, 0x7FC1, 0x7F81, 0xFFC0, 0xFFC1],
            F16: [0x7E00, 0x7E01, 0x7C01, 0xFE00, 0xFE01]}


def nan_rows(dtype, W, k, rng):
    """Rows with NaNs of both signs: sparse, everywhere, a single one, and as
    many sign-clear NaNs as straddle the k-th place."""
    vals = rng.standard_normal((5, W)).astype(np.float32)
    bits = vals.view(np.uint32) if dtype == F32 else (to_bf16_bits(vals) if dtype == BF16
                                                       else to_f16_bits(vals))
    bits = bits.copy()
    pat = np.array(NAN_BITS[dtype], bits.dtype)
    bits[0, ::7] = rng.choice(pat, size=bits[0, ::7].shape)
    bits[1, :] = rng.choice(pat, size=W)
    bits[2, 100] = pat[3]
    cols = rng.choice(W, size=k + 40, replace=False)
    bits[3, cols] = rng.choice(pat[:3], size=cols.size)  # more sign-clear NaNs than k
    cols = rng.choice(W, size=3 * k, replace=False)
    bits[4, cols] = pat[3]  # sign-set NaNs: below everything
    return bits


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_nan_rows(dtype):
    """NaN rows under the order the oracle documents: the count of NaNs of
    each sign selected and the multiset of the other values must match."""
    rng = np.random.default_rng(5 + dtype)
    W, k = 9000, 256
    bits = nan_rows(dtype, W, k, rng)
    wl = _varlen_wl(None, [W, W, 5000, W, W], k, dtype=dtype, raw_bits=bits)
    say(f"NaN rows dtype={dtype}")
    idx, v, _ = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


def test_repeat_calls_reuse_the_workspace():
    wl = workloads.make("dsv32", rows=16)
    x = torch.from_numpy(wl.x.view(np.float32)).cuda()
    seq = torch.from_numpy(wl.seq_lens).cuda()
    import varlen_top_select_amd as vts
    ws = vts.make_workspace(wl.rows, wl.width, wl.k, torch.float32, "cuda")
    say("repeat calls on one workspace")
    outs = []
    for _ in range(5):
        idx, _ = vts.topk_varlen(x, seq, wl.k, workspace=ws)
        outs.append(idx.cpu().numpy())
    for o in outs:
        _assert_ok(check_varlen(wl, o, None))


# ---------------------------------------------------------------------------
# page transform variants
# ---------------------------------------------------------------------------

def test_transform_identity_page_size_1_no_starts():
    wl = workloads.make("page", rows=16)
    W = wl.width
    wl.page_size = 1
    wl.page_table = np.tile(np.arange(W + 8, dtype=np.int32), (wl.rows, 1))
    wl.page_table_row_starts = None
    wl.row_starts = np.zeros(wl.rows, np.int32)
    say("transform page_size 1, identity table, no starts")
    out, raw, _ = run_transform(wl, ptrs=False, starts=False)
    _assert_ok(check_transform_wl(wl, out, raw, ptrs=False, starts=False))
    base, n = oracle.window_rows(wl.lengths, None, W)
    assert np.array_equal(out, raw)


@pytest.mark.parametrize("page_size", [1, 16, 32, 48, 64])
def test_transform_page_sizes_and_table_edges(page_size):
    """Page sizes on both sides of the output translation's LDS staging (a
    power-of-two page size and at most 2560 pages per window; 32 stages 2048
    pages, the first 1024 read ahead of the count and the rest after it; 16
    has 4096 pages and 48 is no power of two, both read the table per entry),
    page-table row starts below zero and tables narrower than the windows, so
    that some pages fall outside the table at either end."""
    wl = workloads.make("page", rows=24)
    W = wl.width
    g = np.random.default_rng(500 + page_size)
    wl.page_size = page_size
    pages = -(-W // page_size)
    cols = 3000 if page_size == 1 else pages - pages // 8
    wl.page_table = g.integers(0, 1 << 20, size=(wl.rows, cols), dtype=np.int32)
    wl.page_table_row_starts = g.integers(-40, 40, size=wl.rows).astype(np.int32)
    lengths = np.array([W, W, 60000, 40000, 2048, 2049, 2500, 2600, 3000, 100, 64 * 2560,
                        64 * 1024 + 5, 0, 1, 70000, 33333, 20000, 10000, 5000, 4097, 4096, 2047,
                        65, 64], np.int64)
    wl.lengths[:] = np.minimum(lengths, W).astype(np.int32)
    wl.row_starts[:] = np.array([0 if wl.lengths[i] >= W else int(g.integers(0, W - wl.lengths[i] + 1))
                                 for i in range(wl.rows)], np.int32)
    say(f"transform page_size {page_size}, table of {cols} columns")
    out, raw, _ = run_transform(wl)
    _assert_ok(check_transform_wl(wl, out, raw))


def test_transform_without_raw_output():
    wl = workloads.make("page", rows=8)
    say("transform without out_raw")
    out, raw, _ = run_transform(wl, with_raw=False)
    _assert_ok(check_transform_wl(wl, out, None))


def test_transform_odd_windows():
    wl = workloads.make("page", rows=16)
    W = wl.width
    wl.lengths[:] = np.array([0, -5, 1, 2047, 2048, 2049, W, W, 5, 3000, 70000, 40000, 7, 9,
                              100, 4096], np.int32)
    wl.row_starts[:] = np.array([0, 0, W, W - 1, 3, 1, 0, 17, -1, W + 1, 5, 12345, 2, 1, 77,
                                 999], np.int32)
    wl.page_table = wl.page_table[:, :300]  # narrow table: some entries fall outside it
    wl.x[:, :] = to_f16_bits(np.random.default_rng(9).standard_normal(wl.x.shape).astype(np.float32))
    say("transform odd windows")
    out, raw, _ = run_transform(wl)
    _assert_ok(check_transform_wl(wl, out, raw))


def test_plan_log():
    """VTS_LOG=1: each call prints the plan it launches, one line on stderr."""
    code = ("import torch, varlen_top_select_amd as vts\n"
            "x = torch.randn(4, 4096, device='cuda')\n"
            "s = torch.tensor([4096, 100, 3000, 1], dtype=torch.int32, device='cuda')\n"
            "vts.topk_varlen(x, s, 512)\n"
            "vts.topk_varlen_ordered(x, s, 512)\n"
            "torch.cuda.synchronize()\n")
    say("plan log in a child process")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, VTS_LOG="1"), cwd=root,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[vts]")]
    assert len(lines) == 2, r.stderr[-2000:]
    assert "vts_topk_varlen: rows 4 width 4096 top_k 512 f32 | kernels any-order" in lines[0]
    assert "vts_topk_varlen_ordered:" in lines[1] and "kernels ordered" in lines[1]
