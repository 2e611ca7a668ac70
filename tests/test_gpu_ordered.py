"""GPU parity of the deterministic mode through the C ABI: the ties at the
k-th value taken at the smallest or largest columns, values compared as
numbers (-0 == +0, NaNs of one sign equal), canonical order (value
descending, then column ascending).  The selection is unique, so indices and
values must equal the oracle's bit for bit, position by position; with
sort=False the same set in any order.  Covers topk_varlen_ordered and the
three windowed transforms in their ordered forms."""
import numpy as np
import pytest
import torch

import oracle
import varlen_top_select_amd as vts
import workloads
from tests.gpu_util import TORCH_DTYPE, run_transform, run_varlen, say, to_device_scores, tuning
from tests.test_gpu_parity import nan_rows
from workloads.synth import BF16, F16, F32, Workload, to_bf16_bits, to_f16_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)


def _same_sets(idx, ref, k):
    for r in range(idx.shape[0]):
        assert sorted(idx[r].tolist()) == sorted(ref[r].tolist()), f"row {r}: selected set differs"


def _check(wl, tie, tune=None, sort=True):
    with tuning(**(tune or {})):
        idx, vals, _ = run_varlen(wl, return_values=True, tie=tie, sort=sort)
    ref_idx, ref_vals, n = oracle.topk_varlen_ordered(
        wl.x[:, :wl.width], wl.dtype, wl.seq_lens, wl.k, tie, next_n=wl.next_n,
        compress_ratio=wl.compress_ratio, return_values=True)
    if sort:
        bad = np.argwhere(idx != ref_idx)
        assert bad.size == 0, (f"indices differ at {bad[:4].tolist()}: "
                               f"{idx[tuple(bad[0])]} vs {ref_idx[tuple(bad[0])]}")
        assert np.array_equal(vals, ref_vals), "values differ"
        return
    # unsorted: the same set, values the selected elements' bits, the
    # identity for rows with n <= k
    _same_sets(idx, ref_idx, wl.k)
    for r in range(wl.rows):
        m = min(int(n[r]), wl.k)
        if n[r] <= wl.k:
            assert idx[r, :m].tolist() == list(range(m)), f"row {r}: short row not the identity"
        assert np.array_equal(vals[r, :m], wl.x[r, idx[r, :m]]), f"row {r}: values"
        assert np.array_equal(vals[r, m:], ref_vals[r, m:]), f"row {r}: padding"


CASES = [("small", {}), ("dsv32", dict(rows=8)), ("dsv4_mtp", dict(rows=32)),
         ("long", dict(rows=8, width=65536)), ("small", dict(variant="relu")),
         ("dsv4_mtp", dict(rows=16, variant="relu"))]


@pytest.mark.parametrize("tie", ["small", "large"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_ordered_workloads(case, tie):
    name, kw = CASES[case]
    wl = workloads.make(name, **kw)
    say(f"ordered {tie} {name} {kw}")
    _check(wl, tie)


# the full workloads in the launch configuration of the benchmark (the long
# batch with the length-balanced placement, the DSv3.2 rows split in four)
@pytest.mark.parametrize("tie", ["small", "large"])
@pytest.mark.parametrize("name", ["long", "dsv4_mtp", "dsv32"])
def test_ordered_full_size(name, tie):
    wl = workloads.make(name)
    say(f"ordered {tie} {name} full {wl.x.shape}")
    _check(wl, tie)


FORCED = {
    "careful": dict(force=1),
    "fallback": dict(force=2),
    "spill": dict(lds=64),
    "overflow": dict(lds=64, spill=64),
    "split8": dict(nsplit=8, min_chunk=1024),
    "split8_spill": dict(nsplit=8, min_chunk=1024, lds=64),
    "split3_fallback": dict(nsplit=3, min_chunk=4096, force=2),
    "split8_careful": dict(nsplit=8, min_chunk=1024, force=1),
}


@pytest.mark.parametrize("tie", ["small", "large"])
@pytest.mark.parametrize("path", sorted(FORCED))
def test_ordered_forced_paths(path, tie):
    wl = workloads.make("dsv4_mtp", rows=16)
    say(f"ordered {tie} forced {path}")
    _check(wl, tie, FORCED[path])


def _custom(bits, n_list, k, dtype):
    R, W = bits.shape
    return Workload(name="custom", kind="varlen", dtype=dtype, x=bits, width=W, k=k,
                    seq_lens=np.asarray(n_list, np.int32), next_n=1, compress_ratio=1,
                    pre_idx=None, return_values=True)


def _bits(vals, dtype):
    if dtype == F32:
        return vals.astype(np.float32).view(np.uint32).copy()
    return to_bf16_bits(vals) if dtype == BF16 else to_f16_bits(vals)


N_TIES = [0, 1, 5, 1000, 1024, 1025, 3000, 9000, 8999, 2048, 7, 6000]


@pytest.mark.parametrize("path", ["normal", "fallback", "split3", "overflow"])
@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_heavy_ties_and_short_rows(tie, path):
    """fp32 rows of small integers (every value tied hundreds of times), with
    rows shorter than, equal to and longer than top_k, and an empty row; the
    whole-row fallback compacts the candidates many times over ties."""
    rng = np.random.default_rng(90)
    R, W, k = len(N_TIES), 9000, 1024
    bits = _bits(rng.integers(1, 40, size=(R, W)).astype(np.float32), F32)
    tune = {"normal": {}, "fallback": dict(force=2), "overflow": dict(lds=64, spill=64),
            "split3": dict(nsplit=3, min_chunk=2048)}[path]
    say(f"ordered {tie} heavy ties {path}")
    _check(_custom(bits, N_TIES, k, F32), tie, tune)


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_signed_zeros(tie, dtype):
    """-0 and +0 tie: rows made mostly of zeros of both signs, so the k-th
    value is zero and the tie-break picks columns among zeros of either sign;
    the returned values keep each zero's sign."""
    rng = np.random.default_rng(70 + dtype)
    R, W, k = len(N_TIES), 9000, 1024
    vals = rng.choice(np.array([0.0, -0.0, 0.0, -0.0, 1.0, -1.0, 0.5], np.float32), size=(R, W))
    say(f"ordered {tie} signed zeros dtype={dtype}")
    _check(_custom(_bits(vals, dtype), N_TIES, k, dtype), tie)
    with_fallback = _custom(_bits(vals, dtype), N_TIES, k, dtype)
    say(f"ordered {tie} signed zeros dtype={dtype}, whole-row fallback")
    _check(with_fallback, tie, dict(force=2))


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_nan_rows(tie, dtype):
    """NaNs of one sign are equal: the tie-break orders them by column."""
    rng = np.random.default_rng(80 + dtype)
    W, k = 9000, 256
    bits = nan_rows(dtype, W, k, rng)
    say(f"ordered {tie} NaN rows dtype={dtype}")
    _check(_custom(bits, [W, W, 5000, W, W], k, dtype), tie)


@pytest.mark.parametrize("path", ["direct", "stream", "split4"])
@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_constant_rows(tie, dtype, path):
    """Every candidate equal (the select's key range is a single key): rows
    short enough to be selected directly, streamed rows and split rows."""
    W, k = {"direct": (3000, 1000), "stream": (50000, 2048), "split4": (50000, 512)}[path]
    n_list = [W, W - 1, k + 1, W // 2]
    bits = _bits(np.full((len(n_list), W), 0.75, np.float32), dtype)
    tune = dict(nsplit=4, min_chunk=1024) if path == "split4" else {}
    say(f"ordered {tie} constant rows dtype={dtype} {path}")
    _check(_custom(bits, n_list, k, dtype), tie, tune)


@pytest.mark.parametrize("tie", ["small", "large"])
@pytest.mark.parametrize("name", ["dsv4_mtp", "long"])
def test_ordered_unsorted(name, tie):
    wl = workloads.make(name, rows=16, width=65536 if name == "long" else None)
    say(f"ordered {tie} unsorted {name}")
    _check(wl, tie, sort=False)


def test_ordered_unsorted_heavy_ties():
    rng = np.random.default_rng(91)
    bits = _bits(rng.integers(1, 40, size=(len(N_TIES), 9000)).astype(np.float32), F32)
    for tie in ("small", "large"):
        say(f"ordered {tie} unsorted heavy ties")
        _check(_custom(bits, N_TIES, 1024, F32), tie, sort=False)


def test_ordered_bit_identical_across_runs():
    wl = workloads.make("dsv4_mtp", rows=64, variant="relu")
    say("ordered repeat runs")
    outs = [run_varlen(wl, return_values=True, tie="large")[:2] for _ in range(3)]
    for i, v in outs[1:]:
        assert np.array_equal(i, outs[0][0]) and np.array_equal(v, outs[0][1])


# ---------------------------------------------------------------------------
# the windowed transforms in the deterministic mode
# ---------------------------------------------------------------------------

def _check_page(wl, tie, sort=True, with_raw=True, tune=None):
    with tuning(**(tune or {})):
        out, raw, _ = run_transform(wl, with_raw=with_raw, tie=tie, sort=sort)
    ref_out, ref_raw, base, n = oracle.topk_page_table_transform_ordered(
        wl.x[:, :wl.width], wl.dtype, wl.lengths, wl.row_starts, wl.page_table,
        wl.page_table_row_starts, wl.page_size, wl.k, tie)
    if sort:
        assert np.array_equal(out, ref_out), "out differs from the oracle's"
        if with_raw:
            assert np.array_equal(raw, ref_raw), "out_raw differs from the oracle's"
        return
    _same_sets(out, ref_out, wl.k)
    if with_raw:
        _same_sets(raw, ref_raw, wl.k)
        want = oracle.page_translate(raw, wl.page_table, wl.page_table_row_starts, base,
                                     wl.page_size)
        assert np.array_equal(out, want), "out is not the translation of out_raw"


@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_page_full(tie):
    wl = workloads.make("page")
    say(f"ordered {tie} page transform full")
    _check_page(wl, tie)


@pytest.mark.parametrize("variant", ["relu", "no_raw", "unsorted", "split4", "fallback"])
def test_ordered_page_variants(variant):
    wl = workloads.make("page", rows=24, variant="relu" if variant == "relu" else None)
    tune = {"split4": dict(nsplit=4, min_chunk=1024), "fallback": dict(force=2)}.get(variant)
    for tie in ("small", "large"):
        say(f"ordered {tie} page transform {variant}")
        _check_page(wl, tie, sort=variant != "unsorted", with_raw=variant != "no_raw", tune=tune)


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_ragged(tie, dtype):
    rng = np.random.default_rng(60 + dtype)
    R, W, k = 24, 40000, 1024
    vals = rng.integers(-20, 20, size=(R, W)).astype(np.float32)  # ties at the boundary
    bits = _bits(vals, dtype)
    lengths = rng.integers(0, W, size=R).astype(np.int32)
    lengths[:3] = [0, 5, k]
    starts = np.array([rng.integers(0, W - L + 1) for L in lengths], np.int32)
    offsets = rng.integers(0, 1 << 30, size=R).astype(np.int32)
    x = to_device_scores(bits, dtype, W)
    say(f"ordered {tie} ragged dtype={dtype}")
    out, raw = vts.topk_transform_ragged(
        x, torch.from_numpy(lengths).cuda(), torch.from_numpy(offsets).cuda(), k,
        row_starts=torch.from_numpy(starts).cuda(), return_raw=True, tie_break=tie)
    torch.cuda.synchronize()
    ref_out, ref_raw, _, _ = oracle.topk_transform_ragged_ordered(bits, dtype, lengths, starts,
                                                                  offsets, k, tie)
    assert np.array_equal(raw.cpu().numpy(), ref_raw)
    assert np.array_equal(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_page1(tie):
    wl = workloads.make("page", rows=32)
    rng = np.random.default_rng(61)
    R, W, k = wl.rows, wl.width, wl.k
    B = 10
    cu = np.concatenate([[1], 1 + np.cumsum(rng.integers(1, 4, size=B))]).astype(np.int32)
    cu[-1] = min(cu[-1], R - 1)
    cu = np.minimum(cu, R - 1)
    pt = rng.integers(0, 1 << 30, size=(B, W - 100)).astype(np.int32)
    x = to_device_scores(wl.x, wl.dtype, W)
    say(f"ordered {tie} page-size-1 transform")
    out, raw = vts.topk_transform_page1(
        x, torch.from_numpy(wl.lengths).cuda(), torch.from_numpy(pt).cuda(),
        torch.from_numpy(cu).cuda(), k, row_starts=torch.from_numpy(wl.row_starts).cuda(),
        return_raw=True, tie_break=tie)
    torch.cuda.synchronize()
    ref_out, ref_raw, _, _ = oracle.topk_transform_page1_ordered(
        wl.x[:, :W], wl.dtype, wl.lengths, wl.row_starts, pt, cu, k, tie)
    assert np.array_equal(raw.cpu().numpy(), ref_raw)
    assert np.array_equal(out.cpu().numpy(), ref_out)
