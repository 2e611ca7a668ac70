"""GPU parity of the deterministic mode (topk_varlen_ordered) through the C
ABI: canonical order (value descending, then column ascending) with the ties at
the k-th value taken at the smallest or largest columns.  The selection is
unique, so indices and values must equal the oracle's bit for bit, position by
position."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import run_varlen, say, tuning
from workloads.synth import F32

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

NEG_ZERO = {0: 0x80000000, 1: 0x8000, 2: 0x8000}


def _check(wl, tie, tune=None):
    # the ordered kernel ranks -0 below +0 and the oracle treats them as equal:
    # the inputs hold no -0 (and no NaN) in the ranked columns
    _, n = oracle.varlen_rows(wl.seq_lens, wl.rows, wl.next_n, wl.compress_ratio, wl.width)
    for r in range(wl.rows):
        row = wl.x[r, :n[r]]
        assert not np.any(row == NEG_ZERO[wl.dtype]), "input holds -0"
        assert not np.any(np.isnan(oracle._as_float(row, wl.dtype))), "input holds NaN"
    with tuning(**(tune or {})):
        idx, vals, _ = run_varlen(wl, return_values=True, tie=tie)
    ref_idx, ref_vals, _ = oracle.topk_varlen_ordered(
        wl.x[:, :wl.width], wl.dtype, wl.seq_lens, wl.k, tie, next_n=wl.next_n,
        compress_ratio=wl.compress_ratio, return_values=True)
    bad = np.argwhere(idx != ref_idx)
    assert bad.size == 0, f"indices differ at {bad[:4].tolist()}: {idx[tuple(bad[0])]} vs {ref_idx[tuple(bad[0])]}"
    assert np.array_equal(vals, ref_vals), "values differ"


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


FORCED = {
    "careful": dict(force=1),
    "fallback": dict(force=2),
    "spill": dict(lds=64),
    "overflow": dict(lds=64, spill=64),
    "split8": dict(nsplit=8, min_chunk=1024),
    "split8_spill": dict(nsplit=8, min_chunk=1024, lds=64),
    "split3_fallback": dict(nsplit=3, min_chunk=4096, force=2),
}


@pytest.mark.parametrize("tie", ["small", "large"])
@pytest.mark.parametrize("path", sorted(FORCED))
def test_ordered_forced_paths(path, tie):
    wl = workloads.make("dsv4_mtp", rows=16)
    say(f"ordered {tie} forced {path}")
    _check(wl, tie, FORCED[path])


@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_heavy_ties_and_short_rows(tie):
    """fp32 rows of small integers (every value tied hundreds of times), with
    rows shorter than, equal to and longer than top_k, and an empty row."""
    rng = np.random.default_rng(90)
    R, W, k = 12, 9000, 1024
    v = rng.integers(1, 40, size=(R, W)).astype(np.float32)
    wl = workloads.make("small", rows=R, width=W)
    wl.x = v.view(np.uint32)
    wl.k = k
    wl.seq_lens = np.array([0, 1, 5, 1000, 1024, 1025, 3000, 9000, 8999, 2048, 7, 6000], np.int32)
    wl.next_n = 1
    wl.compress_ratio = 1
    wl.dtype = F32
    say(f"ordered {tie} heavy ties")
    _check(wl, tie)
