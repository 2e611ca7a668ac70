"""GPU parity for top_k above 2048 (up to 16384, the range of FlashInfer's
radix_filter backend, flashinfer.top_k_varlen, `backend`), through the C ABI:
the wide kernels keep their candidate lists in LDS and the workspace.  Same
tie-aware checks against the oracle as the other parity tests."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import check_transform_wl, check_varlen, run_transform, run_varlen, say, tuning
from tests.test_gpu_parity import _rows_of, _varlen_wl, nan_rows
from workloads.synth import BF16, F16, F32

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

KS = [2049, 4096, 8192, 16384]


def _assert_ok(errs):
    assert errs == [], "\n".join(errs)


def _n_list(k, W):
    return [n for n in (0, 1, k - 1, k, k + 1, 2 * k + 3, 3776, 3777, 8192, 20000, 40000, 65536,
                        100000, W) if n <= W]


@pytest.mark.parametrize("k", KS)
@pytest.mark.parametrize("law", ["normal", "ints", "relu", "constant", "specials", "spike_cluster"])
def test_wide_edge_lengths_and_values(law, k):
    rng = np.random.default_rng(zlib.crc32(f"wide/{law}/{k}".encode()))
    W = 100000
    n_list = _n_list(k, W)
    vals = _rows_of(n_list, W, rng, law)
    wl = _varlen_wl(vals, n_list, k)
    say(f"wide k={k} law={law}")
    idx, v, stats = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("dtype", [BF16, F16])
@pytest.mark.parametrize("k", [4096, 16384])
def test_wide_16bit(dtype, k):
    rng = np.random.default_rng(k + dtype)
    W = 262144
    n_list = [k + 1, 30000, 131072, W]
    vals = np.clip(_rows_of(n_list, W, rng, "normal"), -60000, 60000)
    wl = _varlen_wl(vals, n_list, k, dtype=dtype)
    say(f"wide k={k} dtype={dtype}")
    idx, v, _ = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


PATHS = {
    "normal": {},                     # the default plan splits these rows in four
    "single": dict(nsplit=1),
    "fallback": dict(force=2),        # exact radix passes over the row
    "careful": dict(nsplit=1, force=1),  # forced: the same exact fallback
    "spill": dict(nsplit=1, lds=64),  # almost every candidate in the workspace
    "overflow": dict(nsplit=1, spill=4096),  # lists outgrow their slots: exact fallback
    "tight_sigma": dict(nsplit=1, sigma=1),  # too few candidates, sometimes: exact fallback
    "split4_spill": dict(nsplit=4, min_chunk=4096, lds=64),
    "split4_overflow": dict(nsplit=4, min_chunk=4096, lds=256, spill=512),
    "split4_fallback": dict(nsplit=4, min_chunk=4096, force=2),
    "one_rung": dict(likely=55),
}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("k", [4096, 16384])
def test_wide_forced_paths(path, k):
    wl = workloads.make("long", rows=8, width=131072)
    wl.k = k
    wl.pre_idx = None
    say(f"wide k={k} path {path}")
    with tuning(**PATHS[path]):
        idx, v, stats = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))
    if path.endswith("overflow"):
        assert stats[0] > 0, "the overflow path was not exercised"


@pytest.mark.parametrize("k", [4096, 16384])
def test_wide_dsv4_mtp_shape(k):
    wl = workloads.make("dsv4_mtp", rows=128)
    wl.k = k
    say(f"wide dsv4_mtp k={k}")
    idx, v, _ = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


def test_wide_full_long_batch():
    wl = workloads.make("long")
    wl.k = 16384
    wl.pre_idx = None
    say("wide long batch full size, k=16384")
    idx, v, stats = run_varlen(wl)
    say(f"wide long stats {stats}")
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_wide_nan_rows(dtype):
    rng = np.random.default_rng(40 + dtype)
    W, k = 40000, 4096
    bits = nan_rows(dtype, W, k, rng)
    wl = _varlen_wl(None, [W, W, 30000, W, W], k, dtype=dtype, raw_bits=bits)
    say(f"wide NaN rows dtype={dtype}")
    idx, v, _ = run_varlen(wl)
    _assert_ok(check_varlen(wl, idx, v))


@pytest.mark.parametrize("k", [4096, 16384])
@pytest.mark.parametrize("variant", ["full", "split4", "no_raw"])
def test_wide_page_transform(k, variant):
    wl = workloads.make("page", rows=64 if variant != "full" else None)
    wl.k = k
    say(f"wide page transform k={k} {variant}")
    tune = dict(nsplit=4, min_chunk=4096) if variant == "split4" else {}
    with tuning(**tune):
        out, raw, _ = run_transform(wl, with_raw=variant != "no_raw")
    _assert_ok(check_transform_wl(wl, out, raw if variant != "no_raw" else None))
