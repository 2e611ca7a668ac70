"""GPU parity of the length-balanced units of 512-row batches: the launch has
1024 workgroups, and every row is cut into e = min(8, ceil(n / U)) units,
where U is about the batch's columns per compute unit and at least 128 KB.

Three length profiles: "few" -- a handful of long rows (e up to 8) among
short ones, with lengths one element around a unit bound; "many" -- 200 long
rows, so that U is large and they split in two; "spread" -- log-uniform
lengths, every unit count from 1 to the maximum.  Every case prints its name
before its GPU step.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads.synth import F16, F32, BF16, Workload, to_bf16_bits, to_f16_bits
from tests.gpu_util import (check_transform_wl, check_varlen, run_transform, run_varlen, say,
                            tuning)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

R = 512
W = 196608  # 768 KB of fp32, 384 KB of 16-bit columns


def _split_cols(dtype):
    return (128 * 1024) // (4 if dtype == F32 else 2)


def _lengths(profile, dtype, rng):
    n = rng.integers(100, 3001, size=R).astype(np.int64)
    s = _split_cols(dtype)
    if profile == "few":
        special = [W, s, s - 1, s + 1, 2 * s, 2 * s + 1, 3 * s - 1, (s + W) // 2, W - 7]
        at = rng.choice(R, size=len(special), replace=False)
        n[at] = special
    elif profile == "many":
        at = rng.choice(R, size=200, replace=False)
        n[at] = W - rng.integers(0, 64, size=200)
    else:
        n = np.exp(rng.uniform(np.log(100), np.log(W), size=R)).astype(np.int64)
    return n


def _bits(rng, dtype):
    v = rng.standard_normal((R, W), dtype=np.float32)
    if dtype == F32:
        return v.view(np.uint32)
    return to_bf16_bits(v) if dtype == BF16 else to_f16_bits(v)


def _varlen(profile, dtype, k, seed):
    rng = np.random.default_rng(seed)
    n = _lengths(profile, dtype, rng)
    return Workload(name=f"helpers-{profile}", kind="varlen", dtype=dtype, x=_bits(rng, dtype),
                    width=W, k=k, seq_lens=n.astype(np.int32), next_n=1, compress_ratio=1,
                    pre_idx=None, return_values=True)


def _expected_units(wl):
    """(split rows, most units of a row, units in all) under the placement's
    rule: U = max(128 KB, min(width, 4 * sum(n >> 10) + 4 * R)) columns."""
    n = np.minimum(wl.seq_lens.astype(np.int64), W)
    U = max(_split_cols(wl.dtype), min(W, 4 * int((n >> 10).sum()) + 4 * R))
    e = np.clip(-(-n // U), 1, 8)
    return int((e > 1).sum()), int(e.max()), int(e.sum())


PROFILES = ["few", "many", "spread"]


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("profile", PROFILES)
def test_helpers_varlen(profile, dtype):
    wl = _varlen(profile, dtype, 2048, 700 + dtype + 10 * PROFILES.index(profile))
    split, most, units = _expected_units(wl)
    say(f"units varlen {profile} dtype {dtype}: {split} rows split, up to {most} units, {units} in all")
    assert split > 0 and units <= 2 * R
    idx, vals, _ = run_varlen(wl)
    errs = check_varlen(wl, idx, vals)
    assert errs == [], "\n".join(errs[:8])
    say("the same without the balanced placement (one unit per row)")
    with tuning(no_balance=1):
        idx2, vals2, _ = run_varlen(wl)
    errs = check_varlen(wl, idx2, vals2)
    assert errs == [], "\n".join(errs[:8])


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("profile", PROFILES)
def test_helpers_ordered(profile, dtype):
    wl = _varlen(profile, dtype, 1024, 800 + dtype + 10 * PROFILES.index(profile))
    say(f"units ordered (SMALL) {profile} dtype {dtype}")
    idx, vals, _ = run_varlen(wl, tie="small")
    ref_idx, ref_vals, _ = oracle.topk_varlen_ordered(wl.x[:, :W], wl.dtype, wl.seq_lens, wl.k,
                                                      "small", return_values=True)
    bad = np.argwhere(idx != ref_idx)
    assert bad.size == 0, f"indices differ at {bad[:4].tolist()}"
    assert np.array_equal(vals, ref_vals), "values differ"


def test_helpers_wide():
    wl = _varlen("few", BF16, 4096, 901)
    say("units varlen top_k 4096 (wide kernels), bf16")
    idx, vals, _ = run_varlen(wl)
    errs = check_varlen(wl, idx, vals)
    assert errs == [], "\n".join(errs[:8])


def test_helpers_page_transform():
    rng = np.random.default_rng(902)
    dtype = F16
    n = _lengths("few", dtype, rng)
    starts = np.array([rng.integers(0, W - m + 1) for m in n], np.int64)
    P = W // 64 + 16
    wl = Workload(name="helpers-page", kind="transform", dtype=dtype, x=_bits(rng, dtype),
                  width=W, k=2048)
    wl.lengths = n.astype(np.int32)
    wl.row_starts = starts.astype(np.int32)
    wl.page_size = 64
    wl.page_table = rng.permutation(R * P).astype(np.int32).reshape(R, P)
    wl.page_table_row_starts = rng.integers(0, 16, size=R).astype(np.int32)
    say("units page transform, fp16, page 64")
    out, raw, _ = run_transform(wl)
    errs = check_transform_wl(wl, out, raw)
    assert errs == [], "\n".join(errs[:8])


@pytest.mark.parametrize("seed", [904, 905, 906])
def test_helpers_spread_seeds(seed):
    """More log-uniform length draws (fp32 and bf16 alternately): every unit
    count from 1 to the maximum, at other positions."""
    dtype = F32 if seed % 2 == 0 else BF16
    wl = _varlen("spread", dtype, 2048, seed)
    split, most, units = _expected_units(wl)
    say(f"units varlen spread seed {seed} dtype {dtype}: {split} rows split, up to {most} units")
    idx, vals, _ = run_varlen(wl)
    errs = check_varlen(wl, idx, vals)
    assert errs == [], "\n".join(errs[:8])


def test_helpers_unit_cap():
    """Rows longer than 8 U: the unit count stops at 8 and each unit is longer
    than U (fp32, four rows of 300000 columns among short rows)."""
    Wc = 300000
    rng = np.random.default_rng(903)
    n = rng.integers(100, 3001, size=R).astype(np.int64)
    at = rng.choice(R, size=4, replace=False)
    n[at] = Wc - rng.integers(0, 8, size=4)
    x = rng.standard_normal((R, Wc), dtype=np.float32).view(np.uint32)
    wl = Workload(name="helpers-cap", kind="varlen", dtype=F32, x=x, width=Wc, k=2048,
                  seq_lens=n.astype(np.int32), next_n=1, compress_ratio=1, pre_idx=None,
                  return_values=True)
    U = max(_split_cols(F32), min(Wc, 4 * int((np.minimum(n, Wc) >> 10).sum()) + 4 * R))
    assert -(-int(n.max()) // U) > 8, "the long rows need more than eight units"
    say(f"units varlen capped at 8 units: 4 rows of ~{Wc} fp32 columns, U = {U}")
    idx, vals, _ = run_varlen(wl)
    errs = check_varlen(wl, idx, vals)
    assert errs == [], "\n".join(errs[:8])
