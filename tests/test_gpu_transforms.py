"""GPU parity of SGLang's two index transforms (TopK_Ops page): the ragged-KV
offset (fast_topk_transform_ragged_fused) and the page-size-1 per-request page
table (fast_topk_transform_fused), through the C ABI.  The selection is
checked against the CPU oracle with the tie-aware checker, and `out` must equal
the oracle's translation of the GPU's own raw indices position by position."""
import numpy as np
import pytest
import torch

import oracle
import varlen_top_select_amd as vts
import workloads
from oracle.check import check_rows
from tests.gpu_util import TORCH_DTYPE, say, to_device_scores, tuning
from workloads.synth import F16, F32, BF16, to_bf16_bits, to_f16_bits

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)


def _run(x_bits, dtype, width, lengths, row_starts, offsets, k, with_raw=True, offset=0):
    R = x_bits.shape[0]
    x = to_device_scores(x_bits, dtype, width, offset)
    L = torch.from_numpy(lengths).cuda()
    rs = torch.from_numpy(row_starts).cuda() if row_starts is not None else None
    off = torch.from_numpy(offsets).cuda()
    pad = 64
    ob = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    rb = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    ws = vts.make_workspace(R, width, k, TORCH_DTYPE[dtype], "cuda", transform=True)
    out, raw = vts.topk_transform_ragged(
        x, L, off, k, row_starts=rs, out=ob[pad:pad + R * k],
        out_raw_indices=rb[pad:pad + R * k] if with_raw else None, workspace=ws)
    torch.cuda.synchronize()
    o = ob.cpu().numpy()
    assert np.all(o[:pad] == 0x5A5A5A5A) and np.all(o[pad + R * k:] == 0x5A5A5A5A)
    return out.cpu().numpy(), None if raw is None else raw.cpu().numpy()


def _check(x_bits, dtype, width, lengths, row_starts, offsets, k, out, raw):
    ref_out, ref_raw, base, n = oracle.topk_transform_ragged(
        x_bits[:, :width], dtype, lengths, row_starts, offsets, k)
    if raw is None:  # recover the raw indices from out (offsets are non-negative here)
        raw = np.where(out < 0, -1, out.astype(np.int64) - offsets[:, None]).astype(np.int32)
    errs = check_rows(x_bits, dtype, base, n, k, raw, ref_raw)
    want = oracle.ragged_translate(raw, offsets)
    if not np.array_equal(out, want):
        bad = np.argwhere(out != want)[:4]
        errs.append(f"out is not raw + offset at {bad.tolist()}")
    return errs


@pytest.mark.parametrize("tune", [{}, dict(nsplit=4, min_chunk=1024)])
def test_ragged_page_workload(tune):
    wl = workloads.make("page")
    rng = np.random.default_rng(31)
    offsets = rng.integers(0, 1 << 28, size=wl.rows).astype(np.int32)
    say(f"ragged transform page {wl.x.shape} {tune}")
    with tuning(**tune):
        out, raw = _run(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, offsets, wl.k)
    errs = _check(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, offsets, wl.k, out, raw)
    assert errs == [], "\n".join(errs)


def test_ragged_without_raw_output():
    wl = workloads.make("page", rows=32)
    offsets = (np.arange(wl.rows, dtype=np.int32) * 70000)
    say("ragged transform, no out_raw")
    out, raw = _run(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, offsets, wl.k,
                    with_raw=False)
    assert raw is None
    errs = _check(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, offsets, wl.k, out, None)
    assert errs == [], "\n".join(errs)


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_ragged_dtypes_misaligned(dtype):
    rng = np.random.default_rng(40 + dtype)
    R, W, k = 24, 40000, 1024
    vals = rng.standard_normal((R, W)).astype(np.float32)
    bits = (vals.view(np.uint32) if dtype == F32 else
            to_bf16_bits(vals) if dtype == BF16 else to_f16_bits(vals))
    S = W + 3
    x = np.zeros((R, S), bits.dtype)
    x[:, :W] = bits
    lengths = rng.integers(0, W, size=R).astype(np.int32)
    lengths[:3] = [0, 5, k]
    starts = np.array([rng.integers(0, W - L + 1) for L in lengths], np.int32)
    offsets = rng.integers(0, 1 << 30, size=R).astype(np.int32)
    say(f"ragged transform dtype {dtype}")
    out, raw = _run(x, dtype, W, lengths, starts, offsets, k, offset=1)
    errs = _check(x, dtype, W, lengths, starts, offsets, k, out, raw)
    assert errs == [], "\n".join(errs)


# ---------------------------------------------------------------------------
# page size 1, one page-table row per request (cu_seqlens_q)
# ---------------------------------------------------------------------------

def _requests(rng, R, lead=2, tail=1):
    """cu_seqlens_q covering rows [lead, R - tail) with 1..4 rows per request."""
    sizes = []
    left = R - lead - tail
    while left > 0:
        s = int(min(left, rng.integers(1, 5)))
        sizes.append(s)
        left -= s
    return np.concatenate([[lead], lead + np.cumsum(sizes)]).astype(np.int32)


def _run_page1(x_bits, dtype, width, lengths, row_starts, pt, cu, k, tune=None, offset=0,
               with_raw=True):
    R = x_bits.shape[0]
    x = to_device_scores(x_bits, dtype, width, offset)
    L = torch.from_numpy(lengths).cuda()
    rs = torch.from_numpy(row_starts).cuda() if row_starts is not None else None
    ptd = torch.from_numpy(pt).cuda()
    cud = torch.from_numpy(cu).cuda()
    pad = 64
    ob = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    rb = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    with tuning(**(tune or {})):  # the plan, and so the workspace size, follows the tuning
        ws = vts.make_workspace(R, width, k, TORCH_DTYPE[dtype], "cuda", transform=True)
        out, raw = vts.topk_transform_page1(x, L, ptd, cud, k, row_starts=rs,
                                            out=ob[pad:pad + R * k],
                                            out_raw_indices=rb[pad:pad + R * k] if with_raw else None,
                                            workspace=ws)
        torch.cuda.synchronize()
    o = ob.cpu().numpy()
    assert np.all(o[:pad] == 0x5A5A5A5A) and np.all(o[pad + R * k:] == 0x5A5A5A5A)
    return out.cpu().numpy(), None if raw is None else raw.cpu().numpy()


def _unpage1(out, pt, cu):
    """Raw indices back from page-size-1 outputs, for tables whose rows hold
    distinct non-negative entries (each a permutation slice): -1 stays -1."""
    R, k = out.shape
    raw = np.full((R, k), -1, np.int32)
    for r in range(R):
        b = int(np.searchsorted(cu, r, side="right")) - 1
        if b < 0 or b >= len(cu) - 1:
            continue
        order = np.argsort(pt[b], kind="stable")
        got = out[r] >= 0
        pos = np.searchsorted(pt[b], out[r][got], sorter=order)
        assert np.all(pt[b][order[pos]] == out[r][got]), f"row {r}: output not in its table row"
        raw[r][got] = order[pos]
    return raw


def _check_page1(x_bits, dtype, width, lengths, row_starts, pt, cu, k, out, raw):
    ref_out, ref_raw, base, n = oracle.topk_transform_page1(
        x_bits[:, :width], dtype, lengths, row_starts, pt, cu, k)
    if raw is None:
        raw = _unpage1(out, pt, cu)
        # a row outside every request writes only -1 (checked below): its
        # selection cannot be read back, so it takes the oracle's
        b = np.searchsorted(cu, np.arange(len(out)), side="right") - 1
        outside = (b < 0) | (b >= len(cu) - 1)
        raw[outside] = ref_raw[outside]
    errs = check_rows(x_bits, dtype, base, n, k, raw, ref_raw)
    want = oracle.page1_translate(raw, pt, cu)
    if not np.array_equal(out, want):
        bad = np.argwhere(out != want)[:4]
        errs.append(f"out is not page_table[b(r), idx] at {bad.tolist()}")
    return errs


@pytest.mark.parametrize("tune", [{}, dict(nsplit=4, min_chunk=1024)])
def test_page1_page_workload(tune):
    wl = workloads.make("page")
    rng = np.random.default_rng(51)
    cu = _requests(rng, wl.rows)
    B = len(cu) - 1
    pt = np.stack([rng.permutation(1 << 20)[: wl.width] for _ in range(B)]).astype(np.int32)
    say(f"page-size-1 transform page {wl.x.shape} requests {B} {tune}")
    out, raw = _run_page1(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, pt, cu, wl.k, tune)
    errs = _check_page1(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, pt, cu, wl.k, out, raw)
    assert errs == [], "\n".join(errs)
    assert np.all(out[:2] == -1) and np.all(out[-1] == -1)  # rows outside every request


@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_page1_dtypes_narrow_table(dtype):
    rng = np.random.default_rng(60 + dtype)
    R, W, k = 20, 30000, 512
    vals = rng.standard_normal((R, W)).astype(np.float32)
    bits = (vals.view(np.uint32) if dtype == F32 else
            to_bf16_bits(vals) if dtype == BF16 else to_f16_bits(vals))
    x = np.zeros((R, W + 5), bits.dtype)
    x[:, :W] = bits
    lengths = rng.integers(0, W, size=R).astype(np.int32)
    starts = np.array([rng.integers(0, W - L + 1) for L in lengths], np.int32)
    cu = _requests(rng, R, lead=0, tail=0)
    B = len(cu) - 1
    Wt = 20000  # narrower than some windows: indices past the table give -1
    pt = rng.integers(0, 1 << 24, size=(B, Wt)).astype(np.int32)
    say(f"page-size-1 transform dtype {dtype}")
    out, raw = _run_page1(x, dtype, W, lengths, starts, pt, cu, k, offset=3)
    errs = _check_page1(x, dtype, W, lengths, starts, pt, cu, k, out, raw)
    assert errs == [], "\n".join(errs)


# ---------------------------------------------------------------------------
# both transforms through every internal path, forced, on a reduced page batch
# ---------------------------------------------------------------------------

FORCED = {
    "careful": dict(force=1),
    "fallback": dict(force=2),
    "spill": dict(lds=64),
    "overflow": dict(lds=64, spill=64),
    "split8_spill": dict(nsplit=8, min_chunk=1024, lds=64),
    "split3_fallback": dict(nsplit=3, min_chunk=4096, force=2),
}


@pytest.mark.parametrize("with_raw", [True, False])
@pytest.mark.parametrize("path", sorted(FORCED))
def test_page1_forced_paths(path, with_raw):
    wl = workloads.make("page", rows=24)
    rng = np.random.default_rng(71)
    cu = _requests(rng, wl.rows)
    B = len(cu) - 1
    pt = np.stack([rng.permutation(1 << 20)[: wl.width] for _ in range(B)]).astype(np.int32)
    say(f"page-size-1 transform {path} raw={with_raw}")
    out, raw = _run_page1(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, pt, cu, wl.k,
                          FORCED[path], with_raw=with_raw)
    assert (raw is None) == (not with_raw)
    errs = _check_page1(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, pt, cu, wl.k, out, raw)
    assert errs == [], "\n".join(errs)


@pytest.mark.parametrize("with_raw", [True, False])
@pytest.mark.parametrize("path", sorted(FORCED))
def test_ragged_forced_paths(path, with_raw):
    wl = workloads.make("page", rows=24)
    offsets = np.random.default_rng(72).integers(0, 1 << 28, size=wl.rows).astype(np.int32)
    say(f"ragged transform {path} raw={with_raw}")
    with tuning(**FORCED[path]):
        out, raw = _run(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, offsets, wl.k,
                        with_raw=with_raw)
    errs = _check(wl.x, wl.dtype, wl.width, wl.lengths, wl.row_starts, offsets, wl.k, out, raw)
    assert errs == [], "\n".join(errs)
