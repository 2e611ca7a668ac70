"""GPU parity of the ragged-KV transform (SGLang TopK_Ops page,
fast_topk_transform_ragged_fused) through the C ABI: the selection is checked
against the CPU oracle with the tie-aware checker, and `out` must equal the
oracle's translation of the GPU's own raw indices position by position."""
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
