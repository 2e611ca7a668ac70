"""The allocation-free entry point vts_topk_varlen_noalloc, through the C
ABI: its output must match vts_topk_varlen's (the workspace entry point) on
the same inputs, tie-aware, and the oracle's; three calls in a row on the
device's one scratch array with different layouts, the last one smaller."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import varlen_top_select_amd as vts
import workloads
from oracle.check import check_rows
from tests.gpu_util import TORCH_DTYPE, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)


def _run_both(wl):
    dt = TORCH_DTYPE[wl.dtype]
    raw = torch.from_numpy(wl.x.view(np.int32 if wl.dtype == 0 else np.int16)).cuda()
    x = raw.view(dt)[:, : wl.width]
    seq = torch.from_numpy(wl.seq_lens).cuda()
    R, k = wl.rows, wl.k
    lib = vts.library()
    stream = torch.cuda.current_stream().cuda_stream
    idx_na = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    vals_na = torch.empty((R, k), dtype=dt, device="cuda")
    st = lib.vts_topk_varlen_noalloc(x.data_ptr(), wl.dtype, R, wl.width, x.stride(0),
                                     seq.data_ptr(), k, wl.next_n, wl.compress_ratio, None,
                                     idx_na.data_ptr(), vals_na.data_ptr(), stream)
    assert st == 0, lib.vts_status_string(st)
    torch.cuda.synchronize()
    ws = vts.make_workspace(R, wl.width, k, dt, "cuda")
    idx_ws = torch.empty((R, k), dtype=torch.int32, device="cuda")
    vals_ws = torch.empty((R, k), dtype=dt, device="cuda")
    st = lib.vts_topk_varlen(x.data_ptr(), wl.dtype, R, wl.width, x.stride(0), seq.data_ptr(), k,
                             wl.next_n, wl.compress_ratio, None, idx_ws.data_ptr(),
                             vals_ws.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, lib.vts_status_string(st)
    torch.cuda.synchronize()
    rawt = torch.int32 if wl.dtype == 0 else torch.int16
    as_bits = (lambda v: v.view(rawt).cpu().numpy().view(np.uint32 if wl.dtype == 0 else np.uint16))
    return idx_na.cpu().numpy(), as_bits(vals_na), idx_ws.cpu().numpy(), as_bits(vals_ws)


def _check(wl):
    idx_na, v_na, idx_ws, v_ws = _run_both(wl)
    base, n = oracle.varlen_rows(wl.seq_lens, wl.rows, wl.next_n, wl.compress_ratio, wl.width)
    # against the workspace entry point's output (tie-aware), then the oracle's
    errs = check_rows(wl.x, wl.dtype, base, n, wl.k, idx_na, idx_ws, v_na)
    assert errs == [], "\n".join(errs)
    ref, _, _ = oracle.topk_varlen(wl.x[:, :wl.width], wl.dtype, wl.seq_lens, wl.k, wl.next_n,
                                   wl.compress_ratio)
    errs = check_rows(wl.x, wl.dtype, base, n, wl.k, idx_na, ref, v_na)
    assert errs == [], "\n".join(errs)


def test_noalloc_matches_the_workspace_entry_point():
    # dsv32 rows split in four (split rows publish their lists in the scratch),
    # then the long batch (1024 rows: its row tickets lie where the first
    # call's counts were), then a smaller DSv4 MTP batch
    for name, kw in (("dsv32", {}), ("long", {}), ("dsv4_mtp", dict(rows=64))):
        wl = workloads.make(name, hint=False, **kw) if name != "dsv4_mtp" else workloads.make(name, **kw)
        say(f"noalloc {name} {wl.x.shape}")
        _check(wl)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    x = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    seq = torch.zeros(2048, dtype=torch.int32, device="cuda")
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    # 2048 rows of 262144 columns: 2048 units need more than the 32 MiB scratch;
    # rejected on the host before anything is enqueued
    st = vts.library().vts_topk_varlen_noalloc(x.data_ptr(), 0, 2048, 262144, 262144,
                                               seq.data_ptr(), 2048, 1, 1, None, out.data_ptr(),
                                               None, torch.cuda.current_stream().cuda_stream)
    assert st == -5
    assert b"scratch" in vts.library().vts_status_string(st)
