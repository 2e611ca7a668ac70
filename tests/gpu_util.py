"""Helpers for the GPU parity tests: run the HIP path on a workload, run the
oracle on the same inputs, compare with the tie-aware checker."""
from __future__ import annotations

import contextlib
import sys

import numpy as np
import torch

import oracle
import varlen_top_select_amd as vts
from oracle.check import check_rows, check_transform

TORCH_DTYPE = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}
RAW_TORCH = {0: torch.int32, 1: torch.int16, 2: torch.int16}


def say(msg: str) -> None:
    """Names the case before a GPU step, so a failure can be traced to it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device_scores(x_bits: np.ndarray, dtype: int, width: int, offset: int = 0):
    """Raw bits [R, S] -> device tensor view [R, width] (optionally starting
    `offset` elements into a larger allocation, to misalign the base)."""
    R, S = x_bits.shape
    flat = np.zeros(R * S + offset + 64, dtype=x_bits.dtype)
    flat[offset:offset + R * S] = x_bits.reshape(-1)
    raw = torch.from_numpy(flat.view(np.int32 if dtype == 0 else np.int16)).cuda()
    t = raw.view(TORCH_DTYPE[dtype])
    return t[offset:offset + R * S].view(R, S)[:, :width]


@contextlib.contextmanager
def tuning(**kw):
    keys = dict(nsplit=vts.TUNE_NSPLIT, force=vts.TUNE_FORCE_PATH, lds=vts.TUNE_LDS_SLOTS,
                spill=vts.TUNE_SPILL_SLOTS, sigma=vts.TUNE_SAMPLE_SIGMA,
                min_chunk=vts.TUNE_MIN_CHUNK, likely=vts.TUNE_LIKELY_SIGMA,
                no_balance=vts.TUNE_NO_BALANCE, hint_rung=vts.TUNE_HINT_RUNG)
    try:
        for k, v in kw.items():
            vts.set_tuning(keys[k], v)
        yield
    finally:
        for k in kw:
            vts.set_tuning(keys[k], 0)


def run_varlen(wl, use_hint: bool = True, offset: int = 0, canary: bool = True,
               return_values: bool | None = None, tie: str | None = None, sort: bool = True):
    """Runs topk_varlen (topk_varlen_ordered with `tie`, unsorted if not
    `sort`) on the GPU; returns (idx, vals or None, stats) as numpy."""
    x = to_device_scores(wl.x, wl.dtype, wl.width, offset)
    seq = torch.from_numpy(wl.seq_lens).cuda()
    rv = wl.return_values if return_values is None else return_values
    R, k = wl.rows, wl.k
    pad = 64
    idx_buf = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    out_idx = idx_buf[pad:pad + R * k]
    vals_buf = None
    out_vals = None
    if rv:
        vals_buf = torch.full((R * k + 2 * pad,), 0x5A5A, dtype=RAW_TORCH[wl.dtype], device="cuda")
        out_vals = vals_buf[pad:pad + R * k].view(TORCH_DTYPE[wl.dtype])
    hint = None
    if use_hint and wl.pre_idx is not None:
        hint = torch.from_numpy(wl.pre_idx).cuda()
    ws = vts.make_workspace(R, wl.width, k, TORCH_DTYPE[wl.dtype], "cuda")
    kw = dict(pre_idx=hint, compress_ratio=wl.compress_ratio, next_n=wl.next_n, return_values=rv,
              out_indices=out_idx, out_values=out_vals, workspace=ws)
    if tie is None:
        idx, vals = vts.topk_varlen(x, seq, k, **kw)
    else:
        idx, vals = vts.topk_varlen_ordered(x, seq, k, tie_break=tie, sort=sort, **kw)
    torch.cuda.synchronize()
    stats = vts.workspace_stats(ws)
    # self-restoring workspace: every ticket is back to zero
    L = _ticket_region(ws, R)
    assert int(L.abs().sum()) == 0, "split-row tickets were not restored to zero"
    if canary:
        ib = idx_buf.cpu().numpy()
        assert np.all(ib[:pad] == 0x5A5A5A5A) and np.all(ib[pad + R * k:] == 0x5A5A5A5A), \
            "write outside out_indices"
        if rv:
            vb = vals_buf.cpu().numpy()
            assert np.all(vb[:pad] == 0x5A5A) and np.all(vb[pad + R * k:] == 0x5A5A), \
                "write outside out_values"
    idx_np = idx.cpu().numpy()
    vals_np = None
    if rv:
        v = vals.contiguous().view(RAW_TORCH[wl.dtype]).cpu().numpy()
        vals_np = v.view(np.uint32) if wl.dtype == 0 else v.view(np.uint16)
    return idx_np, vals_np, stats


def _ticket_region(ws: torch.Tensor, rows: int) -> torch.Tensor:
    return ws[256:256 + 4 * rows].view(torch.int32)


def check_varlen(wl, idx, vals, rows=None) -> list[str]:
    ref_idx, _, n = oracle.topk_varlen(wl.x[:, :wl.width], wl.dtype, wl.seq_lens, wl.k,
                                       wl.next_n, wl.compress_ratio)
    base = np.zeros(wl.rows, np.int64)
    return check_rows(wl.x, wl.dtype, base, n, wl.k, idx, ref_idx, vals, rows)


def run_transform(wl, with_raw: bool = True, ptrs: bool = True, starts: bool = True,
                  offset: int = 0, tie: str | None = None, sort: bool = True):
    x = to_device_scores(wl.x, wl.dtype, wl.width, offset)
    L = torch.from_numpy(wl.lengths).cuda()
    rs = torch.from_numpy(wl.row_starts).cuda() if starts else None
    pt = torch.from_numpy(wl.page_table).cuda()
    pr = torch.from_numpy(wl.page_table_row_starts).cuda() if ptrs else None
    R, k = wl.rows, wl.k
    pad = 64
    ob = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    rb = torch.full((R * k + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    ws = vts.make_workspace(R, wl.width, k, TORCH_DTYPE[wl.dtype], "cuda", transform=True)
    out, raw = vts.topk_page_table_transform(
        x, L, pt, k, page_size=wl.page_size, row_starts=rs, page_table_row_starts=pr,
        out=ob[pad:pad + R * k], out_raw_indices=rb[pad:pad + R * k] if with_raw else None,
        workspace=ws, tie_break=tie, sort=sort)
    torch.cuda.synchronize()
    stats = vts.workspace_stats(ws)
    assert int(_ticket_region(ws, R).abs().sum()) == 0
    o, r = ob.cpu().numpy(), rb.cpu().numpy()
    assert np.all(o[:pad] == 0x5A5A5A5A) and np.all(o[pad + R * k:] == 0x5A5A5A5A)
    if not with_raw:
        assert np.all(r == 0x5A5A5A5A), "out_raw written although not requested"
    return o[pad:pad + R * k].reshape(R, k), (r[pad:pad + R * k].reshape(R, k) if with_raw else None), stats


def check_transform_wl(wl, out, raw, ptrs: bool = True, starts: bool = True) -> list[str]:
    rs = wl.row_starts if starts else None
    pr = wl.page_table_row_starts if ptrs else None
    ref_out, ref_raw, base, n = oracle.topk_page_table_transform(
        wl.x[:, :wl.width], wl.dtype, wl.lengths, rs, wl.page_table, pr, wl.page_size, wl.k)
    if raw is None:
        # no out_raw: invert the (injective) translation of every window column
        raw = np.full_like(out, -1)
        for r in range(wl.rows):
            m = int(n[r])
            if m == 0:
                continue
            cols = np.arange(m, dtype=np.int32)[None, :]
            t = oracle.page_translate(cols, wl.page_table[r:r + 1], None if pr is None else pr[r:r + 1],
                                      base[r:r + 1], wl.page_size)[0]
            inv = {int(v): j for j, v in enumerate(t) if v >= 0}
            raw[r] = [inv.get(int(v), -2) if v >= 0 else -1 for v in out[r]]
    return check_transform(wl.x, wl.dtype, base, n, wl.k, out, raw, ref_raw, wl.page_table, pr,
                           wl.page_size)
