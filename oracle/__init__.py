"""CPU oracle for exact batched variable-length top-K selection.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers.  The HIP library never imports,
links or runs anything in this package, and this package shares no code with it.

The arithmetic lives in plain C (``vts_oracle.c``, built to ``liboracle.so`` by
``oracle.build``); this module only marshals numpy arrays into it.  Citations
for every rule are at the top of ``vts_oracle.c``.

Every function here is pinned by ``tests/test_oracle_pins.py`` against things
other than itself: a hand table of the valid-length formula, brute force over
all k-subsets of tiny rows, textbook special cases (argmax, sorted rows,
constant rows), ``torch.topk`` on the CPU as an independent library routine,
and the page-transform identities.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

F32, BF16, F16 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "f16": F16}
ITEMSIZE = {F32: 4, BF16: 2, F16: 2}
PAD_BITS = {F32: 0xFF7FFFFF, BF16: 0xFF7F, F16: 0xFBFF}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def use_library(path: str | None):
    """Points this module at another build of vts_oracle.c (None: the default one).

    Used by the mutation tests, which build copies of the oracle with a planted
    mistake and check that the pins reject them.
    """
    global _lib
    _lib = None if path is None else bind(ctypes.CDLL(path))


def bind(lib):
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.vts_oracle_valid_len.restype = ctypes.c_int64
    lib.vts_oracle_valid_len.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int64]
    lib.vts_oracle_varlen_rows.restype = None
    lib.vts_oracle_varlen_rows.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, i64p, i64p]
    lib.vts_oracle_window_rows.restype = None
    lib.vts_oracle_window_rows.argtypes = [i32p, i32p, ctypes.c_int64, ctypes.c_int64, i64p, i64p]
    lib.vts_oracle_select.restype = ctypes.c_int
    lib.vts_oracle_select.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      i64p, i64p, ctypes.c_int32, i32p, ctypes.c_void_p,
                                      ctypes.c_int]
    lib.vts_oracle_page_translate.restype = ctypes.c_int
    lib.vts_oracle_page_translate.argtypes = [i32p, ctypes.c_int64, ctypes.c_int32, i32p,
                                              ctypes.c_int64, ctypes.c_int64, i32p, i64p,
                                              ctypes.c_int32, i32p]
    return lib


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a is not None else None


def default_threads() -> int:
    """Host threads for the oracle: the visible cores, at most 16."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def valid_len(seq_len: int, next_n: int, t: int, compress_ratio: int, width: int) -> int:
    """Valid column count of row t of a request (FlashInfer top_k_varlen doc, `seq_lens`)."""
    return int(_load().vts_oracle_valid_len(seq_len, next_n, t, compress_ratio, width))


def varlen_rows(seq_lens: np.ndarray, num_rows: int, next_n: int, compress_ratio: int, width: int):
    """(base, n) per row for topk_varlen: base = 0, n from the valid-length rule."""
    s = np.ascontiguousarray(seq_lens, dtype=np.int32)
    assert num_rows % next_n == 0 and s.shape[0] == num_rows // next_n
    base = np.zeros(num_rows, np.int64)
    n = np.zeros(num_rows, np.int64)
    _load().vts_oracle_varlen_rows(_p(s, ctypes.c_int32), num_rows, next_n, compress_ratio, width,
                                   _p(base, ctypes.c_int64), _p(n, ctypes.c_int64))
    return base, n


def window_rows(lengths: np.ndarray, row_starts, width: int):
    """(base, n) per row for the page transform (SGLang fast_topk_v2 lengths/row_starts)."""
    L = np.ascontiguousarray(lengths, dtype=np.int32)
    rs = None if row_starts is None else np.ascontiguousarray(row_starts, dtype=np.int32)
    R = L.shape[0]
    base = np.zeros(R, np.int64)
    n = np.zeros(R, np.int64)
    _load().vts_oracle_window_rows(_p(L, ctypes.c_int32), _p(rs, ctypes.c_int32), R, width,
                                   _p(base, ctypes.c_int64), _p(n, ctypes.c_int64))
    return base, n


def select(x: np.ndarray, dtype: int, base: np.ndarray, n: np.ndarray, k: int,
           return_values: bool = False, nthreads: int | None = None):
    """Exact top-k of each row window by full sort.

    x: 2-D array of raw element bits (uint32 for f32, uint16 for bf16/f16) or
    float32 for f32; rows may be longer than the windows.  Returns
    (idx int32[R, k], values raw-bits[R, k] or None).
    """
    x = np.ascontiguousarray(x)
    assert x.ndim == 2 and x.dtype.itemsize == ITEMSIZE[dtype]
    R = x.shape[0]
    base = np.ascontiguousarray(base, dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    assert base.shape == (R,) and n.shape == (R,)
    assert np.all(base >= 0) and np.all(base + n <= x.shape[1])
    idx = np.empty((R, k), np.int32)
    vals = np.empty((R, k), np.uint32 if dtype == F32 else np.uint16) if return_values else None
    th = nthreads or default_threads()
    rc = _load().vts_oracle_select(x.ctypes.data, dtype, R, x.shape[1], _p(base, ctypes.c_int64),
                                   _p(n, ctypes.c_int64), k, _p(idx, ctypes.c_int32),
                                   None if vals is None else vals.ctypes.data, th)
    if rc != 0:
        raise MemoryError("oracle could not allocate its sort buffer")
    return idx, vals


def page_translate(raw: np.ndarray, page_table: np.ndarray, page_table_row_starts, base: np.ndarray,
                   page_size: int):
    """Page-table transform of window-relative indices (FlashInfer PR body, "Description")."""
    raw = np.ascontiguousarray(raw, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    R, k = raw.shape
    ptrs = None if page_table_row_starts is None else np.ascontiguousarray(page_table_row_starts,
                                                                           dtype=np.int32)
    base = np.ascontiguousarray(base, dtype=np.int64)
    out = np.empty((R, k), np.int32)
    ovf = _load().vts_oracle_page_translate(_p(raw, ctypes.c_int32), R, k, _p(pt, ctypes.c_int32),
                                            pt.shape[1], pt.shape[1], _p(ptrs, ctypes.c_int32),
                                            _p(base, ctypes.c_int64), page_size,
                                            _p(out, ctypes.c_int32))
    if ovf:
        raise OverflowError("translated index does not fit in int32")
    return out


def ragged_translate(raw: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Ragged-KV transform of window-relative indices (SGLang TopK_Ops page,
    fast_topk_transform_ragged_fused): idx + topk_indices_offset[r], -1 kept."""
    raw = np.asarray(raw, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64).reshape(-1, 1)
    out = np.where(raw < 0, -1, raw + off)
    if np.any(out > np.iinfo(np.int32).max) or np.any((raw >= 0) & (out < np.iinfo(np.int32).min)):
        raise OverflowError("translated index does not fit in int32")
    return out.astype(np.int32)


def row_requests(cu_seqlens_q: np.ndarray, num_rows: int) -> np.ndarray:
    """Request of each row (SGLang TopK_Ops page, `cu_seqlens_q`): the b with
    cu[b] <= r < cu[b + 1], or -1 outside [cu[0], cu[-1])."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    r = np.arange(num_rows, dtype=np.int64)
    b = np.searchsorted(cu, r, side="right") - 1
    inside = (r >= cu[0]) & (r < cu[-1]) if cu.size > 1 else np.zeros(num_rows, bool)
    return np.where(inside, b, -1)


def page1_translate(raw: np.ndarray, page_table: np.ndarray, cu_seqlens_q: np.ndarray) -> np.ndarray:
    """Page-size-1 transform (SGLang TopK_Ops page, fast_topk_transform_fused):
    page_table[b(r), idx], -1 for unused slots, rows outside every request and
    indices past the table."""
    raw = np.asarray(raw, dtype=np.int64)
    R, k = raw.shape
    pt = np.asarray(page_table, dtype=np.int64)
    b = row_requests(cu_seqlens_q, R)
    out = np.full((R, k), -1, np.int64)
    for r in range(R):
        if b[r] < 0:
            continue
        for j in range(k):
            i = raw[r, j]
            if 0 <= i < pt.shape[1]:
                out[r, j] = pt[b[r], i]
    return out.astype(np.int32)


def topk_transform_page1(scores: np.ndarray, dtype: int, lengths: np.ndarray, row_starts,
                         page_table: np.ndarray, cu_seqlens_q: np.ndarray, k: int,
                         nthreads: int | None = None):
    """Oracle of the page-size-1 transform: (out, out_raw, base, n)."""
    R, W = scores.shape
    base, n = window_rows(lengths, row_starts, W)
    raw, _ = select(scores, dtype, base, n, k, False, nthreads)
    return page1_translate(raw, page_table, cu_seqlens_q), raw, base, n


def topk_transform_ragged(scores: np.ndarray, dtype: int, lengths: np.ndarray, row_starts,
                          offsets: np.ndarray, k: int, nthreads: int | None = None):
    """Oracle of the ragged transform: (out, out_raw, base, n)."""
    R, W = scores.shape
    base, n = window_rows(lengths, row_starts, W)
    raw, _ = select(scores, dtype, base, n, k, False, nthreads)
    return ragged_translate(raw, offsets), raw, base, n


def topk_varlen(logits: np.ndarray, dtype: int, seq_lens: np.ndarray, k: int, next_n: int = 1,
                compress_ratio: int = 1, return_values: bool = False, nthreads: int | None = None):
    """Oracle of topk_varlen: (idx, values-or-None, n per row)."""
    R, W = logits.shape
    base, n = varlen_rows(seq_lens, R, next_n, compress_ratio, W)
    idx, vals = select(logits, dtype, base, n, k, return_values, nthreads)
    return idx, vals, n


def _as_float(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Raw element bits -> float64 values."""
    if dtype == F32:
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16).view(np.float16).astype(np.float64)


def select_ordered(x: np.ndarray, dtype: int, base: np.ndarray, n: np.ndarray, k: int, tie: str,
                   return_values: bool = False, nthreads: int | None = None):
    """Deterministic mode (FlashInfer page-size PR body on the SGLang PR #33237
    page, "Description" and "Performance": a post-sort of the outputs and a
    SMALL/LARGE choice among tied values).  Every value above the k-th largest,
    then, of those equal to it, the ones at the smallest ("small") or largest
    ("large") columns; each row listed by value descending, then column
    ascending.

    "small" takes `select` itself, whose full sort already orders ties by
    ascending column.  "large" runs `select` on each window reversed (column j
    read as n - 1 - j), so its tie order favours the largest original columns,
    and maps the columns back.  Both then sort each row's entries by value
    descending, column ascending (rows with n <= k come from `select` in column
    order: every column, then -1).  Values compare as `select` compares them:
    as numbers, so -0 equals +0 (TensorRT-LLM PR #17821, "Test coverage":
    signed zeros normalised), with every NaN whose sign bit is clear above
    +inf and every NaN whose sign bit is set below -inf, NaNs of one sign
    equal to each other.
    """
    assert tie in ("small", "large")
    R = x.shape[0]
    n = np.asarray(n, np.int64)
    base = np.asarray(base, np.int64)
    if tie == "small":
        idx, vals = select(x, dtype, base, n, k, True, nthreads)
    else:
        wmax = max(int(n.max()) if R else 0, 1)
        xr = np.zeros((R, wmax), x.dtype)
        for r in range(R):
            m = int(n[r])
            if m:
                xr[r, :m] = x[r, base[r]:base[r] + m][::-1]
        idx_r, vals = select(xr, dtype, np.zeros(R, np.int64), n, k, True, nthreads)
        idx = np.where(idx_r < 0, -1, (n[:, None] - 1 - idx_r)).astype(np.int32)
    sign_shift = 31 if dtype == F32 else 15
    for r in range(R):
        m = min(int(n[r]), k)
        v = _as_float(vals[r, :m], dtype)
        nan = np.isnan(v)
        neg = (vals[r, :m].astype(np.uint64) >> sign_shift) & 1
        cls = np.where(nan, np.where(neg == 1, -1, 1), 0)  # NaN sign class, 0 for numbers
        v = np.where(nan, 0.0, v)
        # NaN class descending, then value descending, then column ascending
        order = np.lexsort((idx[r, :m], -v, -cls))
        idx[r, :m] = idx[r, :m][order]
        vals[r, :m] = vals[r, :m][order]
    return idx, (vals if return_values else None)


def topk_varlen_ordered(logits: np.ndarray, dtype: int, seq_lens: np.ndarray, k: int, tie: str,
                        next_n: int = 1, compress_ratio: int = 1, return_values: bool = False,
                        nthreads: int | None = None):
    """Oracle of topk_varlen_ordered: (idx, values-or-None, n per row)."""
    R, W = logits.shape
    base, n = varlen_rows(seq_lens, R, next_n, compress_ratio, W)
    idx, vals = select_ordered(logits, dtype, base, n, k, tie, return_values, nthreads)
    return idx, vals, n


def _select_windows(scores, dtype, base, n, k, tie, nthreads):
    """Window-relative top-k indices: `select`, or `select_ordered` with a tie."""
    if tie is None:
        return select(scores, dtype, base, n, k, False, nthreads)[0]
    return select_ordered(scores, dtype, base, n, k, tie, False, nthreads)[0]


def topk_page_table_transform_ordered(scores: np.ndarray, dtype: int, lengths: np.ndarray,
                                      row_starts, page_table: np.ndarray, page_table_row_starts,
                                      page_size: int, k: int, tie: str, nthreads: int | None = None):
    """Oracle of the page transform in the deterministic mode: the ordered
    selection of each window (`select_ordered`), translated slot by slot
    (FlashInfer page-size PR body, "Description": `out_raw_indices` stays
    aligned with `out` through the post-sort).  Returns (out, out_raw, base, n)."""
    R, W = scores.shape
    base, n = window_rows(lengths, row_starts, W)
    raw = _select_windows(scores, dtype, base, n, k, tie, nthreads)
    return page_translate(raw, page_table, page_table_row_starts, base, page_size), raw, base, n


def topk_transform_ragged_ordered(scores, dtype, lengths, row_starts, offsets, k, tie,
                                  nthreads=None):
    """Oracle of the ragged transform in the deterministic mode: (out, out_raw, base, n)."""
    R, W = scores.shape
    base, n = window_rows(lengths, row_starts, W)
    raw = _select_windows(scores, dtype, base, n, k, tie, nthreads)
    return ragged_translate(raw, offsets), raw, base, n


def topk_transform_page1_ordered(scores, dtype, lengths, row_starts, page_table, cu_seqlens_q, k,
                                 tie, nthreads=None):
    """Oracle of the page-size-1 transform in the deterministic mode: (out, out_raw, base, n)."""
    R, W = scores.shape
    base, n = window_rows(lengths, row_starts, W)
    raw = _select_windows(scores, dtype, base, n, k, tie, nthreads)
    return page1_translate(raw, page_table, cu_seqlens_q), raw, base, n


def topk_page_table_transform(scores: np.ndarray, dtype: int, lengths: np.ndarray, row_starts,
                              page_table: np.ndarray, page_table_row_starts, page_size: int, k: int,
                              nthreads: int | None = None):
    """Oracle of the fused page transform: (out, out_raw, base, n)."""
    R, W = scores.shape
    base, n = window_rows(lengths, row_starts, W)
    raw, _ = select(scores, dtype, base, n, k, False, nthreads)
    out = page_translate(raw, page_table, page_table_row_starts, base, page_size)
    return out, raw, base, n
