"""Tie-aware comparison of a top-k result against the oracle (test infrastructure only).

A result is accepted when, for every checked row r with n valid columns:

  (i)   slots [0, min(n, k)) hold distinct window-relative indices in [0, n) and
        slots [min(n, k), k) hold -1;
  (ii)  when n <= k the indices are exactly 0, 1, ..., n-1 in order (the
        short-row convention of TensorRT-LLM PR #17821, short-row commit);
  (iii) the sorted multiset of selected values, with -0 mapped to +0, equals
        the oracle's (the exactness test of the same PR: value multiset against
        a reference top-k, signed zeros normalised);
  (iv)  the smallest selected value is >= the largest unselected valid value;
  (v)   returned values are bit copies of the selected elements, and padding
        slots hold the padding bits;
  (vi)  for the page transform, `out` equals the oracle's translation of
        `out_raw`, and `out_raw` passes (i)-(iv).

Which of several tied elements is chosen, and the order of the k slots, are
not checked: the pages leave both open (ties interchangeable, no output order).
Rows holding NaN are compared in the order the oracle documents (a NaN with
the sign bit clear above +inf, one with it set below -inf, NaNs of one sign
tied): (iii) and (iv) then compare (NaN sign class, value) pairs, so the count
of NaNs of each sign that were selected and the multiset of the other
selected values must equal the oracle's.
"""
from __future__ import annotations

import numpy as np

from . import BF16, F16, F32, PAD_BITS, page_translate


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Raw element bits -> float64, with numpy's own converters."""
    with np.errstate(invalid="ignore"):
        if dtype == F32:
            return bits.view(np.float32).astype(np.float64) if bits.dtype != np.float32 else bits.astype(np.float64)
        if dtype == BF16:
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if dtype == F16:
            return bits.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def raw_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return x.view(np.uint32) if x.dtype != np.uint32 else x
    return x.view(np.uint16) if x.dtype != np.uint16 else x


def ranks(bits: np.ndarray, dtype: int) -> tuple[np.ndarray, np.ndarray]:
    """(class, value) of each element in the oracle's order: class +1 for a
    NaN with the sign bit clear, -1 for one with it set, 0 for numbers; value
    0 for NaNs and -0 mapped to +0."""
    v = decode(bits, dtype)
    nan = np.isnan(v)
    sign = (bits.astype(np.uint64) >> (31 if dtype == F32 else 15)) & 1
    cls = np.where(nan, np.where(sign == 1, -1, 1), 0)
    return cls, np.where(nan | (v == 0), 0.0, v)


def check_rows(x: np.ndarray, dtype: int, base: np.ndarray, n: np.ndarray, k: int,
               got_idx: np.ndarray, ref_idx: np.ndarray, got_vals: np.ndarray | None = None,
               rows=None, max_report: int = 8) -> list[str]:
    """Returns a list of failure messages (empty when every checked row passes).

    x: 2-D raw bits (or float32) with rows at least base+n long.
    got_idx / ref_idx: int32[R, k] (ref may be None when only (i), (ii), (iv), (v) are wanted).
    rows: iterable of row ids to check (default: all).
    """
    bits = raw_bits(np.asarray(x), dtype)
    R = bits.shape[0]
    rows = range(R) if rows is None else rows
    errs: list[str] = []
    pad = PAD_BITS[dtype]
    for r in rows:
        if len(errs) >= max_report:
            break
        nr, b0 = int(n[r]), int(base[r])
        gi = np.asarray(got_idx[r], dtype=np.int64)
        m = min(nr, k)
        head, tail = gi[:m], gi[m:]
        if np.any(tail != -1):
            errs.append(f"row {r}: slots [{m},{k}) must be -1 (n={nr})")
            continue
        if np.any(head < 0) or np.any(head >= nr):
            errs.append(f"row {r}: index outside [0,{nr})")
            continue
        if np.unique(head).size != m:
            errs.append(f"row {r}: duplicate indices")
            continue
        if nr <= k and not np.array_equal(head, np.arange(nr)):
            errs.append(f"row {r}: short row (n={nr}<=k={k}) must be the identity")
            continue
        wbits = bits[r, b0:b0 + nr]
        wval = decode(wbits, dtype)
        if got_vals is not None:
            gv = np.asarray(got_vals[r])
            if not np.array_equal(gv[:m].astype(np.uint64), wbits[head].astype(np.uint64)):
                errs.append(f"row {r}: returned values are not bit copies of the selected elements")
                continue
            if np.any(gv[m:].astype(np.uint64) != pad):
                errs.append(f"row {r}: padding values must be {pad:#x}")
                continue
        if nr <= k:
            continue
        cls, val = ranks(wbits, dtype)

        def sorted_pairs(cols):
            o = np.lexsort((val[cols], cls[cols]))
            return cls[cols][o], val[cols][o]

        if ref_idx is not None:
            ri = np.asarray(ref_idx[r], dtype=np.int64)[:m]
            (ca, va), (cb, vb) = sorted_pairs(head), sorted_pairs(ri)
            if not (np.array_equal(ca, cb) and np.array_equal(va, vb)):
                errs.append(f"row {r}: selected value multiset differs from the oracle's")
                continue
        mask = np.ones(nr, bool)
        mask[head] = False
        if mask.any():
            cs, vs = sorted_pairs(head)
            rest = np.flatnonzero(mask)
            cu, vu = sorted_pairs(rest)
            if (cs[0], vs[0]) < (cu[-1], vu[-1]):
                errs.append(f"row {r}: a selected value is below an unselected one")
                continue
    return errs


def check_transform(x: np.ndarray, dtype: int, base: np.ndarray, n: np.ndarray, k: int,
                    got_out: np.ndarray, got_raw: np.ndarray, ref_raw: np.ndarray,
                    page_table: np.ndarray, page_table_row_starts, page_size: int,
                    rows=None) -> list[str]:
    errs = check_rows(x, dtype, base, n, k, got_raw, ref_raw, None, rows)
    if errs:
        return errs
    want = page_translate(np.asarray(got_raw, np.int32), page_table, page_table_row_starts, base,
                          page_size)
    rows = range(got_raw.shape[0]) if rows is None else rows
    for r in rows:
        if not np.array_equal(np.asarray(got_out[r]), want[r]):
            errs.append(f"row {r}: translated output differs from the transform of out_raw")
            if len(errs) >= 8:
                break
    return errs
