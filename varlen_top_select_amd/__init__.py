"""Python binding of libvts: exact batched variable-length top-K selection on MI355X.

Argument marshalling only.  Every step of the selection runs in the HIP
kernels of ``libvts.so`` (built from ``csrc/`` by ``varlen_top_select_amd.build``);
PyTorch supplies device memory and the stream.  There is no fallback: if the
library is missing or the device is not gfx950, the calls raise.

    topk_varlen(logits, seq_lens, top_k, ...)            -> (indices, values | None)
    topk_page_table_transform(scores, lengths, table, top_k, ...) -> (out, out_raw | None)
    topk_transform_ragged(scores, lengths, offsets, top_k, ...)   -> (out, out_raw | None)
    topk_transform_page1(scores, lengths, table, cu_seqlens_q, top_k, ...) -> (out, out_raw | None)

Each has a deterministic mode (``tie_break="small"`` or ``"large"``; the
``topk_varlen_ordered`` entry point, or the ``tie_break`` argument of the
transforms): a unique selection, in canonical order unless ``sort=False``.

The C entry points, their argument contracts and the page citations are in
``include/vts.h``.
"""
from __future__ import annotations

import ctypes
import os
import warnings

import torch

__all__ = ["topk_varlen", "topk_varlen_noalloc", "topk_varlen_ordered", "topk_page_table_transform", "topk_transform_ragged",
           "topk_transform_page1",
           "workspace_bytes", "make_workspace",
           "set_tuning", "workspace_stats", "VtsError", "library", "LIB_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvts.so")

OK, WARN_HINT_DISCARDED = 0, 1
TUNE_NSPLIT, TUNE_FORCE_PATH, TUNE_LDS_SLOTS, TUNE_SPILL_SLOTS, TUNE_SAMPLE_SIGMA = 1, 2, 3, 4, 5
TUNE_MIN_CHUNK = 6
TUNE_LIKELY_SIGMA = 7
TUNE_NO_BALANCE = 8
TUNE_HINT_RUNG = 9

_DTYPE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class VtsError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


_lib = None


def library():
    """The loaded libvts.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m varlen_top_select_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.vts_topk_varlen.restype = ctypes.c_int
    lib.vts_topk_varlen.argtypes = [vp, i32, i64, i64, i64, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.vts_topk_varlen_noalloc.restype = ctypes.c_int
    lib.vts_topk_varlen_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, i32, i32, i32, vp, vp, vp,
                                            vp]
    lib.vts_topk_varlen_ordered.restype = ctypes.c_int
    lib.vts_topk_varlen_ordered.argtypes = [vp, i32, i64, i64, i64, vp, i32, i32, i32, vp, vp, vp,
                                            vp, sz, vp, i32]
    lib.vts_topk_transform_page1.restype = ctypes.c_int
    lib.vts_topk_transform_page1.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i64, i64, vp, i64,
                                             i32, vp, vp, vp, sz, vp]
    lib.vts_topk_transform_ragged.restype = ctypes.c_int
    lib.vts_topk_transform_ragged.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, vp, vp, vp,
                                              sz, vp]
    lib.vts_topk_page_table_transform.restype = ctypes.c_int
    lib.vts_topk_page_table_transform.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i64, i64, vp,
                                                  i32, i32, vp, vp, vp, sz, vp]
    for name in ("vts_topk_page_table_transform", "vts_topk_transform_ragged",
                 "vts_topk_transform_page1"):
        f = getattr(lib, name + "_ordered")
        f.restype = ctypes.c_int
        f.argtypes = getattr(lib, name).argtypes + [i32]
    for name in ("vts_topk_varlen_workspace_bytes", "vts_page_transform_workspace_bytes"):
        f = getattr(lib, name)
        f.restype = sz
        f.argtypes = [i64, i64, i32, i32]
    lib.vts_workspace_init.restype = ctypes.c_int
    lib.vts_workspace_init.argtypes = [vp, sz, vp]
    lib.vts_status_string.restype = ctypes.c_char_p
    lib.vts_status_string.argtypes = [ctypes.c_int]
    lib.vts_workspace_stats.restype = ctypes.c_int
    lib.vts_workspace_stats.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), i32, vp]
    lib.vts_set_tuning.restype = ctypes.c_int
    lib.vts_set_tuning.argtypes = [i32, i64]
    _lib = lib
    return lib


def _check(fn: str, status: int) -> int:
    if status < 0:
        raise VtsError(fn, status, library().vts_status_string(status).decode())
    return status


def _stream_ptr(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def workspace_bytes(num_rows: int, width: int, top_k: int, dtype: torch.dtype,
                    transform: bool = False) -> int:
    lib = library()
    f = lib.vts_page_transform_workspace_bytes if transform else lib.vts_topk_varlen_workspace_bytes
    return int(f(num_rows, width, top_k, _DTYPE[dtype]))


def make_workspace(num_rows: int, width: int, top_k: int, dtype: torch.dtype, device,
                   transform: bool = False, stream=None) -> torch.Tensor:
    """A zero-filled workspace for calls of this shape (allocate once, reuse)."""
    n = workspace_bytes(num_rows, width, top_k, dtype, transform)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check("vts_workspace_init",
           library().vts_workspace_init(ws.data_ptr(), n, _stream_ptr(stream, ws.device)))
    return ws


# one zeroed workspace per (device, stream), grown on demand (the caller may pass its own)
_WS_CACHE: dict = {}


def _default_workspace(need: int, device, stream_ptr: int) -> torch.Tensor:
    key = (device.index, stream_ptr)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            # allocating and zeroing here would record both into the graph
            raise RuntimeError(
                "no workspace for this shape on the capturing stream: pass workspace= "
                "(make_workspace) or make one eager call of this shape on this stream "
                "before capture")
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _check("vts_workspace_init", library().vts_workspace_init(ws.data_ptr(), need, stream_ptr))
        _WS_CACHE[key] = ws
    return ws


def _call(name: str, args: tuple, tie) -> int:
    """Calls the C entry point `name` (its *_ordered variant with a tie code)."""
    if tie is None:
        return _check(name, getattr(library(), name)(*args))
    return _check(name + "_ordered", getattr(library(), name + "_ordered")(*args, tie))


def _check_scores(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if x.dtype not in _DTYPE:
        raise ValueError(f"{name} dtype must be float32, bfloat16 or float16")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if x.stride(1) != 1 or (x.shape[0] > 1 and x.stride(0) < x.shape[1]):
        raise ValueError(f"{name} rows must be contiguous (inner stride 1)")


def _i32(t: torch.Tensor, name: str, numel: int, device):
    if t.dtype != torch.int32 or not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor on {device}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements")
    return t


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (t.dtype != dtype or t.device != device or not t.is_contiguous()
            or t.numel() != shape[0] * shape[1] or t.data_ptr() % 16):
        raise ValueError(f"{name}: expected a contiguous, 16-byte aligned {dtype} buffer of "
                         f"{shape[0]}x{shape[1]} elements on {device}")
    return t.view(shape)


def topk_varlen(logits: torch.Tensor, seq_lens: torch.Tensor, top_k: int,
                pre_idx: torch.Tensor | None = None, compress_ratio: int = 1, next_n: int = 1,
                return_values: bool = False, out_indices: torch.Tensor | None = None,
                out_values: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None):
    """Exact top-k of each row's valid prefix (see vts_topk_varlen in include/vts.h)."""
    return _varlen(logits, seq_lens, top_k, pre_idx, compress_ratio, next_n, return_values,
                   out_indices, out_values, workspace, stream, None)


def topk_varlen_noalloc(logits: torch.Tensor, seq_lens: torch.Tensor, top_k: int,
                        out_indices: torch.Tensor, out_values: torch.Tensor | None = None,
                        pre_idx: torch.Tensor | None = None, compress_ratio: int = 1,
                        next_n: int = 1, stream=None):
    """topk_varlen without a workspace: the library's fixed device scratch
    (vts_topk_varlen_noalloc in include/vts.h).  The caller passes the
    outputs; nothing is allocated.  Calls that can overlap on one device race."""
    _check_scores(logits, "logits")
    R, W = logits.shape
    dev = logits.device
    if next_n < 1 or R % next_n:
        raise ValueError("num_rows must be a multiple of next_n")
    seq_lens = _i32(seq_lens, "seq_lens", R // next_n, dev)
    if out_indices is None:
        raise ValueError("out_indices is required")
    idx = _out(out_indices, (R, top_k), torch.int32, dev, "out_indices")
    vals = None if out_values is None else _out(out_values, (R, top_k), logits.dtype, dev,
                                                "out_values")
    st = library().vts_topk_varlen_noalloc(
        logits.data_ptr(), _DTYPE[logits.dtype], R, W, logits.stride(0) if R > 1 else W,
        seq_lens.data_ptr(), top_k, next_n, compress_ratio, _ptr(pre_idx), idx.data_ptr(),
        _ptr(vals), _stream_ptr(stream, dev))
    _check("vts_topk_varlen_noalloc", st)
    return idx, vals


TIE_BREAK = {"small": 1, "large": 2}
TIE_UNSORTED = 4


def _tie_code(tie_break, sort: bool):
    """C tie_break argument of the deterministic mode (None: unordered)."""
    if tie_break is None:
        if not sort:
            raise ValueError("sort=False needs a tie_break")
        return None
    if tie_break not in TIE_BREAK:
        raise ValueError(f"tie_break must be one of {sorted(TIE_BREAK)}")
    return TIE_BREAK[tie_break] | (0 if sort else TIE_UNSORTED)


def topk_varlen_ordered(logits: torch.Tensor, seq_lens: torch.Tensor, top_k: int,
                        tie_break: str = "small", pre_idx: torch.Tensor | None = None,
                        compress_ratio: int = 1, next_n: int = 1, return_values: bool = False,
                        out_indices: torch.Tensor | None = None,
                        out_values: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None, sort: bool = True):
    """topk_varlen in canonical order (value descending, column ascending) with
    the ties at the k-th value taken at the smallest or largest columns (see
    vts_topk_varlen_ordered in include/vts.h); sort=False: the same set in no
    particular order."""
    return _varlen(logits, seq_lens, top_k, pre_idx, compress_ratio, next_n, return_values,
                   out_indices, out_values, workspace, stream, _tie_code(tie_break, sort))


def _varlen(logits, seq_lens, top_k, pre_idx, compress_ratio, next_n, return_values, out_indices,
            out_values, workspace, stream, tie):
    _check_scores(logits, "logits")
    R, W = logits.shape
    dev = logits.device
    if next_n < 1 or R % next_n:
        raise ValueError("num_rows must be a multiple of next_n")
    seq_lens = _i32(seq_lens, "seq_lens", R // next_n, dev)
    idx = _out(out_indices, (R, top_k), torch.int32, dev, "out_indices")
    vals = _out(out_values, (R, top_k), logits.dtype, dev, "out_values") if return_values else None
    if pre_idx is not None:
        if (pre_idx.dtype != torch.int32 or pre_idx.device != dev or not pre_idx.is_contiguous()
                or tuple(pre_idx.shape) != (R // next_n, top_k)):
            warnings.warn("pre_idx malformed; running without a hint", RuntimeWarning)
            pre_idx = None
    sp = _stream_ptr(stream, dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes(R, W, top_k, logits.dtype), dev, sp)
    args = (logits.data_ptr(), _DTYPE[logits.dtype], R, W, logits.stride(0) if R > 1 else W,
            seq_lens.data_ptr(), top_k, next_n, compress_ratio, _ptr(pre_idx), idx.data_ptr(),
            _ptr(vals), workspace.data_ptr(), workspace.numel(), sp)
    if tie is None:
        st = library().vts_topk_varlen(*args)
        _check("vts_topk_varlen", st)
    else:
        st = library().vts_topk_varlen_ordered(*args, tie)
        _check("vts_topk_varlen_ordered", st)
    if st == WARN_HINT_DISCARDED:
        warnings.warn("pre_idx unusable; ran without a hint", RuntimeWarning)
    return idx, vals


def topk_page_table_transform(scores: torch.Tensor, lengths: torch.Tensor,
                              src_page_table: torch.Tensor, top_k: int, page_size: int = 1,
                              row_starts: torch.Tensor | None = None,
                              page_table_row_starts: torch.Tensor | None = None,
                              out: torch.Tensor | None = None,
                              out_raw_indices: torch.Tensor | None = None,
                              return_raw: bool = False, workspace: torch.Tensor | None = None,
                              stream=None, tie_break: str | None = None, sort: bool = True):
    """Top-k over row windows fused with the page-table transform (include/vts.h);
    with tie_break, in the deterministic mode."""
    tie = _tie_code(tie_break, sort)
    _check_scores(scores, "scores")
    R, W = scores.shape
    dev = scores.device
    lengths = _i32(lengths, "lengths", R, dev)
    if row_starts is not None:
        row_starts = _i32(row_starts, "row_starts", R, dev)
    if page_table_row_starts is not None:
        page_table_row_starts = _i32(page_table_row_starts, "page_table_row_starts", R, dev)
    pt = src_page_table
    if pt.dtype != torch.int32 or pt.dim() != 2 or pt.device != dev or pt.stride(1) != 1:
        raise ValueError("src_page_table must be a 2-D int32 tensor with contiguous rows")
    o = _out(out, (R, top_k), torch.int32, dev, "out")
    raw = None
    if out_raw_indices is not None or return_raw:
        raw = _out(out_raw_indices, (R, top_k), torch.int32, dev, "out_raw_indices")
    sp = _stream_ptr(stream, dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes(R, W, top_k, scores.dtype, True), dev, sp)
    args = (scores.data_ptr(), _DTYPE[scores.dtype], R, W, scores.stride(0) if R > 1 else W,
            lengths.data_ptr(), _ptr(row_starts), pt.data_ptr(), pt.stride(0), pt.shape[1],
            _ptr(page_table_row_starts), page_size, top_k, o.data_ptr(), _ptr(raw),
            workspace.data_ptr(), workspace.numel(), sp)
    _call("vts_topk_page_table_transform", args, tie)
    return o, raw


def topk_transform_ragged(scores: torch.Tensor, lengths: torch.Tensor,
                          topk_indices_offset: torch.Tensor, top_k: int,
                          row_starts: torch.Tensor | None = None, out: torch.Tensor | None = None,
                          out_raw_indices: torch.Tensor | None = None, return_raw: bool = False,
                          workspace: torch.Tensor | None = None, stream=None,
                          tie_break: str | None = None, sort: bool = True):
    """Top-k over row windows, each index offset into a ragged KV buffer (include/vts.h);
    with tie_break, in the deterministic mode."""
    tie = _tie_code(tie_break, sort)
    _check_scores(scores, "scores")
    R, W = scores.shape
    dev = scores.device
    lengths = _i32(lengths, "lengths", R, dev)
    offsets = _i32(topk_indices_offset, "topk_indices_offset", R, dev)
    if row_starts is not None:
        row_starts = _i32(row_starts, "row_starts", R, dev)
    o = _out(out, (R, top_k), torch.int32, dev, "out")
    raw = None
    if out_raw_indices is not None or return_raw:
        raw = _out(out_raw_indices, (R, top_k), torch.int32, dev, "out_raw_indices")
    sp = _stream_ptr(stream, dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes(R, W, top_k, scores.dtype, True), dev, sp)
    args = (scores.data_ptr(), _DTYPE[scores.dtype], R, W, scores.stride(0) if R > 1 else W,
            lengths.data_ptr(), _ptr(row_starts), offsets.data_ptr(), top_k, o.data_ptr(),
            _ptr(raw), workspace.data_ptr(), workspace.numel(), sp)
    _call("vts_topk_transform_ragged", args, tie)
    return o, raw


def topk_transform_page1(scores: torch.Tensor, lengths: torch.Tensor, page_table: torch.Tensor,
                         cu_seqlens_q: torch.Tensor, top_k: int,
                         row_starts: torch.Tensor | None = None, out: torch.Tensor | None = None,
                         out_raw_indices: torch.Tensor | None = None, return_raw: bool = False,
                         workspace: torch.Tensor | None = None, stream=None,
                         tie_break: str | None = None, sort: bool = True):
    """Top-k over row windows with the page-size-1, per-request page-table
    transform (include/vts.h, vts_topk_transform_page1); with tie_break, in
    the deterministic mode."""
    tie = _tie_code(tie_break, sort)
    _check_scores(scores, "scores")
    R, W = scores.shape
    dev = scores.device
    lengths = _i32(lengths, "lengths", R, dev)
    if row_starts is not None:
        row_starts = _i32(row_starts, "row_starts", R, dev)
    pt = page_table
    if pt.dtype != torch.int32 or pt.dim() != 2 or pt.device != dev or pt.stride(1) != 1:
        raise ValueError("page_table must be a 2-D int32 tensor with contiguous rows")
    B = pt.shape[0]
    cu = _i32(cu_seqlens_q, "cu_seqlens_q", B + 1, dev)
    o = _out(out, (R, top_k), torch.int32, dev, "out")
    raw = None
    if out_raw_indices is not None or return_raw:
        raw = _out(out_raw_indices, (R, top_k), torch.int32, dev, "out_raw_indices")
    sp = _stream_ptr(stream, dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes(R, W, top_k, scores.dtype, True), dev, sp)
    args = (scores.data_ptr(), _DTYPE[scores.dtype], R, W, scores.stride(0) if R > 1 else W,
            lengths.data_ptr(), _ptr(row_starts), pt.data_ptr(), pt.stride(0), pt.shape[1],
            cu.data_ptr(), B, top_k, o.data_ptr(), _ptr(raw), workspace.data_ptr(),
            workspace.numel(), sp)
    _call("vts_topk_transform_page1", args, tie)
    return o, raw


def set_tuning(key: int, value: int) -> None:
    """Path switches of the calling thread (see vts_set_tuning in include/vts.h); results never change."""
    _check("vts_set_tuning", library().vts_set_tuning(key, value))


def workspace_stats(workspace: torch.Tensor, stream=None) -> list[int]:
    """[re-filtered workgroups, whole-row re-selections, rows with spilled
    candidates, rows ranked over the whole candidate list]; clears them."""
    out = (ctypes.c_uint32 * 4)()
    _check("vts_workspace_stats", library().vts_workspace_stats(
        workspace.data_ptr(), out, 4, _stream_ptr(stream, workspace.device)))
    return list(out)
