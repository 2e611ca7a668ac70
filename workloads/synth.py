"""Seeded synthetic inputs for the five decode-step workloads, keyed by name.

This module only draws random numbers and lays them out; it holds none of the
selection arithmetic.  Both the HIP path and the CPU oracle take their inputs
from here and from nowhere else.

Every row is drawn from its own child generator (numpy PCG64 seeded from
``SeedSequence(seed).spawn(rows)``), so any subset of rows can be rebuilt on
its own and rows can be generated in parallel.  Shapes, laws and seeds:

  "small"          fp32 [4, 4096], iid N(0,1); seq_lens ~ U{1..4096};
                   top_k 512, next_n 1, compress_ratio 1, values returned.
  "dsv32"          fp32 [64, 163840]; seq_lens ~ U{100000..163840}; each row is
                   N(0,1) with 1 % of its columns (drawn without replacement)
                   raised by U(2,6) ("spikes"); top_k 2048.  The previous-step
                   row P is drawn by the same law; the current row is P shifted
                   right by one column plus N(0, 0.1) noise (column 0 fresh).
                   pre_idx = the previous step's top-2048 of P over its valid
                   prefix (seq_len - 1), largest first.
  "long"           fp32 [1024, 262144], the same spiky law and hint;
                   95 % of seq_lens ~ U{131072..262144}, 5 % ~ U{262145..524288}
                   (longer than the width, so clamped).
  "dsv4_mtp"       bf16 [512, 262144], next_n 2 (256 requests), compress_ratio 4,
                   seq_lens = floor(exp(U * ln(2^20 + 1))) in [1, 2^20] with at
                   least four requests forced to 1 (< next_n: empty rows);
                   top_k 1024; N(0,1) rounded to bf16 (nearest even).
  "page"           fp16 [256, 65536] with row stride 65600; lengths ~ U{1..65536},
                   at least 8 rows with length <= 2048; row_starts ~
                   U{0..65536 - length}; page_size 64; page table int32
                   [256, 1040] whose entries are disjoint random slices of one
                   random permutation of 256*1040 physical pages;
                   page_table_row_starts ~ U{0..15}; top_k 2048.  Columns outside
                   a row's window hold the largest finite fp16 ("poisoned").

Seeds: 20261200 + the workload's seed offset (small 1, dsv32 2, long 3,
dsv4_mtp 4, page 5); the previous-step rows of dsv32 and long use that seed
+ 50.  The pre_idx of dsv32 and long is built with numpy's
partition and sort of the previous-step row: it is workload input (a
previous step's answer), never an expected value, and the oracle does not read it.

Variant "relu" clips values at zero (about half the row becomes an exact tie
at 0).  `poison_outside` sets every column outside given row windows to the
largest finite value of the dtype (3e38 for fp32); the windows come from the
caller.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32, BF16, F16 = 0, 1, 2
BASE_SEED = 20261200

WORKLOADS = {
    "small": dict(seed_offset=1, kind="varlen", dtype=F32, rows=4, width=4096, k=512, next_n=1,
                  cr=1, values=True, law="normal"),
    "dsv32": dict(seed_offset=2, kind="varlen", dtype=F32, rows=64, width=163840, k=2048,
                  next_n=1, cr=1, values=False, law="spiky"),
    "long": dict(seed_offset=3, kind="varlen", dtype=F32, rows=1024, width=262144, k=2048,
                 next_n=1, cr=1, values=False, law="spiky"),
    "dsv4_mtp": dict(seed_offset=4, kind="varlen", dtype=BF16, rows=512, width=262144, k=1024,
                     next_n=2, cr=4, values=False, law="normal"),
    "page": dict(seed_offset=5, kind="transform", dtype=F16, rows=256, width=65536, stride=65600,
                 k=2048, page_size=64, pt_cols=1040, law="normal"),
}


@dataclasses.dataclass
class Workload:
    """One synthetic batch.  `x` holds raw element bits, shape [rows, row_stride]."""

    name: str
    kind: str  # "varlen" | "transform"
    dtype: int
    x: np.ndarray
    width: int
    k: int
    # topk_varlen
    seq_lens: np.ndarray | None = None
    next_n: int = 1
    compress_ratio: int = 1
    pre_idx: np.ndarray | None = None
    return_values: bool = False
    # page transform
    lengths: np.ndarray | None = None
    row_starts: np.ndarray | None = None
    page_table: np.ndarray | None = None
    page_table_row_starts: np.ndarray | None = None
    page_size: int = 1

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def row_stride(self) -> int:
        return self.x.shape[1]

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == F32 else 2


def to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def to_f16_bits(f: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(f, np.float32).astype(np.float16).view(np.uint16)


def _bits(f32: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(f32, np.float32).view(np.uint32)
    return to_bf16_bits(f32) if dtype == BF16 else to_f16_bits(f32)


MAX_FINITE_BITS = {F32: np.float32(3e38).view(np.uint32), BF16: np.uint16(0x7F7F),
                   F16: np.uint16(0x7BFF)}


def _spiky_row(g: np.random.Generator, W: int) -> np.ndarray:
    row = g.standard_normal(W, dtype=np.float32)
    m = int(round(0.01 * W))
    pos = g.choice(W, size=m, replace=False)
    row[pos] += g.uniform(2.0, 6.0, size=m).astype(np.float32)
    return row


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make(name: str, rows: int | None = None, seed: int | None = None, variant: str | None = None,
         width: int | None = None, hint: bool = True) -> Workload:
    """Builds the workload `name` (a key of WORKLOADS).  `rows`/`width` shrink it
    for quick cases."""
    c = dict(WORKLOADS[name])
    R = rows if rows is not None else c["rows"]
    W = width if width is not None else c["width"]
    S = c.get("stride", W) + (W - c["width"] if width is not None and "stride" in c else 0)
    S = max(S, W)
    seed = BASE_SEED + c["seed_offset"] if seed is None else seed
    g = np.random.default_rng(seed)
    k, dtype = c["k"], c["dtype"]
    wl = Workload(name=name, kind=c["kind"], dtype=dtype,
                  x=np.empty((R, S), np.uint32 if dtype == F32 else np.uint16), width=W, k=k)

    # ---- lengths --------------------------------------------------------------
    if c["kind"] == "varlen":
        nn, cr = c["next_n"], c["cr"]
        assert R % nn == 0
        nreq = R // nn
        wl.next_n, wl.compress_ratio, wl.return_values = nn, cr, c["values"]
        if name == "small":
            seq = g.integers(1, W + 1, size=nreq)
        elif name == "dsv32":
            lo = max(1, int(W * 100000 / 163840))
            seq = g.integers(lo, W + 1, size=nreq)
        elif name == "long":
            half = W // 2
            seq = g.integers(half, W + 1, size=nreq)
            longer = g.random(nreq) < 0.05
            seq[longer] = g.integers(W + 1, 2 * W + 1, size=int(longer.sum()))
        else:  # dsv4_mtp
            top = 4 * W  # 2^20 at the full width
            u = g.random(nreq)
            seq = np.floor(np.exp(u * math.log(top + 1))).astype(np.int64)
            seq = np.clip(seq, 1, top)
            forced = g.choice(nreq, size=min(4, nreq), replace=False)
            seq[forced] = 1
        wl.seq_lens = seq.astype(np.int32)
    else:
        lengths = g.integers(1, W + 1, size=R)
        short = g.choice(R, size=min(8, R), replace=False)
        lengths[short] = g.integers(1, min(2048, W) + 1, size=short.size)
        starts = np.array([g.integers(0, W - L + 1) for L in lengths], np.int64)
        wl.lengths = lengths.astype(np.int32)
        wl.row_starts = starts.astype(np.int32)
        wl.page_size = c["page_size"]
        P = c["pt_cols"] if width is None else -(-W // c["page_size"]) + 16
        perm = g.permutation(R * P).astype(np.int32)
        wl.page_table = perm.reshape(R, P)
        wl.page_table_row_starts = g.integers(0, 16, size=R).astype(np.int32)

    # ---- values, one child generator per row --------------------------------------
    children = np.random.SeedSequence(seed).spawn(R)
    prev_children = np.random.SeedSequence(seed + 50).spawn(R)
    spiky = c["law"] == "spiky"
    want_hint = spiky and hint
    pre_idx = np.full((R // wl.next_n, k), -1, np.int32) if want_hint else None
    if want_hint:
        # previous step: one token shorter (these workloads have next_n = compress_ratio = 1)
        assert wl.next_n == 1 and wl.compress_ratio == 1
        n_prev = np.clip(wl.seq_lens.astype(np.int64) - 1, 0, W)

    def fill(r: int):
        gr = np.random.default_rng(children[r])
        if spiky:
            gp = np.random.default_rng(prev_children[r])
            P_row = _spiky_row(gp, W)
            cur = np.empty(W, np.float32)
            cur[1:] = P_row[:-1] + np.float32(0.1) * gr.standard_normal(W - 1, dtype=np.float32)
            cur[0] = gr.standard_normal(dtype=np.float32)
            if want_hint:
                m = int(n_prev[r])
                if m > k:
                    part = np.argpartition(P_row[:m], m - k)[m - k:]
                    order = np.argsort(-P_row[part], kind="stable")
                    pre_idx[r] = part[order]
                else:
                    pre_idx[r, :m] = np.arange(m)
        else:
            cur = gr.standard_normal(W, dtype=np.float32)
        if variant == "relu":
            cur = np.maximum(cur, np.float32(0.0))
        wl.x[r, :W] = _bits(cur, dtype)
        if S > W:
            wl.x[r, W:] = MAX_FINITE_BITS[dtype]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(R)))
    wl.pre_idx = pre_idx

    # ---- poisoned columns outside each window ---------------------------------------
    if c["kind"] == "transform":
        # windows are [row_start, row_start + length), inside the width by construction
        poison_outside(wl, wl.row_starts.astype(np.int64), wl.lengths.astype(np.int64))
    return wl


def poison_outside(wl: Workload, base: np.ndarray, n: np.ndarray) -> None:
    """Sets every column outside [base[r], base[r] + n[r]) to the dtype's largest finite value.

    The windows come from the caller (the test takes them from the oracle).
    """
    S = wl.row_stride
    col = np.arange(S)[None, :]
    outside = (col < base[:, None]) | (col >= (base + n)[:, None])
    wl.x[outside] = MAX_FINITE_BITS[wl.dtype]
