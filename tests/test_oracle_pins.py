"""Pins of the CPU oracle against things other than itself (no GPU needed).

- the valid-length rule against a hand-worked table (tests/golden/valid_len_table.txt);
- selection against brute force over every k-subset of tiny rows;
- textbook special cases: k = 1 is the argmax, a sorted row selects its end,
  a constant row selects k copies, an all -inf row still selects k valid columns;
- torch.topk on the CPU as an independent library routine (value multisets);
- the oracle's bf16/fp16 decoding against numpy's, over every bit pattern;
- short rows, value padding and the page-table transform identities.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import BF16, F16, F32, PAD_BITS
from oracle.check import check_rows, check_transform, decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# valid length
# --------------------------------------------------------------------------

def _table():
    rows = []
    with open(os.path.join(GOLDEN, "valid_len_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def test_valid_len_hand_table():
    rows = _table()
    assert len(rows) >= 30
    for seq, nn, cr, w, t, want in rows:
        assert oracle.valid_len(seq, nn, t, cr, w) == want, (seq, nn, cr, w, t)


def test_varlen_rows_maps_rows_to_requests():
    # request i owns rows i*next_n .. i*next_n + next_n - 1, row t = r % next_n
    seq = np.array([8, 5, 1, 12], np.int32)
    base, n = oracle.varlen_rows(seq, 8, 2, 4, 4096)
    assert base.tolist() == [0] * 8
    assert n.tolist() == [1, 2, 1, 1, 0, 0, 2, 3]


def test_window_rows_clamp():
    L = np.array([10, 10, -3, 100, 5, 7], np.int32)
    rs = np.array([0, 95, 3, 0, 101, -1], np.int32)
    base, n = oracle.window_rows(L, rs, 100)
    assert n.tolist() == [10, 5, 0, 100, 0, 0]
    assert base.tolist() == [0, 95, 3, 0, 0, 0]
    base, n = oracle.window_rows(L, None, 100)
    assert n.tolist() == [10, 10, 0, 100, 5, 7] and base.tolist() == [0] * 6


# --------------------------------------------------------------------------
# selection: brute force on tiny rows
# --------------------------------------------------------------------------

_SMALL_VALUES = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, 1e-45, -1e-45, 3.5],
                         np.float32)


def _valid_subsets(vals, k):
    n = len(vals)
    out = []
    for S in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in S]
        if not rest or min(vals[j] for j in S) >= max(vals[j] for j in rest):
            out.append(S)
    return out


def _norm_sorted(v):
    v = np.asarray(v, np.float64)
    return np.sort(np.where(v == 0, 0.0, v))


@pytest.mark.parametrize("n", [2, 3, 5, 7, 9])
def test_brute_force_tiny_rows(n):
    rng = np.random.default_rng(1000 + n)
    for trial in range(40):
        row = rng.choice(_SMALL_VALUES, size=n)
        x = row[None, :].astype(np.float32)
        for k in range(1, n):
            idx, vals = oracle.select(x, F32, np.array([0]), np.array([n]), k, True)
            S = tuple(sorted(idx[0].tolist()))
            valid = _valid_subsets(row.astype(np.float64), k)
            assert S in valid, (row, k, idx)
            ref = _norm_sorted(row[list(S)])
            for V in valid:
                assert np.array_equal(_norm_sorted(row[list(V)]), ref)
            # values are bit copies, in the order of the indices
            assert np.array_equal(vals[0], x[0].view(np.uint32)[idx[0]])
            # oracle order: descending value, then ascending column
            sel = row[idx[0]].astype(np.float64)
            assert np.all(sel[:-1] >= sel[1:])


# NaN bit patterns of both signs (quiet, with a payload, signalling)
_NAN_BITS = np.array([0x7FC00000, 0x7FC00001, 0x7F800001, 0xFFC00000, 0xFFFFFFFF], np.uint32)


def _rank(bits32):
    """The order the oracle documents for fp32 bits: (NaN class, value) with
    a NaN whose sign bit is clear above +inf and one whose sign bit is set
    below -inf (NaNs of one sign tie), numbers by value, -0 == +0."""
    with np.errstate(invalid="ignore"):
        v = bits32.view(np.float32).astype(np.float64)
    nan = np.isnan(v)
    cls = np.where(nan, np.where(bits32 >> 31 == 1, -1, 1), 0)
    return [(int(c), 0.0 if m else float(x) + 0.0) for c, m, x in zip(cls, nan, v)]


def _valid_subsets_ranked(rank, k):
    n = len(rank)
    out = []
    for S in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in S]
        if not rest or min(rank[j] for j in S) >= max(rank[j] for j in rest):
            out.append(S)
    return out


@pytest.mark.parametrize("n", [3, 5, 8])
def test_brute_force_rows_with_nan(n):
    """NaN order (reading: a sign-clear NaN above +inf, a sign-set one below
    -inf, ties within a sign): the oracle's selection is a valid top-k subset
    under that order, and every valid subset has the same count of NaNs of
    each sign and the same multiset of the other values."""
    rng = np.random.default_rng(300 + n)
    pool = np.concatenate([_SMALL_VALUES.view(np.uint32), _NAN_BITS])
    for trial in range(40):
        bits = rng.choice(pool, size=n).astype(np.uint32)
        rank = _rank(bits)
        for k in range(1, n):
            idx, _ = oracle.select(bits[None, :], F32, np.array([0]), np.array([n]), k)
            S = tuple(sorted(idx[0].tolist()))
            valid = _valid_subsets_ranked(rank, k)
            assert S in valid, (bits, k, idx)
            ref = sorted(rank[j] for j in S)
            for V in valid:
                assert sorted(rank[j] for j in V) == ref
            # listed in descending order of the documented rank
            got = [rank[j] for j in idx[0]]
            assert all(a >= b for a, b in zip(got, got[1:]))


def test_nan_sign_classes_by_hand():
    # +NaN (payloads 0 and 1) above +inf, -NaN below -inf; ties by column
    bits = np.array([0x3F800000, 0xFFC00000, 0x7F800000, 0x7FC00001, 0xFF800000, 0x7FC00000],
                    np.uint32)  # 1, -NaN, +inf, +NaN, -inf, +NaN
    idx, _ = oracle.select(bits[None, :], F32, np.array([0]), np.array([6]), 5)
    assert idx[0].tolist() == [3, 5, 2, 0, 4]


def test_brute_force_bf16_and_f16():
    rng = np.random.default_rng(7)
    for dtype, npdt in ((BF16, None), (F16, np.float16)):
        for trial in range(30):
            n = int(rng.integers(3, 9))
            # small integers (exact in both formats) force ties
            vals = rng.integers(-3, 4, size=n).astype(np.float32)
            if dtype == F16:
                bits = vals.astype(np.float16).view(np.uint16)
            else:
                bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
            x = bits[None, :]
            for k in range(1, n):
                idx, _ = oracle.select(x, dtype, np.array([0]), np.array([n]), k)
                S = tuple(sorted(idx[0].tolist()))
                assert S in _valid_subsets(vals.astype(np.float64), k)


# --------------------------------------------------------------------------
# textbook special cases
# --------------------------------------------------------------------------

def test_k1_is_argmax():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 1000)).astype(np.float32)
    idx, _ = oracle.select(x, F32, np.zeros(16), np.full(16, 1000), 1)
    assert np.array_equal(idx[:, 0], np.argmax(x, axis=1))


def test_sorted_row_selects_its_end():
    x = np.arange(500, dtype=np.float32)[None, :]
    idx, _ = oracle.select(x, F32, np.array([0]), np.array([500]), 37)
    assert idx[0].tolist() == list(range(499, 499 - 37, -1))
    xd = x[:, ::-1].copy()
    idx, _ = oracle.select(xd, F32, np.array([0]), np.array([500]), 37)
    assert idx[0].tolist() == list(range(37))


def test_k_equals_n_minus_1_drops_the_argmin():
    rng = np.random.default_rng(5)
    x = rng.permutation(200).astype(np.float32)[None, :]
    idx, _ = oracle.select(x, F32, np.array([0]), np.array([200]), 199)
    missing = set(range(200)) - set(idx[0].tolist())
    assert missing == {int(np.argmin(x[0]))}


def test_constant_and_all_neg_inf_rows():
    x = np.full((2, 300), 1.25, np.float32)
    x[1] = -np.inf
    idx, vals = oracle.select(x, F32, np.zeros(2), np.full(2, 300), 64, True)
    for r in range(2):
        assert np.unique(idx[r]).size == 64 and idx[r].min() >= 0 and idx[r].max() < 300
        assert np.all(vals[r] == x[r].view(np.uint32)[0])


def test_signed_zero_is_a_tie():
    # four +0/-0 entries compete for two slots behind one positive value
    x = np.array([[-0.0, 0.0, 1.0, -0.0, 0.0, -1.0]], np.float32)
    idx, _ = oracle.select(x, F32, np.array([0]), np.array([6]), 3)
    assert idx[0].tolist() == [2, 0, 1]  # ties by ascending column


def test_denormals_and_infinities_rank_exactly():
    x = np.array([[1e-45, -1e-45, 0.0, np.inf, -np.inf, 1e-38, 3e38]], np.float32)
    idx, _ = oracle.select(x, F32, np.array([0]), np.array([7]), 6)
    assert idx[0].tolist() == [3, 6, 5, 0, 2, 1]


# --------------------------------------------------------------------------
# independent library cross-check: torch.topk on the CPU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_against_torch_topk(dtype):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(20 + dtype)
    R, W, k = 12, 3000, 256
    xf = rng.standard_normal((R, W)).astype(np.float32)
    if dtype == F32:
        t = torch.from_numpy(xf)
        bits = xf.view(np.uint32)
    elif dtype == BF16:
        t = torch.from_numpy(xf).to(torch.bfloat16)
        bits = t.view(torch.int16).numpy().view(np.uint16)
    else:
        t = torch.from_numpy(xf).to(torch.float16)
        bits = t.view(torch.int16).numpy().view(np.uint16)
    n = rng.integers(k + 1, W + 1, size=R)
    idx, _ = oracle.select(bits, dtype, np.zeros(R), n, k)
    for r in range(R):
        ref = torch.topk(t[r, : n[r]].float(), k).values.double().numpy()
        got = decode(bits[r], dtype)[idx[r]]
        assert np.array_equal(_norm_sorted(got), _norm_sorted(ref))


# --------------------------------------------------------------------------
# decoding of every 16-bit pattern, against numpy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [BF16, F16])
def test_every_16bit_pattern_orders_like_numpy(dtype):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = decode(allbits, dtype)
    finite_or_inf = allbits[~np.isnan(v)]
    rng = np.random.default_rng(3)
    row = rng.permutation(finite_or_inf)[None, :]
    n = row.shape[1]
    k = n - 1  # forces a full ordering of all but one element
    idx, vals = oracle.select(row, dtype, np.array([0]), np.array([n]), k, True)
    got = decode(vals[0], dtype)
    ref = np.sort(decode(row[0], dtype))[::-1][:k]
    assert np.array_equal(np.where(got == 0, 0.0, got), np.where(ref == 0, 0.0, ref))
    assert np.all(got[:-1] >= got[1:])


# --------------------------------------------------------------------------
# short rows and padding
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [F32, BF16, F16])
def test_short_and_empty_rows(dtype):
    k = 16
    R, W = 4, 40
    item = np.uint32 if dtype == F32 else np.uint16
    x = np.arange(R * W, dtype=item).reshape(R, W)
    n = np.array([0, 1, 15, 16])
    idx, vals = oracle.select(x, dtype, np.zeros(R), n, k, True)
    for r in range(R):
        m = int(n[r])
        assert idx[r].tolist() == list(range(m)) + [-1] * (k - m)
        assert np.array_equal(vals[r, :m], x[r, :m])
        assert np.all(vals[r, m:] == PAD_BITS[dtype])


def test_window_base_offsets_the_selection():
    x = np.zeros((1, 50), np.float32)
    x[0, 30] = 9.0  # inside the window at local column 10
    x[0, 5] = 99.0  # outside the window
    idx, _ = oracle.select(x, F32, np.array([20]), np.array([25]), 1)
    assert idx[0, 0] == 10


# --------------------------------------------------------------------------
# page-table transform identities
# --------------------------------------------------------------------------

def test_transform_identity_page_table_page_size_1():
    rng = np.random.default_rng(9)
    R, W, k = 5, 500, 32
    x = rng.standard_normal((R, W)).astype(np.float32)
    L = rng.integers(0, W + 1, size=R).astype(np.int32)
    pt = np.tile(np.arange(W, dtype=np.int32), (R, 1))
    out, raw, base, n = oracle.topk_page_table_transform(x, F32, L, None, pt, None, 1, k)
    assert np.array_equal(out, raw)


def test_transform_page_size_64_inverse_permutation():
    rng = np.random.default_rng(10)
    R, W, k, ps, P = 6, 4096, 64, 64, 80
    x = rng.standard_normal((R, W)).astype(np.float32)
    L = rng.integers(1, 2000, size=R).astype(np.int32)
    rs = rng.integers(0, W - 2000, size=R).astype(np.int32)
    ptrs = rng.integers(0, 10, size=R).astype(np.int32)
    perm = rng.permutation(R * P).astype(np.int32).reshape(R, P)
    out, raw, base, n = oracle.topk_page_table_transform(x, F32, L, rs, perm, ptrs, ps, k)
    inv = np.argsort(perm.reshape(-1))
    for r in range(R):
        m = min(int(n[r]), k)
        assert np.all(out[r, m:] == -1) and np.all(raw[r, m:] == -1)
        page_pos = inv[out[r, :m] // ps]  # flat position r*P + col in the table
        assert np.all(page_pos // P == r)
        col = page_pos % P
        assert np.array_equal(col * ps + out[r, :m] % ps, ptrs[r] * ps + raw[r, :m])


def test_transform_out_of_table_page_is_minus_one():
    raw = np.array([[0, 63, 64, 200]], np.int32)
    pt = np.array([[5, 7, 9]], np.int32)
    out = oracle.page_translate(raw, pt, np.array([0], np.int32), np.array([0]), 64)
    assert out[0].tolist() == [5 * 64, 5 * 64 + 63, 7 * 64, -1]


def test_ragged_transform_hand_worked():
    # row 0: the three largest of [1, 5, 3, 9, 7] are columns 3, 4, 1 (9, 7, 5);
    # row 1: window of 2 columns <= k, so the identity then -1 (short-row rule)
    x = np.array([[1, 5, 3, 9, 7], [4, 2, 8, 6, 0]], np.float32)
    L = np.array([5, 2], np.int32)
    off = np.array([100, 7], np.int32)
    out, raw, base, n = oracle.topk_transform_ragged(x, F32, L, None, off, 3)
    assert raw.tolist() == [[3, 4, 1], [0, 1, -1]]
    assert out.tolist() == [[103, 104, 101], [7, 8, -1]]


def test_ragged_transform_identities():
    rng = np.random.default_rng(12)
    R, W, k = 7, 3000, 64
    x = rng.standard_normal((R, W)).astype(np.float32)
    L = rng.integers(0, 1500, size=R).astype(np.int32)
    rs = rng.integers(0, W - 1500, size=R).astype(np.int32)
    zero = np.zeros(R, np.int32)
    out0, raw0, _, _ = oracle.topk_transform_ragged(x, F32, L, rs, zero, k)
    assert np.array_equal(out0, raw0)  # offset 0: the raw indices
    off = rng.integers(0, 1 << 30, size=R).astype(np.int32)
    out, raw, base, n = oracle.topk_transform_ragged(x, F32, L, rs, off, k)
    assert np.array_equal(raw, raw0)  # the selection ignores the offsets
    sel = raw >= 0
    assert np.array_equal((out - off[:, None])[sel], raw[sel])
    assert np.all(out[~sel] == -1)
    # the selection is the page transform's (same windows): identity table, page 1
    pt = np.tile(np.arange(W, dtype=np.int32), (R, 1))
    pout, praw, _, _ = oracle.topk_page_table_transform(x, F32, L, rs, pt, rs, 1, k)
    assert np.array_equal(praw, raw)


def test_row_requests_brute_force():
    # cu = [2, 2, 5, 6]: rows 0-1 and 6+ are outside, request 0 is empty,
    # rows 2-4 belong to request 1, row 5 to request 2
    cu = np.array([2, 2, 5, 6], np.int32)
    assert oracle.row_requests(cu, 8).tolist() == [-1, -1, 1, 1, 1, 2, -1, -1]
    rng = np.random.default_rng(13)
    cu = np.concatenate([[0], np.cumsum(rng.integers(0, 4, size=50))]).astype(np.int32)
    R = int(cu[-1]) + 3
    got = oracle.row_requests(cu, R)
    for r in range(R):
        want = [b for b in range(len(cu) - 1) if cu[b] <= r < cu[b + 1]]
        assert got[r] == (want[0] if want else -1)


def test_page1_transform_hand_worked():
    # two requests: rows 0-1 -> request 0, row 2 -> request 1
    x = np.array([[1, 5, 3, 9, 7], [4, 2, 8, 6, 0], [0, 1, 2, 3, 4]], np.float32)
    L = np.array([5, 5, 2], np.int32)
    pt = np.array([[10, 11, 12, 13, 14], [20, 21, 22, 23, 24]], np.int32)
    cu = np.array([0, 2, 3], np.int32)
    out, raw, base, n = oracle.topk_transform_page1(x, F32, L, None, pt, cu, 3)
    assert raw.tolist() == [[3, 4, 1], [2, 3, 0], [0, 1, -1]]
    assert out.tolist() == [[13, 14, 11], [12, 13, 10], [20, 21, -1]]


def test_page1_transform_identity_and_permutation():
    rng = np.random.default_rng(14)
    B, W, k = 6, 2000, 40
    cu = np.concatenate([[0], np.cumsum(rng.integers(1, 4, size=B))]).astype(np.int32)
    R = int(cu[-1])
    x = rng.standard_normal((R, W)).astype(np.float32)
    L = rng.integers(0, W, size=R).astype(np.int32)
    ident = np.tile(np.arange(W, dtype=np.int32), (B, 1))
    out, raw, _, _ = oracle.topk_transform_page1(x, F32, L, None, ident, cu, k)
    assert np.array_equal(out, raw)  # identity table: the raw indices
    perm = np.stack([rng.permutation(W) for _ in range(B)]).astype(np.int32)
    out, raw2, _, _ = oracle.topk_transform_page1(x, F32, L, None, perm, cu, k)
    assert np.array_equal(raw2, raw)
    b = oracle.row_requests(cu, R)
    inv = np.argsort(perm, axis=1)
    sel = raw >= 0
    rows = np.nonzero(sel)[0]
    assert np.array_equal(inv[b[rows], out[sel]], raw[sel])  # the table is undone per request
    assert np.all(out[~sel] == -1)


def test_ragged_transform_overflow_is_flagged():
    with pytest.raises(OverflowError):
        oracle.ragged_translate(np.array([[5]], np.int32), np.array([2 ** 31 - 3], np.int64))


# --------------------------------------------------------------------------
# the checker rejects wrong answers and accepts tie-equivalent ones
# --------------------------------------------------------------------------

def _case():
    rng = np.random.default_rng(42)
    R, W, k = 3, 400, 20
    x = rng.integers(-5, 6, size=(R, W)).astype(np.float32)  # heavy ties
    n = np.array([400, 10, 250])
    idx, vals = oracle.select(x, F32, np.zeros(R), n, k, True)
    return x, n, k, idx, vals


def test_checker_accepts_oracle_and_tie_swaps():
    x, n, k, idx, vals = _case()
    base = np.zeros(3, np.int64)
    assert check_rows(x, F32, base, n, k, idx, idx, vals) == []
    # swap one tied element for another unselected element of equal value
    g = idx.copy()
    r = 0
    kth = x[r, g[r]].min()
    tied_out = [j for j in range(n[r]) if x[r, j] == kth and j not in g[r]]
    pos = int(np.where(x[r, g[r]] == kth)[0][0])
    g[r, pos] = tied_out[0]
    gv = vals.copy()
    gv[r, pos] = x[r].view(np.uint32)[tied_out[0]]
    # slot order is free for rows with n > k
    g[0], gv[0] = g[0, ::-1].copy(), gv[0, ::-1].copy()
    assert check_rows(x, F32, base, n, k, g, idx, gv) == []


@pytest.mark.parametrize("mistake", ["dup", "range", "suffix", "swap", "values", "pad", "short_order"])
def test_checker_rejects(mistake):
    x, n, k, idx, vals = _case()
    base = np.zeros(3, np.int64)
    g, gv = idx.copy(), vals.copy()
    if mistake == "dup":
        g[0, 1] = g[0, 0]
    elif mistake == "range":
        g[2, 3] = 300  # >= n for row 2
    elif mistake == "suffix":
        g[1, 15] = 3
    elif mistake == "swap":
        lo = int(np.argmin(x[0, :400]))
        g[0, 0] = lo
        gv[0, 0] = x[0].view(np.uint32)[lo]
    elif mistake == "values":
        gv[2, 4] ^= 1
    elif mistake == "pad":
        gv[1, 12] = 0
    elif mistake == "short_order":
        g[1, [0, 1]] = g[1, [1, 0]]
        gv[1, [0, 1]] = gv[1, [1, 0]]
    assert check_rows(x, F32, base, n, k, g, idx, gv) != []


def test_checker_on_nan_rows():
    """Rows holding NaN: a NaN of one sign may stand for another NaN of that
    sign (and its payload may differ), but trading a sign-clear NaN for a
    sign-set one, or for +inf, is a different selection."""
    bits = np.array([[0x7FC00000, 0x3F800000, 0xFFC00000, 0x7F800000, 0x7FC00001, 0xFF800000,
                      0x40000000, 0xFFC00001]], np.uint32)  # +NaN 1 -NaN +inf +NaN' -inf 2 -NaN'
    n, k, base = np.array([8]), 3, np.zeros(1, np.int64)
    idx, _ = oracle.select(bits, F32, base, n, k)
    assert sorted(idx[0].tolist()) == [0, 3, 4]  # both sign-clear NaNs, then +inf
    assert check_rows(bits, F32, base, n, k, idx, idx) == []
    assert check_rows(bits, F32, base, n, k, np.array([[4, 3, 0]]), idx) == []  # order free
    for bad in ([0, 3, 2], [0, 3, 6], [0, 4, 6]):  # -NaN, 2 in place of a +NaN / +inf
        assert check_rows(bits, F32, base, n, k, np.array([bad]), idx) != [], bad
    # the lowest ones: -inf ranks above both sign-set NaNs
    idx7, _ = oracle.select(bits, F32, base, n, 7)
    assert sorted(set(range(8)) - set(idx7[0].tolist())) in ([2], [7])
    assert check_rows(bits, F32, base, n, 7, np.array([[0, 1, 3, 4, 5, 6, 7]]), idx7) == []
    assert check_rows(bits, F32, base, n, 7, np.array([[0, 1, 3, 4, 2, 6, 7]]), idx7) != []


def test_transform_checker_rejects_bad_translation():
    rng = np.random.default_rng(12)
    R, W, k, ps, P = 2, 1000, 16, 64, 20
    x = rng.standard_normal((R, W)).astype(np.float32)
    L = np.array([900, 10], np.int32)
    pt = rng.permutation(R * P).astype(np.int32).reshape(R, P)
    ptrs = np.array([2, 3], np.int32)
    out, raw, base, n = oracle.topk_page_table_transform(x, F32, L, None, pt, ptrs, ps, k)
    assert check_transform(x, F32, base, n, k, out, raw, raw, pt, ptrs, ps) == []
    bad = out.copy()
    bad[0, 3] += 1
    assert check_transform(x, F32, base, n, k, bad, raw, raw, pt, ptrs, ps) != []


# ---------------------------------------------------------------------------
# deterministic mode: canonical order and the SMALL / LARGE tie-break
# ---------------------------------------------------------------------------

def _ordered_cases():
    for line in open(os.path.join(GOLDEN, "ordered_ties.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        head, vals, want = (part.split() for part in line.split("|"))
        yield head[0], int(head[1]), [float(v) for v in vals], [int(w) for w in want]


@pytest.mark.parametrize("case", list(_ordered_cases()), ids=lambda c: f"{c[0]}-k{c[1]}-{len(c[2])}")
def test_ordered_hand_table(case):
    tie, k, vals, want = case
    x = np.array([vals], np.float32).view(np.uint32)
    idx, v, _ = oracle.topk_varlen_ordered(x, F32, np.array([len(vals)], np.int32), k, tie,
                                           return_values=True)
    assert idx[0].tolist() == want
    sel = [j for j in want if j >= 0]
    assert v[0][:len(sel)].tolist() == x[0][sel].tolist()  # bit copies (signs of zeros kept)


@pytest.mark.parametrize("tie", ["small", "large"])
def test_ordered_brute_force_subsets(tie):
    """Every k-subset of tiny rows with many ties: the valid top-k subsets are
    those whose smallest value is >= every value left out; "small" is the one
    with the least column sum, "large" the greatest (they differ only in which
    tied columns they hold).  The output lists it by value descending, then
    column ascending."""
    rng = np.random.default_rng(5 if tie == "small" else 6)
    # small integers, both signed zeros and NaNs of both signs: ties everywhere
    pool = np.concatenate([np.array([-2.0, -1.0, -0.0, 0.0, 0.0, 1.0, 2.0, -0.0],
                                    np.float32).view(np.uint32), _NAN_BITS[[0, 1, 3]]])
    for _ in range(300):
        n = int(rng.integers(1, 8))
        k = int(rng.integers(1, 8))
        bits = rng.choice(pool, size=n).astype(np.uint32)
        rank = _rank(bits)
        x = bits[None, :]
        idx, v, _ = oracle.topk_varlen_ordered(x, F32, np.array([n], np.int32), k, tie,
                                               return_values=True)
        m = min(n, k)
        best = None
        for sub in _valid_subsets_ranked(rank, m):
            key = sum(sub) if tie == "small" else -sum(sub)
            if best is None or key < best[0]:
                best = (key, sub)
        chosen = sorted(best[1])
        got = [j for j in idx[0].tolist() if j >= 0]
        assert sorted(got) == chosen, (bits, k, got, chosen)
        assert idx[0].tolist()[m:] == [-1] * (k - m)
        for a, b in zip(got, got[1:]):
            assert rank[a] > rank[b] or (rank[a] == rank[b] and a < b), (bits, got)
        assert np.array_equal(v[0][:m], bits[got])  # values: the elements' own bits
