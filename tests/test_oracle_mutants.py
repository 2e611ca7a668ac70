"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies oracle/vts_oracle.c, plants one mistake with a textual edit (a
dropped term, a flipped sign, a swapped operand, an off-by-one, a wrong
constant), builds the copy into a temporary library, points the oracle module
at it and runs the pin battery.  At least one pin must fail for every mutant;
the unmodified oracle passes the same battery.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "vts_oracle.c")

MUTANTS = {
    "dropped_row_offset_t": ("- (int64_t)next_n + (int64_t)t + 1", "- (int64_t)next_n + 1"),
    "flipped_next_n_sign": ("- (int64_t)next_n + (int64_t)t + 1", "+ (int64_t)next_n + (int64_t)t + 1"),
    "missing_width_clamp": ("return n < width ? n : width;", "return n;"),
    "request_index_modulo": ("seq_lens[r / next_n]", "seq_lens[r % next_n]"),
    "ascending_sort": ("if (a->v > b->v) return -1;\n        if (a->v < b->v) return 1;",
                       "if (a->v < b->v) return -1;\n        if (a->v > b->v) return 1;"),
    "short_row_off_by_one": ("if (n <= k) {", "if (n < k) {"),
    "rank_not_column": ("oi[j] = (int32_t)buf[j].col;", "oi[j] = (int32_t)j;"),
    "f16_implicit_bit": ("(double)(m + 1024)", "(double)(m + 512)"),
    "f16_subnormal_scale": ("ldexp((double)m, -24)", "ldexp((double)m, -23)"),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "pad_value": ("0xFBFFu", "0xFC00u"),
    "page_div_mod_swapped": ("int64_t col = pt_start + idx / page_size;",
                             "int64_t col = pt_start + idx % page_size;"),
    "page_offset_dropped": ("res = page * page_size + idx % page_size;", "res = page * page_size;"),
    "page_start_ignores_ptrs": ("page_table_row_starts ? (int64_t)page_table_row_starts[r] : base[r]",
                                "base[r]"),
    "window_start_ignored": ("int64_t base = row_starts ? (int64_t)row_starts[r] : 0;",
                             "int64_t base = 0;"),
    "window_no_room_clamp": ("n = len < 0 ? 0 : (len > room ? room : len);",
                             "n = len < 0 ? 0 : len;"),
    "values_from_rank": ("copy_elem(J->x, J->dtype, row_off + buf[j].col, J->out_vals, r * k + j);",
                         "copy_elem(J->x, J->dtype, row_off + j, J->out_vals, r * k + j);"),
}


def _battery():
    pins.test_valid_len_hand_table()
    pins.test_varlen_rows_maps_rows_to_requests()
    pins.test_window_rows_clamp()
    for n in (3, 5, 7):
        pins.test_brute_force_tiny_rows(n)
    pins.test_brute_force_bf16_and_f16()
    pins.test_k1_is_argmax()
    pins.test_sorted_row_selects_its_end()
    pins.test_k_equals_n_minus_1_drops_the_argmin()
    pins.test_constant_and_all_neg_inf_rows()
    pins.test_signed_zero_is_a_tie()
    pins.test_denormals_and_infinities_rank_exactly()
    for dt in (oracle.F32, oracle.BF16, oracle.F16):
        pins.test_against_torch_topk(dt)
        pins.test_short_and_empty_rows(dt)
    for dt in (oracle.BF16, oracle.F16):
        pins.test_every_16bit_pattern_orders_like_numpy(dt)
    pins.test_window_base_offsets_the_selection()
    pins.test_transform_identity_page_table_page_size_1()
    pins.test_transform_page_size_64_inverse_permutation()
    pins.test_transform_out_of_table_page_is_minus_one()


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", str(src), "-o",
                    str(lib), "-lm"], check=True)
    return str(lib)


def test_unmodified_oracle_passes_battery(tmp_path):
    lib = _build(tmp_path, "orig", open(SRC).read())
    try:
        oracle.use_library(lib)
        _battery()
    finally:
        oracle.use_library(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    lib = _build(tmp_path, name, text.replace(old, new))
    caught = False
    try:
        oracle.use_library(lib)
        _battery()
    except (AssertionError, OverflowError, ValueError, IndexError):
        caught = True
    finally:
        oracle.use_library(None)
    assert caught, f"no pin failed for the planted mistake {name}"
    np.testing.assert_equal(oracle.valid_len(8, 2, 1, 4, 100), 2)  # default oracle restored
