"""Pins for the oracle's byte accounting and tail-waste identities (CPU only).

Values come from ``tests/golden/kv_bytes.json`` and ``tail_waste.json``,
which record what the pages print; the identities of the auturnal.com
review's equations (2) and (3) are checked exactly with rationals, with the
mean computed by enumeration rather than from the closed form.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def test_bytes_per_token_example():
    g = _golden("kv_bytes.json")
    ex = g["example"]
    per_tok = accounting.kv_bytes_per_token(ex["num_layers"], ex["num_kv_heads"], ex["head_dim"],
                                            ex["elem_bytes"])
    assert per_tok == g["bytes_per_token"] == 128 * 1024
    assert accounting.kv_bytes([g["request_tokens"]], ex["num_layers"], ex["num_kv_heads"],
                               ex["head_dim"], ex["elem_bytes"]) == g["request_bytes"]
    assert g["request_bytes"] == 2 ** 29  # 0.5 GiB
    many = accounting.kv_bytes([g["request_tokens"]] * g["concurrent_requests"], ex["num_layers"],
                               ex["num_kv_heads"], ex["head_dim"], ex["elem_bytes"])
    assert many == g["concurrent_bytes"]
    mha = accounting.kv_bytes([g["request_tokens"]], ex["num_layers"], g["mha_kv_heads"],
                              ex["head_dim"], ex["elem_bytes"])
    assert mha == g["request_bytes_mha"] == 2 * 2 ** 30


def test_gqa_and_mqa_ratios():
    r = _golden("kv_bytes.json")["head_ratio"]
    base = accounting.kv_bytes_per_token(1, r["mha_heads"], 128, 2)
    assert Fraction(accounting.kv_bytes_per_token(1, r["gqa_heads"], 128, 2), base) == Fraction(1, 4)
    assert float(Fraction(1, 4)) == r["gqa_fraction"]
    mqa = Fraction(accounting.kv_bytes_per_token(1, r["mqa_heads"], 128, 2), base)
    assert mqa == Fraction(1, 32) and round(float(mqa), 2) == r["mqa_fraction_approx"]


def test_review_record_bytes_per_token():
    rec = _golden("review_record.json")
    assert accounting.kv_bytes_per_token(32, 8, 128, 2) == rec["bytes_per_token"]


@pytest.mark.parametrize("block_size", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_mean_tail_waste_is_b_minus_1_over_2_when_b_divides_512(block_size):
    g = _golden("tail_waste.json")
    got = accounting.mean_tail_waste_uniform(block_size, g["uniform_max_len"])
    assert got == Fraction(block_size - 1, 2)


@pytest.mark.parametrize("block_size,want", [(16, Fraction(15, 2)), (32, Fraction(31, 2))])
def test_mean_tail_waste_at_4096(block_size, want):
    assert accounting.mean_tail_waste_uniform(block_size, 4096) == want


def test_mean_tail_waste_differs_when_b_does_not_divide():
    # equation (3) needs the maximum length to be a multiple of B
    assert accounting.mean_tail_waste_uniform(3, 10) != Fraction(1, 1)


def test_reservation_comparison():
    g = _golden("tail_waste.json")
    r = g["reservation"]
    assert accounting.mean_reservation_waste_uniform(r["reserved"], r["max_len"]) == Fraction(511, 2)
    assert float(Fraction(511, 2)) == r["mean_waste"]
    ex = g["reservation_example"]
    assert accounting.reservation_waste(ex["reserved"], ex["used"]) == ex["wasted"]


def test_tail_waste_bound_and_allocation_brute_force():
    rng = np.random.default_rng(4)
    for B in (1, 5, 16, 32):
        lens = rng.integers(1, 4097, size=200)
        w = accounting.tail_waste(lens, B)
        assert 0 <= w <= accounting.tail_waste_bound(len(lens), B)
        allocated_slots = 0
        for t in lens:  # allocate one page at a time as tokens arrive
            pages, filled = 0, 0
            for _ in range(int(t)):
                if filled == pages * B:
                    pages += 1
                filled += 1
            allocated_slots += pages * B
        assert allocated_slots - int(lens.sum()) == w


def test_tiny_config_tables_waste():
    # four sequences of 1, 17, 40 and 100 tokens at B = 16: 1+2+3+7 = 13 pages
    lens = [1, 17, 40, 100]
    assert sum(accounting.blocks_needed(t, 16) for t in lens) == 13
    assert accounting.tail_waste(lens, 16) == 13 * 16 - 158 == 50


def test_printed_request_examples():
    # request A: 40 tokens in 3 pages (8 used in the last); request B: 20 in 2
    assert accounting.blocks_needed(40, 16) == 3 and accounting.tail_waste([40], 16) == 8
    assert accounting.blocks_needed(20, 16) == 2 and accounting.tail_waste([20], 16) == 12
