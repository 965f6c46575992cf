"""Pins for the oracle's attention (CPU only).

The oracle's plain definition is checked against PyTorch's float64
``scaled_dot_product_attention`` (a library routine that reduces to the
textbook formula), against closed forms, and against the special cases the
pages call out (extreme logits).  The block recurrence and the split-KV merge
are checked against the plain definition at many block and partition sizes,
in the spirit of the float64 comparison recorded by the auturnal.com review
(``tests/golden/review_record.json``).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, formats, paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, keys, values, scale):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None, :], torch.from_numpy(keys)[None, None],
        torch.from_numpy(values)[None, None], scale=scale)
    return out[0, 0, 0].numpy()


@pytest.mark.parametrize("n,d", [(1, 4), (2, 8), (17, 64), (100, 128), (513, 32)])
def test_dense_matches_library_sdpa_float64(n, d):
    rng = np.random.default_rng(n * 1000 + d)
    q, keys, values = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    scale = 1.0 / math.sqrt(d)
    np.testing.assert_allclose(attention.dense_attention(q, keys, values, scale),
                               _sdpa(q, keys, values, scale), rtol=0, atol=1e-13)


def test_dense_scale_is_applied():
    rng = np.random.default_rng(5)
    q, keys, values = rng.standard_normal(16), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    a = attention.dense_attention(q, keys, values, 0.25)
    b = attention.dense_attention(q, keys, values, 1.0)
    np.testing.assert_allclose(a, _sdpa(q, keys, values, 0.25), atol=1e-13)
    assert np.abs(a - b).max() > 1e-3


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 32))
    out = attention.dense_attention(rng.standard_normal(32), rng.standard_normal((1, 32)), v, 0.3)
    assert np.array_equal(out, v[0])


def test_zero_query_averages_values():
    rng = np.random.default_rng(8)
    values = rng.standard_normal((37, 16))
    out = attention.dense_attention(np.zeros(16), rng.standard_normal((37, 16)), values, 0.5)
    np.testing.assert_allclose(out, values.mean(axis=0), rtol=0, atol=1e-15)


def test_two_tokens_closed_form():
    rng = np.random.default_rng(9)
    q, keys, values = rng.standard_normal(8), rng.standard_normal((2, 8)), rng.standard_normal((2, 8))
    scale = 0.7
    s0, s1 = scale * keys[0] @ q, scale * keys[1] @ q
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    want = w0 * values[0] + (1.0 - w0) * values[1]
    np.testing.assert_allclose(attention.dense_attention(q, keys, values, scale), want, atol=1e-15)


def test_dominant_logit_returns_that_value():
    """A score ahead of every other by more than 40 selects its value row."""
    rng = np.random.default_rng(10)
    d, n, j = 16, 50, 31
    keys = rng.standard_normal((n, d)) * 0.1
    values = rng.standard_normal((n, d))
    q = np.zeros(d)
    q[0] = 1.0
    keys[:, 0] = 0.0
    keys[j, 0] = 45.0  # score margin 45 at scale 1
    out = attention.dense_attention(q, keys, values, 1.0)
    np.testing.assert_allclose(out, values[j], rtol=0, atol=1e-15)


@pytest.mark.parametrize("magnitude", [80.0, 1000.0])
def test_extreme_logits_stay_finite_and_correct(magnitude):
    rng = np.random.default_rng(12)
    d, n = 32, 200
    q, keys, values = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    scores = keys @ q
    scale = magnitude / np.abs(scores).max()
    out = attention.dense_attention(q, keys, values, scale)
    assert np.all(np.isfinite(out))
    ref = _sdpa(q, keys, values, scale)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    online = attention.online_softmax_attention(q, keys, values, scale, 16)
    np.testing.assert_allclose(online, out, atol=1e-12)
    split = attention.split_kv_attention(q, keys, values, scale, 16, 64)
    np.testing.assert_allclose(split, out, atol=1e-12)


def test_row_permutation_invariance():
    rng = np.random.default_rng(13)
    q, keys, values = rng.standard_normal(24), rng.standard_normal((77, 24)), rng.standard_normal((77, 24))
    perm = rng.permutation(77)
    a = attention.dense_attention(q, keys, values, 0.2)
    b = attention.dense_attention(q, keys[perm], values[perm], 0.2)
    np.testing.assert_allclose(a, b, atol=1e-15)


def test_empty_sequence_gives_zero_row():
    out = attention.dense_attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.array_equal(out, np.zeros(4))


# ------------------------------------------------- recurrence and split-KV

_ERRORS = []


@pytest.mark.parametrize("n", [1, 15, 16, 17, 100, 1000])
@pytest.mark.parametrize("block", [1, 2, 3, 7, 16, 32, 512, "n"])
def test_online_recurrence_matches_dense(n, block):
    rng = np.random.default_rng(n)
    d = 64
    q, keys, values = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    scale = 1.0 / math.sqrt(d)
    b = n if block == "n" else block
    diff = np.abs(attention.online_softmax_attention(q, keys, values, scale, b)
                  - attention.dense_attention(q, keys, values, scale)).max()
    _ERRORS.append(diff)
    assert diff <= 1e-12


@pytest.mark.parametrize("n", [1, 16, 17, 511, 512, 513, 4096])
@pytest.mark.parametrize("parts", [16, 64, 512])
def test_split_kv_lse_merge_matches_dense(n, parts):
    rng = np.random.default_rng(n + parts)
    d = 32
    q, keys, values = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    scale = 1.0 / math.sqrt(d)
    got = attention.split_kv_attention(q, keys, values, scale, 16, parts)
    assert np.abs(got - attention.dense_attention(q, keys, values, scale)).max() <= 1e-12


def test_lse_merge_of_disjoint_halves_equals_whole():
    rng = np.random.default_rng(21)
    q, keys, values = rng.standard_normal(8), rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    s1 = attention.online_softmax_attention(q, keys[:11], values[:11], 0.5, 4, return_state=True)
    s2 = attention.online_softmax_attention(q, keys[11:], values[11:], 0.5, 4, return_state=True)
    merged = attention.lse_merge([s1[0], s2[0]], [s1[1], s2[1]], np.stack([s1[2], s2[2]]))
    np.testing.assert_allclose(merged, _sdpa(q, keys, values, 0.5), atol=1e-14)


def test_recurrence_error_is_a_few_ulp_like_the_review_record():
    """Context for the review's recorded largest error (2.22e-16): eight
    seeded float64 cases at several block sizes stay within a few ulp."""
    with open(os.path.join(GOLDEN, "review_record.json"), encoding="utf-8") as f:
        record = json.load(f)
    worst = 0.0
    for case in range(record["attention_cases"]):
        rng = np.random.default_rng(case)
        n, d = 8 + 5 * case, 4
        q, keys, values = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
        dense = attention.dense_attention(q, keys, values, 0.5)
        for b in (1, 2, 4, 8):
            worst = max(worst, np.abs(attention.online_softmax_attention(q, keys, values, 0.5, b)
                                      - dense).max())
    assert worst <= 16 * record["largest_absolute_error"]


# -------------------------------------------------------- paged decode


def _paged_case(rng, seq_lens, num_heads, num_kv_heads, dim, block_size):
    need = [-(-t // block_size) for t in seq_lens]
    pool = sum(need) + 3
    perm = rng.permutation(pool)
    tables = np.full((len(seq_lens), max(max(need), 1)), -1, np.int32)
    start = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[start:start + n]
        start += n
    kc = np.full((pool, num_kv_heads, block_size, dim), np.nan, np.float32)
    vc = np.full((pool, num_kv_heads, block_size, dim), np.nan, np.float32)
    keys = [rng.standard_normal((t, num_kv_heads, dim)).astype(np.float32) for t in seq_lens]
    values = [rng.standard_normal((t, num_kv_heads, dim)).astype(np.float32) for t in seq_lens]
    for i, T in enumerate(seq_lens):
        slots = np.array([tables[i][t // block_size] * block_size + t % block_size for t in range(T)])
        paging.reshape_and_cache(kc, vc, keys[i], values[i], slots, block_size)
    q = rng.standard_normal((len(seq_lens), num_heads, dim)).astype(np.float32)
    return kc, vc, tables, keys, values, q


def test_paged_decode_equals_contiguous_dense_bitwise():
    rng = np.random.default_rng(31)
    B, dim, H, Hkv = 16, 64, 4, 4
    seq_lens = [1, 15, 16, 17, 40, 100]
    kc, vc, tables, keys, values, q = _paged_case(rng, seq_lens, H, Hkv, dim, B)
    scale = float(np.float32(1 / 8))
    out = attention.paged_decode(q, "f32", kc, vc, "f32", tables, seq_lens, B, scale)
    for i, T in enumerate(seq_lens):
        for h in range(H):
            want = attention.dense_attention(q[i, h].astype(np.float64), keys[i][:, h].astype(np.float64),
                                             values[i][:, h].astype(np.float64), scale)
            assert np.array_equal(out[i, h], want)


def test_paged_decode_independent_of_physical_placement():
    rng = np.random.default_rng(32)
    B = 16
    kc, vc, tables, keys, values, q = _paged_case(rng, [33, 70], 2, 2, 8, B)
    out = attention.paged_decode(q, "f32", kc, vc, "f32", tables, [33, 70], B, 0.3)
    perm = rng.permutation(kc.shape[0])
    inv = np.argsort(perm)
    kc2, vc2 = kc[perm], vc[perm]  # physical block b moved to inv[b]
    tables2 = np.where(tables >= 0, inv[np.maximum(tables, 0)], -1)
    out2 = attention.paged_decode(q, "f32", kc2, vc2, "f32", tables2, [33, 70], B, 0.3)
    assert np.array_equal(out, out2)


def test_gqa_query_heads_read_kv_head_h_div_g():
    B, dim, H, Hkv = 4, 3, 8, 2
    kc = np.zeros((2, Hkv, B, dim), np.float32)
    vc = np.zeros((2, Hkv, B, dim), np.float32)
    for g in range(Hkv):
        vc[:, g] = g + 1.0
    q = np.zeros((1, H, dim), np.float32)
    out = attention.paged_decode(q, "f32", kc, vc, "f32", np.array([[1, 0]]), [6], B, 1.0)
    for h in range(H):
        np.testing.assert_allclose(out[0, h], h // (H // Hkv) + 1.0, rtol=0, atol=1e-15)


def test_fp8_values_are_code_times_head_scale():
    B, dim, Hkv = 4, 2, 2
    kc = np.zeros((1, Hkv, B, dim), np.uint8)  # code 0 -> 0.0 keys, equal scores
    vc = np.zeros((1, Hkv, B, dim), np.uint8)
    vc[0, 0] = 0x38  # 1.0
    vc[0, 1] = 0x40  # 2.0
    v_scale = np.array([0.5, 3.0], np.float32)
    q = np.zeros((1, 4, dim), np.uint16)
    out = attention.paged_decode(q, "bf16", kc, vc, "fp8_e4m3", np.array([[0]]), [3], B, 1.0,
                                 k_scale=np.ones(2, np.float32), v_scale=v_scale)
    np.testing.assert_allclose(out[0, :2], 0.5, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 2:], 6.0, rtol=0, atol=1e-14)


def test_zero_length_sequence_row_is_zero():
    kc = np.ones((1, 1, 4, 2), np.float32)
    out = attention.paged_decode(np.ones((1, 1, 2), np.float32), "f32", kc, kc, "f32",
                                 np.array([[0]]), [0], 4, 1.0)
    assert np.array_equal(out, np.zeros((1, 1, 2)))


def test_bf16_query_is_widened_not_rounded_again():
    bits = np.array([[[0x3F81, 0x0000]]], np.uint16)  # q = (1 + 2^-7, 0)
    kc = np.zeros((1, 1, 2, 2), np.float32)
    kc[0, 0, 0, 0] = 1.0
    vc = np.zeros((1, 1, 2, 2), np.float32)
    vc[0, 0, 0] = [1.0, 0.0]
    vc[0, 0, 1] = [0.0, 1.0]
    out = attention.paged_decode(bits, "bf16", kc, vc, "f32", np.array([[0]]), [2], 2, 1.0)
    s0 = 1.0 + 2.0 ** -7
    w0 = 1.0 / (1.0 + math.exp(-s0))
    np.testing.assert_allclose(out[0, 0], [w0, 1 - w0], atol=1e-15)
    assert formats.decode_elements(bits, "bf16")[0, 0, 0] == s0
