"""Pins of the multi-query (prefill) oracle: the matrix form against the
row-by-row form, against decode, against torch's scaled_dot_product_attention
with a causal mask (float64), and on extreme logits."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle.formats import decode_elements


def _pools(wl):
    c = wl.cache
    kc = np.zeros(c.pool_shape(), c.keys.dtype)
    vc = np.zeros(c.pool_shape(), c.keys.dtype)
    oracle.reshape_and_cache(kc, vc, c.keys, c.values, c.slots, c.block_size)
    return kc, vc


def _run(wl, fn, kc, vc):
    c = wl.cache
    return fn(wl.q, c.q_dtype, wl.query_start, kc, vc, c.kv_dtype, c.block_tables, c.seq_lens, c.block_size,
              float(c.scale), c.k_scale, c.v_scale)


@pytest.mark.parametrize("chunk", [None, 1, 7, 16, 33])
def test_matrix_form_equals_row_by_row(chunk):
    wl = workloads.prefill(1, num_seqs=4, max_len=70, chunk=chunk, num_heads=4, num_kv_heads=2, head_dim=16)
    kc, vc = _pools(wl)
    a = _run(wl, oracle.paged_prefill, kc, vc)
    b = _run(wl, oracle.paged_prefill_rowwise, kc, vc)
    assert np.max(np.abs(a - b)) < 1e-13


def test_last_row_of_each_sequence_is_the_decode_output():
    """The last query of a chunk sits at the last cached position, so it
    attends to every cached token: exactly the decode query's result."""
    wl = workloads.prefill(2, num_seqs=5, max_len=300, chunk=40, num_heads=8, num_kv_heads=2, head_dim=32)
    c = wl.cache
    kc, vc = _pools(wl)
    got = _run(wl, oracle.paged_prefill, kc, vc)
    last_rows = wl.query_start[1:] - 1
    want = oracle.paged_decode(wl.q[last_rows], c.q_dtype, kc, vc, c.kv_dtype, c.block_tables, c.seq_lens,
                               c.block_size, float(c.scale))
    assert np.max(np.abs(got[last_rows] - want)) < 1e-13


@pytest.mark.parametrize("chunk", [None, 9])
def test_against_torch_sdpa_with_causal_mask(chunk):
    """Contiguous K/V of one sequence, the chunk's queries with the mask
    key_pos <= query_pos, through torch in float64 (GQA by repeating kv
    heads)."""
    wl = workloads.prefill(3, num_seqs=3, max_len=90, chunk=chunk, num_heads=6, num_kv_heads=3, head_dim=8,
                           block_size=16)
    c = wl.cache
    kc, vc = _pools(wl)
    got = _run(wl, oracle.paged_prefill, kc, vc)
    q = decode_elements(wl.q, c.q_dtype)
    keys = decode_elements(c.keys, c.kv_dtype)
    values = decode_elements(c.values, c.kv_dtype)
    for i in range(c.num_seqs):
        T, Q = int(c.seq_lens[i]), int(wl.query_lens[i])
        r0 = int(wl.query_start[i])
        o0 = int(c.token_offsets[i])
        qi = torch.from_numpy(q[r0:r0 + Q]).permute(1, 0, 2)                     # [H][Q][d]
        k = torch.from_numpy(keys[o0:o0 + T]).permute(1, 0, 2).repeat_interleave(2, 0)
        v = torch.from_numpy(values[o0:o0 + T]).permute(1, 0, 2).repeat_interleave(2, 0)
        pos = torch.arange(T - Q, T)
        mask = torch.arange(T)[None, :] <= pos[:, None]
        want = torch.nn.functional.scaled_dot_product_attention(qi, k, v, attn_mask=mask,
                                                                scale=float(c.scale)).permute(1, 0, 2).numpy()
        assert np.max(np.abs(got[r0:r0 + Q] - want)) < 1e-12


def test_first_token_of_a_full_prefill_returns_its_own_value():
    """Position 0 attends only to itself: its output is v_0 exactly."""
    wl = workloads.prefill(4, num_seqs=3, max_len=50, num_heads=4, num_kv_heads=4, head_dim=16)
    c = wl.cache
    kc, vc = _pools(wl)
    got = _run(wl, oracle.paged_prefill, kc, vc)
    values = decode_elements(c.values, c.kv_dtype)
    for i in range(c.num_seqs):
        assert np.array_equal(got[int(wl.query_start[i])], values[int(c.token_offsets[i])])


def test_extreme_logits_stay_finite():
    wl = workloads.prefill(5, num_seqs=2, max_len=60, chunk=20, num_heads=2, num_kv_heads=1, head_dim=16)
    c = wl.cache
    kc, vc = _pools(wl)
    qf = decode_elements(wl.q, c.q_dtype) * 400.0  # logits of several hundred
    q_big = qf.astype(np.float32)  # f32 storage holds them exactly enough
    got = oracle.paged_prefill(q_big, "f32", wl.query_start, kc, vc, c.kv_dtype, c.block_tables, c.seq_lens,
                               c.block_size, float(c.scale))
    assert np.all(np.isfinite(got))
    # each output row is a convex combination of the value rows it may see
    values = decode_elements(c.values, c.kv_dtype)
    for i in range(c.num_seqs):
        o0, T = int(c.token_offsets[i]), int(c.seq_lens[i])
        vmax = np.abs(values[o0:o0 + T]).max()
        r0, r1 = int(wl.query_start[i]), int(wl.query_start[i + 1])
        assert np.abs(got[r0:r1]).max() <= vmax + 1e-12


def test_empty_chunk_writes_nothing():
    wl = workloads.build_prefill_workload("p0", 6, seq_lens=[30, 12], query_lens=[0, 12], num_heads=2,
                                          num_kv_heads=1, head_dim=8, block_size=16, kv_dtype="f32", q_dtype="f32")
    kc, vc = _pools(wl)
    got = _run(wl, oracle.paged_prefill, kc, vc)
    assert got.shape == (12, 2, 8)
