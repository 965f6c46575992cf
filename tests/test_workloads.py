"""Seeded input generators (CPU): structure of the tables, slots and copy
pairs, determinism, stored formats, and the generator -> oracle chain
(scatter every token, gather every sequence, compare with the logical rows)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads.generators import build_decode_workload


def _structure(wl):
    B = wl.block_size
    used = []
    for i, T in enumerate(wl.seq_lens):
        n = -(-int(T) // B)
        row = wl.block_tables[i]
        assert np.all(row[:n] >= 0) and np.all(row[n:] == -1)
        used += row[:n].tolist()
    assert len(used) == len(set(used)), "a block is owned twice"
    assert all(0 <= b < wl.num_blocks for b in used)
    # slots agree with the tables
    for i, T in enumerate(wl.seq_lens):
        lo = int(wl.token_offsets[i])
        for t in (0, int(T) // 2, int(T) - 1) if T else ():
            assert wl.slots[lo + t] == wl.block_tables[i][t // B] * B + t % B
    # copy pairs: used sources, spare distinct destinations
    src, dst = wl.copy_pairs[:, 0], wl.copy_pairs[:, 1]
    assert set(src.tolist()) <= set(used)
    assert not set(dst.tolist()) & set(used) and len(set(dst.tolist())) == len(dst)
    assert len(wl.prefill_rows()) + len(wl.step_rows()) == int(wl.seq_lens.sum())


def test_tiny_config_matches_its_description():
    wl = workloads.tiny(0)
    assert wl.seq_lens.tolist() == [1, 17, 40, 100] and wl.num_blocks == 32
    assert (wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.block_size) == (4, 4, 64, 16)
    assert wl.keys.dtype == np.float32 and len(wl.copy_pairs) == 3
    assert wl.scale == np.float32(0.125)
    assert oracle.accounting.tail_waste(wl.seq_lens, 16) == 50
    _structure(wl)


def test_gqa_small_structure_and_determinism():
    a = workloads.gqa(3, num_seqs=9, max_len=700)
    b = workloads.gqa(3, num_seqs=9, max_len=700)
    _structure(a)
    for f in ("seq_lens", "block_tables", "keys", "values", "q", "copy_pairs", "slots"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = workloads.gqa(4, num_seqs=9, max_len=700)
    assert not np.array_equal(a.keys[:100], c.keys[:100])
    assert a.keys.dtype == np.uint16 and a.kv_dtype == "bf16"


def test_bf16_storage_is_round_to_nearest_of_normals():
    wl = workloads.gqa(0, num_seqs=2, max_len=40)
    vals = oracle.decode_elements(wl.keys, "bf16")
    assert abs(vals.mean()) < 0.05 and 0.9 < vals.std() < 1.1
    # every stored value is a bfloat16 (low 16 bits of the float32 are zero)
    f32 = torch.from_numpy(vals.astype(np.float32))
    assert torch.equal(f32.to(torch.bfloat16).to(torch.float32), f32)


def test_fp8_codes_and_scales():
    wl = workloads.long_fp8(0, num_seqs=2, seq_len=300)
    _structure(wl)
    assert wl.keys.dtype == np.uint8 and wl.k_scale.shape == (8,) and wl.v_scale.dtype == np.float32
    table = oracle.e4m3fn_table()
    assert not np.isnan(table[wl.keys]).any() and not np.isnan(table[wl.values]).any()
    # the largest |code| of every head reaches the format's maximum
    assert np.all(np.abs(table[wl.keys]).max(axis=(0, 2)) == 448.0)
    deq = table[wl.keys] * wl.k_scale.astype(np.float64)[None, :, None]
    assert 0.85 < deq.std() < 1.15


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("gqa", dict(num_seqs=5, max_len=300)),
                                     ("mha", dict(num_seqs=4, max_len=200)),
                                     ("long_fp8", dict(num_seqs=2, seq_len=100))])
def test_generator_to_oracle_round_trip(name, kw):
    wl = workloads.make(name, 1, **kw)
    _structure(wl)
    kc = np.zeros(wl.pool_shape(), wl.keys.dtype)
    vc = np.zeros(wl.pool_shape(), wl.keys.dtype)
    oracle.reshape_and_cache(kc, vc, wl.keys, wl.values, wl.slots, wl.block_size)
    for i, T in enumerate(wl.seq_lens):
        lo, hi = wl.token_offsets[i], wl.token_offsets[i + 1]
        g = oracle.gather_sequence(kc, wl.block_tables[i], int(T), wl.block_size)
        assert np.array_equal(g, wl.keys[lo:hi].transpose(1, 0, 2))
        g = oracle.gather_sequence(vc, wl.block_tables[i], int(T), wl.block_size)
        assert np.array_equal(g, wl.values[lo:hi].transpose(1, 0, 2))


def test_shared_prefix_extreme_queries_reach_target():
    wl = workloads.shared_prefix(0, num_prompts=2, beams=2, max_suffix=20)
    G = wl.num_heads // wl.num_kv_heads
    q = oracle.decode_elements(wl.q, "bf16")
    for s in range(wl.num_seqs):
        keys = oracle.decode_elements(wl.logical_rows(s, "k"), "bf16")
        mags = [np.abs(keys[:, h // G] @ q[s, h]).max() * float(wl.scale) for h in range(wl.num_heads)]
        if wl.extreme[s]:
            assert all(abs(m - 80.0) < 1.0 for m in mags)  # bf16 rounding of q moves it slightly
        else:
            assert max(mags) < 10.0


def test_edge_lengths_with_empty_sequence():
    wl = build_decode_workload("edge", 0, seq_lens=[0, 1, 16, 17], num_heads=4, num_kv_heads=2, head_dim=64,
                               block_size=16, kv_dtype="bf16", q_dtype="bf16", spare_blocks=2, num_copy_pairs=1,
                               partition_size=32)
    _structure(wl)
    assert np.all(wl.block_tables[0] == -1)


def test_prefill_logit_target_reaches_the_target():
    """Each query row's largest visible |scale q.k| is the target, up to the
    rounding of q to bf16 (relative 2^-8 per element)."""
    wl = workloads.build_prefill_workload("px", 3, seq_lens=[5, 40], query_lens=[5, 17], num_heads=4,
                                          num_kv_heads=2, head_dim=16, block_size=16, kv_dtype="bf16",
                                          q_dtype="bf16", logit_target=80.0)
    c = wl.cache
    q = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    k = torch.from_numpy(c.keys.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for i in range(c.num_seqs):
        T, Q = int(c.seq_lens[i]), int(wl.query_lens[i])
        keys = k[c.token_offsets[i]:c.token_offsets[i + 1]]
        for j in range(Q):
            pos = T - Q + j
            for h in range(4):
                top = np.abs(keys[:pos + 1, h // 2, :] @ q[wl.query_start[i] + j, h]).max() * float(c.scale)
                assert abs(top - 80.0) <= 80.0 * 2.0 ** -6, (i, j, h, top)
