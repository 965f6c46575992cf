"""pa_decode_append_cow on the GPU: the copy-on-write copies, the new tokens'
store and the decode in one call give bitwise the pools and outputs of
pa_copy_blocks followed by pa_decode_append -- with destinations no table
names (the decode reads none of them; their sources are blocks no sequence
appends to this step, as the call requires), with a pair outside the pool
(skipped by both), and in a fork: two sequences share their last block, one of them
has been given a private copy that this step makes, and both append their new
token at the same row.  The fork's output is also checked against the oracle
(copy, then store, then decode, from pools it builds itself).  The GQA-4
kernel and the generic kernel (every other group and format) take the copies
in their launch; the FP8 matrix-core shape (G = 8, head_dim 128) and more
than 16 pairs make the two calls and must agree as well.  Given no tokens,
the call is pa_copy_blocks then pa_decode: one launch for the FP8
matrix-core shape, two calls elsewhere, bitwise equal either way.

The copy-on-write steps follow the explainer's section "Copy-on-Write（CoW）に
よるメモリ共有" (copy the shared block, remap the writer's table entry)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_142_amd as pa
import workloads
from gpu_util import TOL, DeviceCase, assert_close, oracle_out, oracle_pools, out_as_f64, poison_host, to_host_raw

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def _new_tokens(case, wl):
    """[N][H_kv][d] rows of each sequence's newest token (zeros for empty ones)."""
    keys = case.keys.index_select(0, case.step).contiguous()
    values = case.values.index_select(0, case.step).contiguous()
    if len(case.step) == wl.num_seqs:
        return keys, values
    full_k = torch.zeros((wl.num_seqs,) + tuple(keys.shape[1:]), dtype=keys.dtype, device="cuda")
    full_v = torch.zeros_like(full_k)
    has = torch.from_numpy(np.nonzero(wl.seq_lens > 0)[0]).cuda()
    full_k[has] = keys
    full_v[has] = values
    return full_k, full_v


def _sources_off_last_blocks(wl, seed):
    """The workload's pairs with every source moved off the blocks the step
    appends to (sequences' last blocks): a pair from such a block to a
    destination no appending sequence owns would race with the store of the
    new token (pagedattn.h, pa_decode_append_cow)."""
    B = wl.block_size
    lens = wl.seq_lens.astype(np.int64)
    last = {int(wl.block_tables[i, (t - 1) // B]) for i, t in enumerate(lens) if t > 0}
    named = wl.block_tables[wl.block_tables >= 0].ravel()
    pool = np.array(sorted({int(b) for b in named} - last), np.int64)
    src = np.random.default_rng(seed).choice(pool, size=len(wl.copy_pairs), replace=False)
    return np.stack([src, wl.copy_pairs[:, 1]], axis=1).astype(np.int64)


def _run(wl, pairs_np):
    """(output, K pool, V pool) bytes of the one call and of the two calls."""
    res = []
    for fused in (True, False):
        case = DeviceCase(wl)  # pools hold every token but each sequence's newest
        key, value = _new_tokens(case, wl)
        pairs = torch.from_numpy(np.ascontiguousarray(pairs_np, dtype=np.int64)).cuda()
        if fused:
            pa.pa_decode_append_cow(**case.decode_args(), key=key, value=value, block_pairs=pairs)
        else:
            if len(pairs_np):
                pa.pa_copy_blocks(case.k_cache, case.v_cache, pairs)
            pa.pa_decode_append(**case.decode_args(), key=key, value=value)
        torch.cuda.synchronize()
        res.append((_bytes(case.out), _bytes(case.k_cache), _bytes(case.v_cache), case))
    (o1, k1, v1, case), (o0, k0, v0, _) = res
    assert np.array_equal(k0, k1), "K pool differs from copy + decode with append"
    assert np.array_equal(v0, v1), "V pool differs from copy + decode with append"
    assert np.array_equal(o0, o1), "output differs from copy + decode with append"
    return case


@pytest.mark.parametrize("kv,block,P,npairs", [
    ("bf16", 16, 832, 15),   # 15 pairs and one outside the pool: one launch (at most 16 pairs)
    ("bf16", 16, 512, 15),
    ("f16", 32, 512, 15),
    ("bf16", 16, 832, 40),   # more pairs: pa_copy_blocks, then pa_decode_append
])
def test_cow_spare_destinations_match_two_calls(kv, block, P, npairs):
    wl = workloads.build_decode_workload(
        f"cow_spare_{kv}_{block}_{P}", 7, seq_lens=np.random.default_rng(7).integers(1, 3000, size=24),
        num_heads=32, num_kv_heads=8, head_dim=128, block_size=block, kv_dtype=kv, q_dtype=kv, spare_blocks=48,
        num_copy_pairs=npairs, partition_size=P)
    spare = _sources_off_last_blocks(wl, 71)
    pairs = np.concatenate([spare, [[wl.num_blocks + 5, int(spare[0, 1])]]])  # one pair outside the pool
    print(f"[case] cow spare {wl.name}: {len(pairs)} pairs", flush=True)
    _run(wl, pairs)


@pytest.mark.parametrize("kv,q,heads,kv_heads,dim,block,P,npairs", [
    ("f16", "f16", 40, 40, 128, 16, 512, 15),     # G = 1, 40 kv heads: each block copy in 10 chunks
    ("f32", "f32", 8, 4, 64, 16, 256, 15),        # G = 2, fp32
    ("fp8_e4m3", "bf16", 32, 8, 128, 16, 512, 12),  # FP8 through the generic kernel (G = 4)
    ("bf16", "bf16", 64, 8, 128, 32, 512, 15),    # G = 8, 16-bit
    ("fp8_e4m3", "bf16", 64, 8, 128, 16, 512, 10),  # FP8 matrix-core shape: the two calls
])
def test_cow_generic_shapes_match_two_calls(kv, q, heads, kv_heads, dim, block, P, npairs):
    wl = workloads.build_decode_workload(
        f"cow_gen_{kv}_{heads}_{kv_heads}_{dim}_{block}", 9, seq_lens=np.random.default_rng(9).integers(1, 1500, size=20),
        num_heads=heads, num_kv_heads=kv_heads, head_dim=dim, block_size=block, kv_dtype=kv, q_dtype=q,
        spare_blocks=40, num_copy_pairs=npairs, partition_size=P)
    spare = _sources_off_last_blocks(wl, 91)
    pairs = np.concatenate([spare, [[-3, int(spare[0, 1])]]])  # one pair outside the pool
    print(f"[case] cow generic {wl.name}: {len(pairs)} pairs", flush=True)
    _run(wl, pairs)


def _fork_workload(kv, block, lens, P, heads=32, kv_heads=8):
    """Sequences 0 and 1 share every block (the same length); sequence 0's
    last block has been given a private copy (a block no table named), and
    sequence 2's first block too; the pairs make those copies."""
    wl = workloads.build_decode_workload(
        f"cow_fork_{kv}_{block}_{P}_{heads}_{kv_heads}", 11, seq_lens=lens, num_heads=heads, num_kv_heads=kv_heads,
        head_dim=128, block_size=block, kv_dtype=kv, q_dtype=kv, spare_blocks=8, num_copy_pairs=0, partition_size=P)
    bt = wl.block_tables.copy()
    assert lens[0] == lens[1]
    bt[1] = bt[0]  # sequence 1 now shares sequence 0's blocks (its own become unreferenced)
    used = set(int(x) for x in bt[bt >= 0].ravel())
    free = [b for b in range(wl.num_blocks) if b not in used]
    last0 = (int(lens[0]) - 1) // block
    pairs = [[int(bt[0, last0]), free[0]], [int(bt[2, 0]), free[1]]]
    bt[0, last0] = free[0]
    bt[2, 0] = free[1]
    return dataclasses.replace(wl, block_tables=bt), np.array(pairs, dtype=np.int64)


def _oracle_after(wl, pairs, key_raw, value_raw):
    """Oracle pools after copy, then the new tokens' store, and its output."""
    kc = poison_host(wl.pool_shape(), wl.kv_dtype)
    vc = poison_host(wl.pool_shape(), wl.kv_dtype)
    pre = wl.prefill_rows()
    oracle.reshape_and_cache(kc, vc, wl.keys[pre], wl.values[pre], wl.slots[pre], wl.block_size)
    oracle.copy_blocks(kc, vc, pairs)
    seqs = np.nonzero(wl.seq_lens > 0)[0]
    pos = wl.seq_lens[seqs].astype(np.int64) - 1
    slots = wl.block_tables[seqs, pos // wl.block_size].astype(np.int64) * wl.block_size + pos % wl.block_size
    oracle.reshape_and_cache(kc, vc, key_raw[seqs], value_raw[seqs], slots, wl.block_size)
    out = oracle.paged_decode(wl.q, wl.q_dtype, kc, vc, wl.kv_dtype, wl.block_tables, wl.seq_lens, wl.block_size,
                              float(wl.scale), None, None)
    return kc, vc, out


@pytest.mark.parametrize("kv,block,lens,heads,kv_heads", [
    ("bf16", 16, [65, 65, 300, 40, 1000], 32, 8),    # new token at the first row of a block
    ("bf16", 16, [80, 80, 17, 2000, 5], 32, 8),      # at the last row
    ("f16", 32, [33, 33, 640, 1, 129], 32, 8),
    ("f16", 16, [80, 80, 17, 2000, 5], 16, 16),      # the generic kernel (G = 1)
    ("bf16", 32, [65, 65, 300, 40, 1000], 16, 8),    # the generic kernel (G = 2)
])
def test_cow_fork_matches_two_calls_and_oracle(kv, block, lens, heads, kv_heads):
    wl, pairs = _fork_workload(kv, block, np.array(lens), 512, heads, kv_heads)
    print(f"[case] cow fork {wl.name}: lens {lens}, pairs {pairs.tolist()}", flush=True)
    case = _run(wl, pairs)
    st = wl.step_rows()
    key_raw = np.zeros((wl.num_seqs,) + wl.keys.shape[1:], wl.keys.dtype)
    value_raw = np.zeros_like(key_raw)
    key_raw[wl.seq_lens > 0] = wl.keys[st]
    value_raw[wl.seq_lens > 0] = wl.values[st]
    kc, vc, want = _oracle_after(wl, pairs, key_raw, value_raw)

    assert np.array_equal(to_host_raw(case.k_cache, kv), kc), "K pool differs from the oracle's"
    assert np.array_equal(to_host_raw(case.v_cache, kv), vc), "V pool differs from the oracle's"
    assert_close(out_as_f64(case.out), want, TOL[kv], "fork decode vs oracle")


def test_cow_g1_matches_two_calls():
    wl = workloads.build_decode_workload(
        "cow_g1", 3, seq_lens=[5, 300, 17, 1024], num_heads=8, num_kv_heads=8, head_dim=128, block_size=16,
        kv_dtype="f16", q_dtype="f16", spare_blocks=8, num_copy_pairs=4, partition_size=512)
    print(f"[case] cow g1 {wl.name}", flush=True)
    _run(wl, wl.copy_pairs)


def test_cow_without_pairs_is_decode_with_append():
    wl = workloads.build_decode_workload(
        "cow_none", 5, seq_lens=[100, 2000, 1], num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        kv_dtype="bf16", q_dtype="bf16", spare_blocks=4, num_copy_pairs=0, partition_size=512)
    print(f"[case] cow none {wl.name}", flush=True)
    _run(wl, np.zeros((0, 2), np.int64))



def _run_no_tokens(wl):
    """(output, K pool, V pool) bytes of pa_decode_append_cow without tokens
    against pa_copy_blocks then pa_decode, after the step's scatter (quantized
    on write for FP8 pools), with the workload's pairs."""
    res = []
    for fused in (True, False):
        case = DeviceCase(wl)
        if case.quantize_step:
            pa.pa_reshape_and_cache_fp8(case.step_keys, case.step_values, case.k_cache, case.v_cache, case.k_scale,
                                        case.v_scale, case.step_slots)
        else:
            pa.pa_reshape_and_cache(case.step_keys, case.step_values, case.k_cache, case.v_cache, case.step_slots)
        if fused:
            pa.pa_decode_append_cow(**case.decode_args(), key=None, value=None, block_pairs=case.pairs)
        else:
            pa.pa_copy_blocks(case.k_cache, case.v_cache, case.pairs)
            case.decode()
        torch.cuda.synchronize()
        res.append((_bytes(case.out), _bytes(case.k_cache), _bytes(case.v_cache), case))
    (o1, k1, v1, case), (o0, k0, v0, _) = res
    assert np.array_equal(k0, k1), "K pool differs from copy + decode"
    assert np.array_equal(v0, v1), "V pool differs from copy + decode"
    assert np.array_equal(o0, o1), "output differs from copy + decode"
    return case


@pytest.mark.parametrize("kv,q,heads,kv_heads,block,P,npairs", [
    ("fp8_e4m3", "bf16", 64, 8, 16, 512, 15),   # FP8 matrix-core shape: one launch
    ("fp8_e4m3", "bf16", 64, 8, 32, 512, 15),
    ("fp8_e4m3", "bf16", 64, 8, 16, 1024, 15),  # partitions of 64 blocks
    ("fp8_e4m3", "bf16", 64, 8, 16, 512, 40),   # more pairs: the two calls
    ("bf16", "bf16", 32, 8, 16, 512, 15),       # other shapes: the two calls
])
def test_cow_without_tokens_matches_copy_then_decode(kv, q, heads, kv_heads, block, P, npairs):
    """Sources anywhere (no token is stored in the call, so a copy races with
    nothing), destinations both spare blocks and blocks that tables name (read
    through their sources), one pair outside the pool.  One case is also
    checked against the oracle (scatter, copy, decode on its own pools)."""
    wl = workloads.build_decode_workload(
        f"cow_nt_{kv}_{heads}_{kv_heads}_{block}_{P}", 13, seq_lens=np.random.default_rng(13).integers(1, 3000, size=12),
        num_heads=heads, num_kv_heads=kv_heads, head_dim=128, block_size=block, kv_dtype=kv, q_dtype=q,
        spare_blocks=48, num_copy_pairs=npairs, partition_size=P)
    pairs = wl.copy_pairs.copy()
    # the first three destinations: blocks some table names, none of them a source
    srcs = set(pairs[:, 0].tolist())
    named = np.unique(wl.block_tables[wl.block_tables >= 0])
    pairs[:3, 1] = [int(b) for b in np.random.default_rng(14).permutation(named) if int(b) not in srcs][:3]
    pairs = np.concatenate([pairs, [[wl.num_blocks + 2, int(pairs[-1, 1])]]]).astype(np.int64)
    wl = dataclasses.replace(wl, copy_pairs=pairs)
    print(f"[case] cow without tokens {wl.name}: {len(pairs)} pairs", flush=True)
    case = _run_no_tokens(wl)
    if npairs == 15 and kv == "fp8_e4m3" and block == 16 and P == 512:
        in_pool = dataclasses.replace(wl, copy_pairs=pairs[:-1])  # the oracle copies in-pool pairs only
        kc, vc = oracle_pools(in_pool)
        assert_close(out_as_f64(case.out), oracle_out(in_pool, kc, vc), TOL[kv], "copy + decode vs oracle")
