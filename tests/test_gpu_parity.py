"""GPU parity of the hot path (C ABI) against the float64 oracle.

Every test fills the pool through ``pa_reshape_and_cache``, runs one step
(the step's new tokens, the block copies, then ``pa_decode``) and compares:

* the whole K and V pools byte for byte with the oracle's scatter/copy (the
  pools start as 0xFF poison, so untouched slots are checked too);
* ``out`` element by element with the oracle, within 1e-5 (fp32 KV), 1e-2
  (fp16/bf16 KV) or 2e-2 (fp8 KV, oracle on the dequantized values).

Small variants are compared on every row; so is every full-size workload on
seed 0 (gqa on three seeds); other seeds of mha and long_fp8 on sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_142_amd as pa
import workloads
from workloads.generators import build_decode_workload
from gpu_util import (TOL, DeviceCase, assert_close, oracle_out, oracle_pools, out_as_f64, to_host_raw)

pytestmark = pytest.mark.gpu


def _pools_bitwise(case, wl, kc, vc):
    gk = to_host_raw(case.k_cache, wl.kv_dtype)
    gv = to_host_raw(case.v_cache, wl.kv_dtype)
    assert np.array_equal(gk.view(np.uint8), kc.view(np.uint8)), "K pool differs from the oracle"
    assert np.array_equal(gv.view(np.uint8), vc.view(np.uint8)), "V pool differs from the oracle"


def _run_and_check(wl, rows=None, tol=None, check_pools=True, out_fmt="f32"):
    print(f"[case] {wl.name} seed={wl.seed} N={wl.num_seqs} H={wl.num_heads}/{wl.num_kv_heads} "
          f"d={wl.head_dim} B={wl.block_size} P={wl.partition_size} kv={wl.kv_dtype} "
          f"sumT={int(wl.seq_lens.sum())}", flush=True)
    case = DeviceCase(wl, out_fmt=out_fmt)
    case.run_step()
    torch.cuda.synchronize()
    kc, vc = oracle_pools(wl)
    if check_pools:
        _pools_bitwise(case, wl, kc, vc)
    got = out_as_f64(case.out)
    assert np.all(np.isfinite(got)), "non-finite output rows"
    want = oracle_out(wl, kc, vc, rows=rows)
    if rows is not None:
        got = got[rows]
    t = TOL[wl.kv_dtype] if tol is None else tol
    return case, assert_close(got, want, t, wl.name)


# ------------------------------------------------------------- small, all rows

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_fp32(seed):
    _run_and_check(workloads.tiny(seed))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gqa_bf16_small(seed):
    _run_and_check(workloads.gqa(seed, num_seqs=12, max_len=1500))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mha_fp16_small(seed):
    _run_and_check(workloads.mha(seed, num_seqs=16, max_len=700))


@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_small(block_size, seed):
    _run_and_check(workloads.long_fp8(seed, block_size=block_size, num_seqs=3, seq_len=1300))


@pytest.mark.parametrize("partition_size", [16, 64, 256, 1024, 4096, 8192])
def test_partition_sizes(partition_size):
    """Four query heads per kv head, partitions from one block to more than
    64 blocks per wave."""
    _run_and_check(workloads.gqa(3, num_seqs=10, max_len=9000 if partition_size > 1024 else 2100,
                                 partition_size=partition_size))


@pytest.mark.parametrize("kv,q,heads,num_seqs", [("bf16", "bf16", 32, 65), ("bf16", "bf16", 32, 64),
                                                  ("fp8_e4m3", "bf16", 64, 80), ("f16", "f16", 8, 100)])
def test_work_order_sources(kv, q, heads, num_seqs):
    """Up to 64 sequences, partition workgroups derive the largest-first work
    order from the lengths themselves; beyond that a plan kernel writes it.
    Both orders cover every (sequence, partition) once."""
    lens = np.random.default_rng(num_seqs).integers(0, 1400, size=num_seqs)
    wl = build_decode_workload(f"order_{kv}_{num_seqs}", 14, seq_lens=lens, num_heads=heads, num_kv_heads=8,
                               head_dim=128, block_size=16, kv_dtype=kv, q_dtype=q, spare_blocks=4,
                               num_copy_pairs=2, partition_size=256)
    _run_and_check(wl)


def test_gqa4_one_block_partitions_long_sequences():
    """Partitions of one block over long sequences: hundreds of partition
    states per row for the reduce."""
    lens = [9000] * 7 + [8191]
    wl = build_decode_workload("gqa4_many", 13, seq_lens=lens, num_heads=32, num_kv_heads=8, head_dim=128,
                               block_size=16, kv_dtype="bf16", q_dtype="bf16", spare_blocks=4,
                               num_copy_pairs=2, partition_size=16)
    _run_and_check(wl, rows=[0, 3, 7])


@pytest.mark.parametrize("block_size,partition_size", [
    (16, 16), (16, 48), (16, 80), (16, 1024), (16, 2048), (32, 32), (32, 96), (32, 2048)])
def test_fp8_group8_partitions(block_size, partition_size):
    """FP8 KV with eight query heads per kv head: partitions of one block, of
    an odd number of blocks (a 32-token step that crosses the partition end),
    and of more than 64 blocks."""
    lens = [1, 31, 33, 47, 100, 511, 700, 1025, 2100, 2600]
    wl = build_decode_workload(f"fp8g8_{block_size}_{partition_size}", 9, seq_lens=lens, num_heads=64,
                               num_kv_heads=8, head_dim=128, block_size=block_size, kv_dtype="fp8_e4m3",
                               q_dtype="bf16", spare_blocks=4, num_copy_pairs=3, partition_size=partition_size)
    _run_and_check(wl)


def test_fp8_group8_one_block_partitions_long_sequences():
    """Partitions of one block over long sequences: hundreds of partition
    states per row for the reduce."""
    lens = [9000] * 7 + [8191]
    wl = build_decode_workload("fp8g8_many", 12, seq_lens=lens, num_heads=64, num_kv_heads=8, head_dim=128,
                               block_size=16, kv_dtype="fp8_e4m3", q_dtype="bf16", spare_blocks=4,
                               num_copy_pairs=2, partition_size=16)
    _run_and_check(wl, rows=[0, 3, 7])


EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 511, 512, 513, 1023, 1024, 1025]


@pytest.mark.parametrize("kv,q,heads,kv_heads,dim,block", [
    ("bf16", "bf16", 32, 8, 128, 16),
    ("bf16", "bf16", 32, 8, 128, 32),   # GQA-4, 32-token blocks staged as two 16-row tiles
    ("bf16", "bf16", 8, 4, 64, 32),
    ("bf16", "bf16", 16, 2, 128, 32),
    ("bf16", "bf16", 16, 4, 64, 16),
    ("f16", "f16", 32, 8, 64, 32),
    ("f16", "f16", 32, 8, 128, 32),
    ("f16", "f16", 4, 4, 128, 16),
    ("f16", "f16", 8, 1, 64, 16),
    ("f32", "f32", 4, 4, 64, 16),
    ("f32", "f32", 8, 4, 128, 32),
    ("fp8_e4m3", "bf16", 64, 8, 128, 16),
    ("fp8_e4m3", "bf16", 64, 8, 128, 32),
    ("fp8_e4m3", "bf16", 16, 4, 64, 32),
    ("fp8_e4m3", "bf16", 16, 2, 128, 16),
])
def test_edge_lengths_and_shapes(kv, q, heads, kv_heads, dim, block):
    wl = build_decode_workload(f"edge_{kv}_{heads}_{kv_heads}_{dim}_{block}", 5, seq_lens=EDGE_LENS,
                               num_heads=heads, num_kv_heads=kv_heads, head_dim=dim, block_size=block,
                               kv_dtype=kv, q_dtype=q, spare_blocks=4, num_copy_pairs=3, partition_size=512)
    case, _ = _run_and_check(wl)
    got = out_as_f64(case.out)
    assert np.array_equal(got[0], np.zeros_like(got[0])), "empty sequence must give a zero row"


@pytest.mark.parametrize("out_fmt", ["bf16", "f16"])
def test_low_precision_output(out_fmt):
    wl = workloads.gqa(4, num_seqs=8, max_len=1200)
    case = DeviceCase(wl, out_fmt=out_fmt)
    case.run_step()
    torch.cuda.synchronize()
    kc, vc = oracle_pools(wl)
    want = oracle_out(wl, kc, vc)
    ulp_dtype = torch.bfloat16 if out_fmt == "bf16" else torch.float16
    want_rounded = torch.from_numpy(want).to(ulp_dtype).double().numpy()
    got = out_as_f64(case.out)
    # within the fp32 tolerance of the oracle rounded to the output format,
    # or one unit in the last place of that format
    ulp = np.abs(want_rounded) * (2.0 ** -7 if out_fmt == "bf16" else 2.0 ** -10) + 1e-30
    err = np.abs(got - want_rounded)
    print(f"[parity] out={out_fmt}: max abs err vs rounded oracle {err.max():.3e}", flush=True)
    assert np.all((err <= TOL["bf16"]) | (err <= ulp))


# ---------------------------------------------------- full-size workloads

def _sample_rows(wl, k, seed=0):
    lens = wl.seq_lens
    rows = {0, wl.num_seqs - 1, int(np.argmax(lens)), int(np.argmin(lens))}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.choice(wl.num_seqs, size=min(k, wl.num_seqs), replace=False))
    return sorted(rows)


@pytest.mark.parametrize("seed,partition_size", [(0, 832), (0, 768), (0, 512), (1, 832), (2, 832)])
def test_gqa_full_size_all_rows(seed, partition_size):
    _run_and_check(workloads.gqa(seed, partition_size=partition_size))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mha_full_size(seed):
    """Seed 0: all 256 rows; the other seeds: sampled rows (the pools are
    compared whole for every seed)."""
    wl = workloads.mha(seed)
    _run_and_check(wl, rows=None if seed == 0 else _sample_rows(wl, 24, seed))


@pytest.mark.parametrize("seed,block_size", [(0, 16), (0, 32), (1, 16), (2, 32)])
def test_long_fp8_full_size(seed, block_size):
    """Seed 0: all 16 rows at both block sizes; the other seeds: sampled rows."""
    wl = workloads.long_fp8(seed, block_size=block_size)
    _run_and_check(wl, rows=None if seed == 0 else sorted({0, 15, 3 + 4 * seed}))


def test_empty_and_invalid_rows():
    """Empty sequences get zero rows and a sequence whose length exceeds
    max_seq_len gets a NaN row; every other row matches the oracle."""
    lens = [0, 700, 0, 1500, 2000, 0, 33]
    wl = build_decode_workload("fill_rows", 10, seq_lens=lens, num_heads=32, num_kv_heads=8, head_dim=128,
                               block_size=16, kv_dtype="bf16", q_dtype="bf16", spare_blocks=4,
                               num_copy_pairs=2, partition_size=256)
    case = DeviceCase(wl)
    case.run_cache_ops()
    case.out.fill_(123.0)
    bad_lens = case.seq_lens.clone()
    bad_lens[3] = wl.max_seq_len + 1  # beyond the host bound: invalid
    args = case.decode_args()
    args["seq_lens"] = bad_lens
    pa.pa_decode(**args)
    torch.cuda.synchronize()
    got = out_as_f64(case.out)
    for i in (0, 2, 5):
        assert np.array_equal(got[i], np.zeros_like(got[i])), f"row {i} of an empty sequence"
    assert np.isnan(got[3]).all(), "row of an invalid sequence must be NaN"
    kc, vc = oracle_pools(wl)
    rows = [1, 4, 6]
    assert_close(got[rows], oracle_out(wl, kc, vc, rows=rows), TOL["bf16"], "rows beside empty/invalid ones")


# ------------------------------------------------ indexing, determinism

def test_deterministic_and_placement_independent():
    wl = workloads.gqa(6, num_seqs=16, max_len=3000)
    case = DeviceCase(wl)
    case.run_step()
    first = case.out.clone()
    case.decode()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int32), case.out.view(torch.int32)), "repeat call differs"
    # relabel physical blocks: block b moves to inv[b]
    perm = torch.from_numpy(np.random.default_rng(1).permutation(wl.num_blocks)).to("cuda")
    inv = torch.argsort(perm)
    k2 = case.k_cache.index_select(0, perm).contiguous()
    v2 = case.v_cache.index_select(0, perm).contiguous()
    bt = case.block_tables.long()
    bt2 = torch.where(bt >= 0, inv[bt.clamp(min=0)], bt).to(torch.int32).contiguous()
    out2 = torch.empty_like(case.out)
    case.decode(out=out2, block_tables=bt2, k_cache=k2, v_cache=v2)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int32), out2.view(torch.int32)), "output depends on placement"


def _bf16_bits(x):
    return np.array([x], np.float32).view(np.uint32)[0] >> 16


@pytest.mark.parametrize("position", [0, 15, 16, 255, 511, 512, 513, 1000, "last"])
def test_one_hot_probe_selects_value_bitwise(position):
    """A key whose score beats every other by > 200 selects its value row
    exactly (exp(-200) underflows to 0 in float32)."""
    wl = workloads.gqa(7, num_seqs=4, max_len=1100)
    i, g = 1, 3
    T = int(wl.seq_lens[i])
    if T < 1030:  # make the probed sequence long enough for every position
        lens = wl.seq_lens.copy()
        lens[i] = 1037
        wl = build_decode_workload("probe", 7, seq_lens=lens, num_heads=32, num_kv_heads=8, head_dim=128,
                                   block_size=16, kv_dtype="bf16", q_dtype="bf16", spare_blocks=4,
                                   num_copy_pairs=2, partition_size=512)
        T = 1037
    j = T - 1 if position == "last" else position
    G = wl.num_heads // wl.num_kv_heads
    lo, hi = int(wl.token_offsets[i]), int(wl.token_offsets[i + 1])
    wl.keys[lo:hi, g, 0] = 0
    wl.keys[lo + j, g, 0] = _bf16_bits(4096.0)
    wl.q[i, g * G:(g + 1) * G, :] = 0
    wl.q[i, g * G:(g + 1) * G, 0] = _bf16_bits(1.0)
    case = DeviceCase(wl)
    case.run_step()
    torch.cuda.synchronize()
    got = case.out[i, g * G:(g + 1) * G].cpu().numpy()
    vj = torch.from_numpy(wl.values[lo + j, g].view(np.int16)).view(torch.bfloat16).float().numpy()
    for h in range(G):
        assert np.array_equal(got[h], vj), f"head {h}: output is not exactly v[{j}]"


@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("position", [0, 31, 32, 511, 512, 1000, "last"])
def test_one_hot_probe_fp8_group8(block_size, position):
    """FP8 KV, eight query heads per kv head: a key whose score beats every
    other by far more than 200 selects its dequantized value exactly."""
    lens = [700, 1037, 33]
    wl = build_decode_workload("probe8", 8, seq_lens=lens, num_heads=64, num_kv_heads=8, head_dim=128,
                               block_size=block_size, kv_dtype="fp8_e4m3", q_dtype="bf16", spare_blocks=4,
                               num_copy_pairs=2, partition_size=512)
    i, g, G, T = 1, 5, 8, 1037
    j = T - 1 if position == "last" else position
    lo = int(wl.token_offsets[i])
    wl.keys[lo:lo + T, g, 0] = 0
    wl.step_keys_src[i, g, 0] = 0
    if j == T - 1:
        wl.step_keys_src[i, g, 0] = _bf16_bits(1.0e6)  # saturates to the largest code, 448
    else:
        wl.keys[lo + j, g, 0] = 0x7E  # 448
    wl.q[i, g * G:(g + 1) * G, :] = 0
    wl.q[i, g * G:(g + 1) * G, 0] = _bf16_bits(16384.0)
    case = DeviceCase(wl)
    case.run_step()
    torch.cuda.synchronize()
    got = case.out[i, g * G:(g + 1) * G].cpu().numpy()
    kc, vc = oracle_pools(wl)
    blk = int(wl.block_tables[i, j // block_size])
    assert oracle.decode_elements(kc[blk, g, j % block_size, :1], "fp8_e4m3")[0] == 448.0
    vj = (oracle.decode_elements(vc[blk, g, j % block_size], "fp8_e4m3") * np.float64(wl.v_scale[g])).astype(
        np.float32)
    for h in range(G):
        assert np.array_equal(got[h], vj), f"head {h}: output is not exactly v[{j}]"


@pytest.mark.parametrize("kv,q,heads,kv_heads,block", [
    ("fp8_e4m3", "bf16", 64, 8, 16),
    ("fp8_e4m3", "bf16", 64, 8, 32),
    ("bf16", "bf16", 32, 8, 16),
    ("f16", "f16", 8, 8, 16),
])
def test_out_of_range_block_id_gives_nan_row(kv, q, heads, kv_heads, block):
    """A block id outside the pool (too large, or negative) is never used as an
    address: its sequence gets rows of NaN and the other rows are unaffected."""
    lens = [1500, 2100, 700, 1200, 333]
    wl = build_decode_workload(f"badid_{kv}_{heads}_{block}", 11, seq_lens=lens, num_heads=heads,
                               num_kv_heads=kv_heads, head_dim=128, block_size=block, kv_dtype=kv, q_dtype=q,
                               spare_blocks=4, num_copy_pairs=2, partition_size=512)
    case = DeviceCase(wl)
    case.run_cache_ops()
    bt = case.block_tables.clone()
    bt[1, 40] = wl.num_blocks + 7  # inside a middle partition of sequence 1
    bt[2, 5] = -3                  # inside the first partition of sequence 2
    case.decode(block_tables=bt)
    torch.cuda.synchronize()
    got = out_as_f64(case.out)
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all(), "rows with a bad block id must be NaN"
    kc, vc = oracle_pools(wl)
    rows = [0, 3, 4]
    want = oracle_out(wl, kc, vc, rows=rows)
    assert_close(got[rows], want, TOL[kv], f"rows next to bad ids ({kv}, B={block})")
