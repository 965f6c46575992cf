"""pa_decode_append on the GPU: storing each sequence's newest token and
decoding in one call gives bitwise the pools and outputs of
pa_reshape_and_cache followed by pa_decode, both for the shapes whose
partition kernel stores the token itself (GQA-4, bf16/f16) and for the others
(a copy kernel first), over lengths that put the new token at every kind of
position: the first row of a block, the last row, a one-token sequence, a
partition of more than 64 blocks.  The reference path is checked against the
oracle by the other parity tests; one case here is checked against it too."""

import numpy as np
import pytest
import torch

import paged_kv_cache_142_amd as pa
import workloads
from gpu_util import TOL, DeviceCase, assert_close, oracle_out, oracle_pools, out_as_f64

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 100, 511, 512, 513, 1500, 2049, 0, 4000]


def _bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def _edge(kv, q, heads, kv_heads, dim, block, partition_size):
    return workloads.build_decode_workload(
        f"append_edge_{kv}_{heads}_{kv_heads}_{dim}_{block}_{partition_size}", 31, seq_lens=EDGE_LENS,
        num_heads=heads, num_kv_heads=kv_heads, head_dim=dim, block_size=block, kv_dtype=kv, q_dtype=q,
        spare_blocks=4, num_copy_pairs=0, partition_size=partition_size)


def _compare(wl):
    print(f"[case] append {wl.name}: N={wl.num_seqs} H={wl.num_heads}/{wl.num_kv_heads} d={wl.head_dim} "
          f"B={wl.block_size} P={wl.partition_size} kv={wl.kv_dtype}", flush=True)
    kvd = wl.kv_dtype if wl.kv_dtype == "fp8_e4m3" else None
    results = []
    for fused_call in (False, True):
        case = DeviceCase(wl)  # pools hold every token but each sequence's newest
        keys = case.keys.index_select(0, case.step).contiguous()
        values = case.values.index_select(0, case.step).contiguous()
        if len(case.step) != wl.num_seqs:  # empty sequences have no row: scatter only the others
            full_k = torch.zeros((wl.num_seqs,) + tuple(keys.shape[1:]), dtype=keys.dtype, device="cuda")
            full_v = torch.zeros_like(full_k)
            has = torch.from_numpy(np.nonzero(wl.seq_lens > 0)[0]).cuda()
            full_k[has] = keys
            full_v[has] = values
        else:
            full_k, full_v = keys, values
        if fused_call:
            pa.pa_decode_append(**case.decode_args(), key=full_k, value=full_v)
        else:
            pa.pa_reshape_and_cache(keys, values, case.k_cache, case.v_cache, case.step_slots, kv_dtype=kvd)
            case.decode()
        torch.cuda.synchronize()
        results.append((_bytes(case.out), _bytes(case.k_cache), _bytes(case.v_cache), case))
    (o0, k0, v0, _), (o1, k1, v1, case) = results
    assert np.array_equal(k0, k1), "K pool differs from scatter + decode"
    assert np.array_equal(v0, v1), "V pool differs from scatter + decode"
    assert np.array_equal(o0, o1), "output differs from scatter + decode"
    return case


@pytest.mark.parametrize("kv,q,heads,kv_heads,dim,block,P", [
    ("bf16", "bf16", 32, 8, 128, 16, 256),    # GQA-4 kernel stores the token
    ("bf16", "bf16", 32, 8, 128, 16, 2048),   # a partition of 128 blocks
    ("f16", "f16", 32, 8, 128, 32, 512),
    ("bf16", "bf16", 16, 4, 64, 16, 512),
    ("f16", "f16", 16, 16, 128, 16, 512),     # G = 1: copy kernel first
    ("bf16", "bf16", 64, 8, 128, 32, 512),    # G = 8
    ("f32", "f32", 8, 4, 64, 16, 256),
    ("fp8_e4m3", "bf16", 64, 8, 128, 16, 512),
])
def test_append_matches_scatter_then_decode(kv, q, heads, kv_heads, dim, block, P):
    _compare(_edge(kv, q, heads, kv_heads, dim, block, P))


def test_append_gqa_workload_and_oracle():
    wl = workloads.gqa(4, num_seqs=20, max_len=3000, partition_size=768)
    case = _compare(wl)
    kc, vc = oracle_pools(wl)
    assert_close(out_as_f64(case.out), oracle_out(wl, kc, vc), TOL["bf16"], "append vs oracle")


def test_append_plan_kernel_order():
    # more than 64 sequences: the work order comes from the plan kernel
    _compare(workloads.gqa(5, num_seqs=90, max_len=1200, partition_size=256))


@pytest.mark.parametrize("heads,kv_heads", [(32, 8), (16, 16)])
def test_append_invalid_last_block_stores_nothing(heads, kv_heads):
    """A sequence whose last block id lies outside the pool gets a NaN row and
    no store; the other sequences are unaffected (fused and copy-kernel paths)."""
    wl = workloads.build_decode_workload(f"append_bad_{heads}_{kv_heads}", 33, seq_lens=[300, 40, 1000, 17],
                                         num_heads=heads, num_kv_heads=kv_heads, head_dim=128, block_size=16,
                                         kv_dtype="bf16", q_dtype="bf16", spare_blocks=4, num_copy_pairs=0,
                                         partition_size=256)
    print(f"[case] append with an out-of-pool block, H={heads}/{kv_heads}", flush=True)
    case = DeviceCase(wl)
    torch.cuda.synchronize()
    before_k, before_v = _bytes(case.k_cache), _bytes(case.v_cache)
    bad = wl.block_tables.copy()
    bad[2, (1000 - 1) // 16] = wl.num_blocks + 5
    keys = case.keys.index_select(0, case.step).contiguous()
    values = case.values.index_select(0, case.step).contiguous()
    pa.pa_decode_append(**case.decode_args(block_tables=torch.from_numpy(bad).cuda()), key=keys, value=values)
    torch.cuda.synchronize()
    out = out_as_f64(case.out)
    assert np.isnan(out[2]).all() and np.isfinite(out[[0, 1, 3]]).all()
    # only the three valid sequences' new rows changed in the pools
    slots = set()
    for i in (0, 1, 3):
        T = int(wl.seq_lens[i])
        slots.add(int(wl.block_tables[i, (T - 1) // 16]) * 16 + (T - 1) % 16)
    for before, after in ((before_k, _bytes(case.k_cache)), (before_v, _bytes(case.v_cache))):
        elems = np.nonzero(after.reshape(-1).view(np.uint16) != before.reshape(-1).view(np.uint16))[0]
        blk = elems // (kv_heads * 16 * 128)
        row = (elems % (16 * 128)) // 128
        assert len(elems) == len(slots) * kv_heads * 128
        assert set((blk * 16 + row).tolist()) == slots


def _shared_prefix_append(heads, kv_heads, fmt, block, P, groups, bitwise_out=True):
    """pa_decode_shared_prefix given each sequence's newest token against the
    same call over pools that already hold the tokens: bitwise equal pools,
    and outputs bitwise equal (the same kernels run) or, when the calls share
    differently, each within tolerance of the oracle."""
    from test_gpu_shared_prefix import _grouped_case
    from gpu_util import poison_device, to_device

    lens, tables, starts, prefixes, hk, hv, q = _grouped_case(41, num_heads=heads, num_kv_heads=kv_heads,
                                                              head_dim=128, block_size=block, fmt=fmt, groups=groups)
    print(f"[case] shared-prefix decode with append H={heads}/{kv_heads} {fmt} B={block} P={P} "
          f"groups={[(p, m) for p, m in groups]}", flush=True)
    N, H, d = q.shape
    msl = int(lens.max())
    last_blk = np.array([tables[i, (int(T) - 1) // block] for i, T in enumerate(lens)])
    last_row = (lens - 1) % block
    new_k = np.stack([hk[b, :, r, :] for b, r in zip(last_blk, last_row)])
    new_v = np.stack([hv[b, :, r, :] for b, r in zip(last_blk, last_row)])
    grp = dict(group_start=torch.from_numpy(starts).cuda(), group_prefix=torch.from_numpy(prefixes).cuda(),
               max_group_size=int(np.diff(starts).max()), max_prefix_len=int(prefixes.max()))
    outs, pools = [], []
    for append in (False, True):
        kc, vc = to_device(hk, fmt), to_device(hv, fmt)
        if append:  # the newest rows are not in the pool yet
            for b, r in zip(last_blk, last_row):
                kc[int(b), :, int(r), :] = float("nan")
                vc[int(b), :, int(r), :] = float("nan")
        out = poison_device((N, H, d), "f32")
        ws = torch.empty(pa.pa_decode_workspace_size(N, H, d, msl, P), dtype=torch.uint8, device="cuda")
        extra = dict(key=to_device(new_k, fmt), value=to_device(new_v, fmt)) if append else {}
        pa.pa_decode_shared_prefix(out, to_device(q, fmt), kc, vc, torch.from_numpy(tables).cuda(),
                                   torch.from_numpy(lens).cuda(), msl, 1.0 / np.sqrt(d), P, ws, **grp, **extra)
        torch.cuda.synchronize()
        outs.append(_bytes(out))
        pools.append((_bytes(kc), _bytes(vc)))
    assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])
    if bitwise_out:
        assert np.array_equal(outs[0], outs[1])
        return
    import oracle
    expect = oracle.paged_decode(q, fmt, hk, hv, fmt, tables, lens, block, float(np.float32(1.0 / np.sqrt(d))))
    for o in outs:
        got = o.view(np.float32).reshape(N, H, d).astype(np.float64)
        assert_close(got, expect, TOL[fmt], "shared-prefix decode with append vs oracle")


@pytest.mark.parametrize("heads,kv_heads,fmt,block,P", [
    (32, 8, "bf16", 16, 256),   # G = 4: the suffix partitions' kernel stores the token
    (16, 16, "bf16", 16, 256),  # G = 1: copy kernel first
    (32, 4, "f16", 32, 512),    # G = 8
    (32, 8, "bf16", 16, 1024),  # 64 blocks per partition: the most the partition kernel stores the token for
    (32, 8, "f16", 32, 512),    # G = 4 combined launch, f16, 32-token blocks
    (32, 8, "bf16", 32, 256),   # G = 4 combined launch, bf16, 32-token blocks
])
def test_shared_prefix_decode_with_append(heads, kv_heads, fmt, block, P):
    groups = [(2 * P, [2 * P + 5, 2 * P + 90, 2 * P + 1]), (P + 2 * block, [P + 2 * block + 1, P + 100]),
              (0, [40, 300])]
    _shared_prefix_append(heads, kv_heads, fmt, block, P, groups)


@pytest.mark.parametrize("heads,kv_heads", [(32, 8), (16, 16)])
def test_shared_prefix_append_member_holding_only_shared_partitions(heads, kv_heads):
    """A group whose only member's newest token falls inside its shared
    partitions (length exactly the shared partitions; the contract forbids
    it): the member is computed alone, so its newest token is stored and its
    row equals the one over a pool that already holds the token."""
    P, block = 256, 16
    groups = [(2 * P, [2 * P]), (2 * P, [2 * P + 7, 2 * P + 40]), (P, [3 * P])]
    _shared_prefix_append(heads, kv_heads, "bf16", block, P, groups, bitwise_out=False)
