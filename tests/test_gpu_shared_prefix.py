"""Shared-prefix beam workload on the GPU: 8 prompts x 6 beams share the
prompt's blocks through ref-counted tables; each beam's first write into the
partially filled boundary block triggers copy-on-write (``pa_copy_blocks``)
before its suffix is scattered; odd sequences carry queries whose logits
reach +-80.

The expected output is the oracle's plain attention over each beam's
LOGICAL rows (prompt followed by its own suffix), independent of the block
manager's placement decisions; the oracle's paged gather over the block
manager's tables and the host copy of the pool must agree with it too.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_142_amd as pa
import workloads
from workloads.generators import round_to_storage
from gpu_util import TOL, assert_close, out_as_f64, poison_device, poison_host, to_device, to_host_raw

pytestmark = pytest.mark.gpu


def _assemble(wl, seed):
    """Block manager + device pool after prompt fill, fork, CoW and suffix writes."""
    B, Hkv, d = wl.block_size, wl.num_kv_heads, wl.head_dim
    prompt_blocks = -(-wl.prompt_len // B)
    longest_suffix = max(256, int(wl.suffix_lens.max()))
    pool = wl.num_prompts * prompt_blocks + wl.num_seqs * (-(-longest_suffix // B) + 2) + 8
    bm = pa.BlockManager(pool, B, free_order=np.random.default_rng(seed).permutation(pool))
    shape = (pool, Hkv, B, d)
    kc, vc = poison_device(shape, "bf16"), poison_device(shape, "bf16")
    hk, hv = poison_host(shape, "bf16"), poison_host(shape, "bf16")

    # prompts
    beams = []
    for k in range(wl.num_prompts):
        s = bm.add_sequence()
        slots = np.array([bm.append_slot(s)[0] for _ in range(wl.prompt_len)], np.int64)
        pa.pa_reshape_and_cache(to_device(wl.prompt_keys[k], "bf16"), to_device(wl.prompt_values[k], "bf16"),
                                kc, vc, torch.from_numpy(slots).cuda())
        oracle.reshape_and_cache(hk, hv, wl.prompt_keys[k], wl.prompt_values[k], slots, B)
        beams += bm.fork(s, wl.beams)
        bm.free_sequence(s)
    bm.check_invariants()

    # suffixes: collect CoW pairs and slots first, copy, then scatter
    pairs, slots, rows_k, rows_v = [], [], [], []
    for n, s in enumerate(beams):
        for t in range(int(wl.suffix_lens[n])):
            slot, pair = bm.append_slot(s)
            if pair is not None:
                pairs.append(pair)
            slots.append(slot)
        rows_k.append(wl.suffix_keys[n])
        rows_v.append(wl.suffix_values[n])
    bm.check_invariants()
    pairs = np.array(pairs, np.int64).reshape(-1, 2)
    dsts = pairs[:, 1]
    assert len(set(dsts.tolist())) == len(dsts) and not set(dsts.tolist()) & set(pairs[:, 0].tolist())
    if len(pairs):
        pa.pa_copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    oracle.copy_blocks(hk, hv, pairs)
    slots = np.array(slots, np.int64)
    sk, sv = np.concatenate(rows_k), np.concatenate(rows_v)
    if len(slots):
        pa.pa_reshape_and_cache(to_device(sk, "bf16"), to_device(sv, "bf16"), kc, vc,
                                torch.from_numpy(slots).cuda())
    oracle.reshape_and_cache(hk, hv, sk, sv, slots, B)
    tables = bm.tables_array(beams)
    for n, s in enumerate(beams):
        assert bm.seq_len(s) == wl.prompt_len + int(wl.suffix_lens[n])
    return bm, beams, kc, vc, hk, hv, tables, pairs


@pytest.mark.parametrize("prompt_len", [1032, 1024])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_shared_prefix_beams(prompt_len, seed):
    wl = workloads.shared_prefix(seed, prompt_len=prompt_len)
    print(f"[case] shared_prefix prompt={prompt_len} seed={seed} seqs={wl.num_seqs}", flush=True)
    bm, beams, kc, vc, hk, hv, tables, pairs = _assemble(wl, seed)
    if prompt_len % wl.block_size:
        writers = int((wl.suffix_lens > 0).reshape(wl.num_prompts, wl.beams).sum())
        assert 0 < len(pairs) <= writers
    else:
        assert len(pairs) == 0  # no partially filled shared block: nothing to copy
    lens = wl.seq_lens()
    msl = int(lens.max())
    q = to_device(wl.q, "bf16")
    out = poison_device((wl.num_seqs, wl.num_heads, wl.head_dim), "f32")
    ws = torch.empty(pa.pa_decode_workspace_size(wl.num_seqs, wl.num_heads, wl.head_dim, msl, 512),
                     dtype=torch.uint8, device="cuda")
    pa.pa_decode(out, q, kc, vc, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), msl,
                 float(wl.scale), 512, ws)
    torch.cuda.synchronize()

    assert np.array_equal(to_host_raw(kc, "bf16"), hk) and np.array_equal(to_host_raw(vc, "bf16"), hv)
    paged = oracle.paged_decode(wl.q, "bf16", hk, hv, "bf16", tables, lens, wl.block_size, float(wl.scale))
    logical = np.zeros_like(paged)
    G = wl.num_heads // wl.num_kv_heads
    qf = oracle.decode_elements(wl.q, "bf16")
    for s in range(wl.num_seqs):
        keys = oracle.decode_elements(wl.logical_rows(s, "k"), "bf16")
        vals = oracle.decode_elements(wl.logical_rows(s, "v"), "bf16")
        for h in range(wl.num_heads):
            logical[s, h] = oracle.dense_attention(qf[s, h], keys[:, h // G], vals[:, h // G], float(wl.scale))
    np.testing.assert_allclose(paged, logical, rtol=0, atol=1e-12)
    got = out_as_f64(out)
    assert_close(got, logical, TOL["bf16"], f"shared_prefix p={prompt_len}")
    assert_close(got[wl.extreme], logical[wl.extreme], TOL["bf16"], "extreme-logit half")


def _beam_groups(wl):
    """Groups of the beams of each prompt and the tokens their tables share:
    the prompt's whole blocks (a partially filled boundary block may have been
    copied on write)."""
    starts = torch.arange(0, wl.num_seqs + 1, wl.beams, dtype=torch.int32, device="cuda")
    shared = (wl.prompt_len // wl.block_size) * wl.block_size
    prefix = torch.full((wl.num_prompts,), shared, dtype=torch.int32, device="cuda")
    return starts, prefix, shared


@pytest.mark.parametrize("prompt_len,partition_size", [(1032, 512), (1024, 512), (1032, 256), (1024, 256), (1024, 1024)])
def test_shared_prefix_decode_beams(prompt_len, partition_size):
    """pa_decode_shared_prefix over the forked beams: the oracle's plain
    attention over each beam's logical rows, and pa_decode's output."""
    seed = 3
    wl = workloads.shared_prefix(seed, prompt_len=prompt_len)
    print(f"[case] shared_prefix_decode prompt={prompt_len} P={partition_size}", flush=True)
    bm, beams, kc, vc, hk, hv, tables, pairs = _assemble(wl, seed)
    lens = wl.seq_lens()
    msl = int(lens.max())
    starts, prefix, shared = _beam_groups(wl)
    q = to_device(wl.q, "bf16")
    t_dev, l_dev = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    ws = torch.empty(pa.pa_decode_workspace_size(wl.num_seqs, wl.num_heads, wl.head_dim, msl, partition_size),
                     dtype=torch.uint8, device="cuda")
    out = poison_device((wl.num_seqs, wl.num_heads, wl.head_dim), "f32")
    pa.pa_decode_shared_prefix(out, q, kc, vc, t_dev, l_dev, msl, float(wl.scale), partition_size, ws,
                               group_start=starts, group_prefix=prefix, max_group_size=wl.beams,
                               max_prefix_len=shared)
    plain = poison_device((wl.num_seqs, wl.num_heads, wl.head_dim), "f32")
    pa.pa_decode(plain, q, kc, vc, t_dev, l_dev, msl, float(wl.scale), partition_size, ws)
    torch.cuda.synchronize()
    expect = oracle.paged_decode(wl.q, "bf16", hk, hv, "bf16", tables, lens, wl.block_size, float(wl.scale))
    got = out_as_f64(out)
    assert_close(got, expect, TOL["bf16"], "shared-prefix decode")
    assert_close(got[wl.extreme], expect[wl.extreme], TOL["bf16"], "extreme-logit half")
    assert_close(got, out_as_f64(plain), TOL["bf16"], "shared-prefix decode vs pa_decode")


def _grouped_case(seed, *, num_heads, num_kv_heads, head_dim, block_size, fmt, groups):
    """Sequences in groups whose members' tables name the same first blocks.

    ``groups``: list of ``(prefix_tokens, member_lengths)``.  Every member's
    first ``ceil(min(prefix, T) / B)`` table entries are the group's shared
    block ids, the rest private ones; block ids are scattered over the pool
    by a seeded permutation.  Pool contents and queries are seeded standard
    normal draws rounded to ``fmt``.
    """
    rng = np.random.default_rng(seed)
    B = block_size
    lens, rows, starts, prefixes = [], [], [0], []
    next_id = 0
    for pre, members in groups:
        nshared = -(-pre // B)
        shared_ids = list(range(next_id, next_id + nshared))
        next_id += nshared
        for T in members:
            nb = -(-T // B)
            own = min(nb, nshared)
            row = shared_ids[:own] + list(range(next_id, next_id + nb - own))
            next_id += nb - own
            rows.append(row)
            lens.append(T)
        starts.append(len(lens))
        prefixes.append(pre)
    num_blocks = next_id + 5
    perm = rng.permutation(num_blocks)
    max_blocks = max(len(r) for r in rows) if rows else 1
    tables = np.full((len(rows), max_blocks), -1, np.int32)
    for i, r in enumerate(rows):
        tables[i, :len(r)] = perm[np.array(r, np.int64)]
    shape = (num_blocks, num_kv_heads, B, head_dim)
    hk = round_to_storage(rng.standard_normal(shape, dtype=np.float32), fmt)
    hv = round_to_storage(rng.standard_normal(shape, dtype=np.float32), fmt)
    q = round_to_storage(rng.standard_normal((len(lens), num_heads, head_dim), dtype=np.float32), fmt)
    return (np.array(lens, np.int32), tables, np.array(starts, np.int32), np.array(prefixes, np.int32), hk, hv, q)


def _run_grouped(case, *, fmt, block_size, partition_size, max_group_size=None, max_prefix_len=None,
                 out_fmt="f32", check_plain=True, ws=None):
    lens, tables, starts, prefixes, hk, hv, q = case
    N, H, d = q.shape
    msl = int(lens.max())
    scale = 1.0 / np.sqrt(d)
    sizes = np.diff(starts)
    mgs = int(sizes.max()) if max_group_size is None else max_group_size
    mpl = int(prefixes.max()) if max_prefix_len is None else max_prefix_len
    kc, vc, qd = to_device(hk, fmt), to_device(hv, fmt), to_device(q, fmt)
    t_dev, l_dev = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    if ws is None:
        ws = torch.empty(pa.pa_decode_workspace_size(N, H, d, msl, partition_size), dtype=torch.uint8,
                         device="cuda")
    out = poison_device((N, H, d), out_fmt)
    pa.pa_decode_shared_prefix(out, qd, kc, vc, t_dev, l_dev, msl, scale, partition_size, ws,
                               group_start=torch.from_numpy(starts).cuda(),
                               group_prefix=torch.from_numpy(prefixes).cuda(), max_group_size=mgs,
                               max_prefix_len=mpl)
    plain = poison_device((N, H, d), out_fmt)
    if check_plain:
        pa.pa_decode(plain, qd, kc, vc, t_dev, l_dev, msl, scale, partition_size, ws)
    torch.cuda.synchronize()
    expect = oracle.paged_decode(q, fmt, hk, hv, fmt, tables, lens, block_size, scale)
    tol = max(TOL[fmt], TOL[out_fmt])
    got = out_as_f64(out)
    assert_close(got, expect, tol, "shared-prefix decode vs oracle")
    if check_plain:
        assert_close(got, out_as_f64(plain), tol, "shared-prefix decode vs pa_decode")


def _mixed_groups(rng, P, n_target):
    """Groups that exercise every sharing rule: no prefix, prefixes shorter
    than one partition, not a multiple of it, members shorter than the
    shared partitions, a member of exactly one partition, a short leader,
    a single-member group, an empty group, and groups wider than one tile."""
    g = []
    g.append((3 * P, [3 * P + int(x) for x in rng.integers(1, 400, 5)]))           # 3 whole partitions
    g.append((2 * P + 37, [2 * P + 37 + int(x) for x in rng.integers(0, 300, 4)]))  # 2 whole + tail
    g.append((P - 1, [P - 1 + int(x) for x in rng.integers(1, 200, 3)]))            # below one partition
    g.append((0, [int(x) for x in rng.integers(1, 3 * P, 2)]))                      # nothing shared
    g.append((2 * P, [2 * P + 10, P + 3, 2 * P, 40, 2 * P + 700]))                  # short members
    g.append((P, [P, P + 1, P]))                                                    # single-partition members
    g.append((2 * P, [P + 5, 2 * P + 9, 2 * P + 100]))                              # short leader: none shared
    g.append((2 * P, [2 * P + 3]))                                                  # one member
    g.append((P, []))                                                               # empty group
    n = sum(len(m) for _, m in g)
    wide = max(n_target - n, 20)
    g.append((P + P // 2, [P + P // 2 + int(x) for x in rng.integers(0, 2 * P, wide)]))  # wider than a tile
    return g


@pytest.mark.parametrize("heads,kv_heads,fmt,block,P,n", [
    (32, 8, "bf16", 16, 512, 80),   # G = 4, plan-kernel work order (more than 64 sequences)
    (32, 8, "bf16", 16, 512, 60),   # G = 4, in-kernel work order
    (32, 4, "f16", 32, 256, 60),    # G = 8
    (16, 16, "bf16", 16, 256, 70),  # G = 1
    (16, 8, "bf16", 32, 512, 50),   # G = 2
    (32, 8, "f16", 32, 512, 60),    # G = 4 combined launch, f16, 32-token blocks
    (32, 8, "bf16", 32, 256, 60),   # G = 4 combined launch, bf16, 32-token blocks
])
def test_shared_prefix_decode_groups(heads, kv_heads, fmt, block, P, n):
    seed = heads * 7 + kv_heads + block + P + n
    rng = np.random.default_rng(seed)
    groups = _mixed_groups(rng, P, n)
    print(f"[case] shared_prefix_groups H={heads}/{kv_heads} {fmt} B={block} P={P} "
          f"seqs={sum(len(m) for _, m in groups)}", flush=True)
    case = _grouped_case(seed, num_heads=heads, num_kv_heads=kv_heads, head_dim=128, block_size=block, fmt=fmt,
                         groups=groups)
    _run_grouped(case, fmt=fmt, block_size=block, partition_size=P)


def test_shared_prefix_decode_grid_bounds():
    """max_group_size / max_prefix_len below the real ones: the members and
    partitions past them are computed alone, with the same result."""
    P = 512
    rng = np.random.default_rng(11)
    groups = [(3 * P, [3 * P + int(x) for x in rng.integers(0, 300, 40)]),
              (2 * P, [2 * P + int(x) for x in rng.integers(0, 300, 7)])]
    case = _grouped_case(11, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, fmt="bf16", groups=groups)
    print("[case] shared_prefix grid bounds", flush=True)
    _run_grouped(case, fmt="bf16", block_size=16, partition_size=P, max_group_size=20, max_prefix_len=P + 100)
    _run_grouped(case, fmt="bf16", block_size=16, partition_size=P, max_group_size=0, check_plain=False)
    _run_grouped(case, fmt="bf16", block_size=16, partition_size=P, max_prefix_len=P - 1, check_plain=False)


def test_shared_prefix_decode_bf16_out_and_fallback_shapes():
    """bf16 output rows; head_dim 64 (no matrix-core tile) runs pa_decode."""
    P = 256
    rng = np.random.default_rng(5)
    groups = [(2 * P, [2 * P + int(x) for x in rng.integers(0, 300, 9)]), (P, [P, P + 70, 3 * P])]
    print("[case] shared_prefix bf16 out / d=64", flush=True)
    case = _grouped_case(5, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, fmt="bf16", groups=groups)
    _run_grouped(case, fmt="bf16", block_size=16, partition_size=P, out_fmt="bf16")
    case = _grouped_case(6, num_heads=32, num_kv_heads=8, head_dim=64, block_size=16, fmt="bf16", groups=groups)
    _run_grouped(case, fmt="bf16", block_size=16, partition_size=P)


def test_shared_prefix_decode_regrouped_workspace():
    """Two calls on one workspace with different groupings: the second call's
    skips replace the first's everywhere."""
    P = 512
    rng = np.random.default_rng(9)
    lens_a = [3 * P + int(x) for x in rng.integers(0, 200, 12)]
    case1 = _grouped_case(9, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, fmt="bf16",
                          groups=[(3 * P, lens_a)])
    lens, tables, starts, prefixes, hk, hv, q = case1
    print("[case] shared_prefix regrouped", flush=True)
    ws = torch.empty(pa.pa_decode_workspace_size(len(lens), 32, 128, int(lens.max()), P), dtype=torch.uint8,
                     device="cuda")
    _run_grouped(case1, fmt="bf16", block_size=16, partition_size=P, check_plain=False, ws=ws)
    # same pool and tables, now as singletons (nothing shared): stale skips must not survive
    N = len(lens)
    case2 = (lens, tables, np.arange(N + 1, dtype=np.int32), np.zeros(N, np.int32), hk, hv, q)
    _run_grouped(case2, fmt="bf16", block_size=16, partition_size=P, max_prefix_len=3 * P, check_plain=False,
                 ws=ws)


def test_shared_prefix_decode_long_prompt():
    """Two 4096-token prompts forked into 4 beams each: eight shared
    partitions per group, computed once, then merged with each beam's own."""
    wl = workloads.shared_prefix(4, prompt_len=4096, num_prompts=2, beams=4, max_suffix=600)
    print("[case] shared_prefix_decode prompt=4096 prompts=2 beams=4", flush=True)
    bm, beams, kc, vc, hk, hv, tables, pairs = _assemble(wl, 4)
    lens = wl.seq_lens()
    msl = int(lens.max())
    starts, prefix, shared = _beam_groups(wl)
    q = to_device(wl.q, "bf16")
    t_dev, l_dev = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    ws = torch.empty(pa.pa_decode_workspace_size(wl.num_seqs, wl.num_heads, wl.head_dim, msl, 512),
                     dtype=torch.uint8, device="cuda")
    out = poison_device((wl.num_seqs, wl.num_heads, wl.head_dim), "f32")
    pa.pa_decode_shared_prefix(out, q, kc, vc, t_dev, l_dev, msl, float(wl.scale), 512, ws,
                               group_start=starts, group_prefix=prefix, max_group_size=wl.beams,
                               max_prefix_len=shared)
    torch.cuda.synchronize()
    expect = oracle.paged_decode(wl.q, "bf16", hk, hv, "bf16", tables, lens, wl.block_size, float(wl.scale))
    got = out_as_f64(out)
    assert_close(got, expect, TOL["bf16"], "shared-prefix decode, 4096-token prompts")
    assert_close(got[wl.extreme], expect[wl.extreme], TOL["bf16"], "extreme-logit half")
