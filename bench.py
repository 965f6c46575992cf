"""Benchmark of one decode step of the paged-attention hot path on one GPU.

A step is one pass of the whole path over the batch: the step's block
copies (``pa_copy_blocks``), the scatter of each sequence's new token into
the pool, and the decode itself.  Where one call can do the last two
(bf16/f16/f32 pools), the step is one ``pa_decode_append_cow`` call: its
partition launch also makes the copies and stores the tokens
(``--separate-cow``: ``pa_copy_blocks`` then ``pa_decode_append``).  The
grouped shared-prefix workloads run ``pa_copy_blocks`` then
``pa_decode_shared_prefix`` given the new tokens.  For FP8 pools (quantized
on write) it is the scatter (``pa_reshape_and_cache_fp8``), then
``pa_decode_append_cow`` without tokens: the copies in the matrix-core
partition launch, then the reduce (``--separate-cow``: ``pa_copy_blocks``,
``pa_decode_partition``, ``pa_decode_reduce``).
``step_calls`` in the output names them.
Inputs are resident in HBM before the timed region.  Throughput is the
effective KV bandwidth: sum_i T_i * 2 * H_kv * d * b_kv bytes per step.
By default two copies of the K/V pool alternate between steps, so that no
step finds the previous step's K/V in the 256 MB Infinity Cache (on MI355X
this costs about 1% against re-reading one pool; ``--pools 1`` for that).

Timing: ``--settle-ms`` of untimed steps (reported) and ``--warmup`` untimed
steps, then exactly ``--steps`` steps between one event pair, with events at
up to ten batch boundaries inside for the median and p10/p90 over batches.
Then each call alone, ``--steps`` times back to back between one event pair
(``kernels_us``; ``decode_alone_*`` is ``pa_decode``), from which the
roofline of the partition kernel is taken.

Prints one JSON line.  ``--gpus`` above 1 is refused: this path runs on one
GPU.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attn: effective KV GB/s (% of HBM peak), µs/step, seqs/s"
KERNEL_SOURCES = ["paged_kv_cache_142_amd/csrc/pa_decode_kernel.hpp", "paged_kv_cache_142_amd/csrc/pa_decode_gqa.hpp",
                  "paged_kv_cache_142_amd/csrc/pa_common.hpp", "paged_kv_cache_142_amd/csrc/pa_decode_bf16.hip",
                  "paged_kv_cache_142_amd/csrc/pa_decode_api.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partition_gqa_traffic.json")
# shared_prefix_long: 8 prompts of this many tokens, 6 beams each; the prompts'
# K/V (268 MB, twice with two pool copies) exceed the 256 MB Infinity Cache
LONG_PROMPT = 8192


def _parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5, help="untimed steps after the settle phase")
    p.add_argument("--config", default="gqa",
                   choices=["gqa", "mha", "long_fp8", "long_fp8_b32", "tiny", "shared_prefix", "shared_prefix_cow",
                            "shared_prefix_grouped", "shared_prefix_cow_grouped", "shared_prefix_long",
                            "shared_prefix_long_grouped", "prefill", "prefill_chunk"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--partition-size", type=int, default=None,
                   help="split-KV partition size (default: the fastest in same-box sweeps where the workload "
                        "leaves it open: 832 for gqa (512..1024 tried), 256 for shared_prefix_grouped and "
                        "shared_prefix_cow_grouped (128..512 tried), 1024 for shared_prefix_long_grouped "
                        "(256..1024 tried); 512 for the other workloads, the pages' value for the long-context "
                        "case)")
    p.add_argument("--settle-ms", type=float, default=1000.0,
                   help="before --warmup, run untimed steps for at least this many milliseconds (reported in the "
                        "line). On MI355X the clocks rise from idle over the first second of load; with 5 warm-up "
                        "steps alone, per-call times drifted by about 5%% between the loops of one run")
    p.add_argument("--identity-tables", action="store_true",
                   help="relabel physical blocks so that every sequence's blocks are consecutive (the paging "
                        "indirection with a trivial layout)")
    p.add_argument("--paging-ab", action="store_true",
                   help="instead of the benchmark, time pa_decode with shuffled and with identity block tables, "
                        "alternating in one process")
    p.add_argument("--ab-rounds", type=int, default=15)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle baseline sample")
    p.add_argument("--pools", type=int, default=2,
                   help="copies of the K/V pool; step i uses copy i %% pools, so back-to-back steps read K/V that "
                        "the 256 MB Infinity Cache does not hold (1: every step re-reads the same pool)")
    p.add_argument("--separate-cow", action="store_true",
                   help="issue the step's copy-on-write copies as a pa_copy_blocks launch before pa_decode_append "
                        "instead of inside pa_decode_append_cow")
    p.add_argument("--graph", action="store_true",
                   help="replay the step as a captured HIP graph (the four launches) instead of eager calls")
    p.add_argument("--swap-mib", type=int, default=0,
                   help="instead of the benchmark, time pa_swap_blocks moving this many MiB of blocks to pinned "
                        "host memory and back (host-link GB/s)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="instead of the benchmark, run a plain device copy of this many MiB per step "
                        "(reference for scaling the FETCH_SIZE/WRITE_SIZE counters)")
    return p.parse_args()


def copy_calibration(mib, steps):
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


def shared_prefix_step(seed, partition_size, prompt_len):
    """The shared-prefix beam workload as one decode step.

    8 prompts of ``prompt_len`` tokens, each forked into 6 beams by the host
    block manager (every prompt block shared, reference count 6), then each
    beam's suffix appended through it: the first write into a shared,
    partially filled boundary block takes a private copy (copy-on-write).
    The cached state before the step is what those copies and writes leave:
    each private boundary block holds the prompt's tail rows and the beam's
    own suffix.  The timed step scatters every beam's newest token, copies
    as many blocks as copy-on-write needed (into spare blocks no table
    references, so that repeating the step leaves the state unchanged) and
    decodes.  Odd beams carry queries whose logits reach +-80.
    """
    import paged_kv_cache_142_amd as pa
    import workloads
    from workloads.generators import DecodeWorkload
    sp = workloads.shared_prefix(seed, prompt_len=prompt_len)
    B = sp.block_size
    prompt_blocks = -(-prompt_len // B)
    live = sp.num_prompts * prompt_blocks + sp.num_seqs * (-(-256 // B) + 2) + 8
    bm = pa.BlockManager(live, B, free_order=np.random.default_rng(seed).permutation(live))
    beams, cow = [], []
    for k in range(sp.num_prompts):
        root = bm.add_sequence()
        for _ in range(prompt_len):
            bm.append_slot(root)
        beams += bm.fork(root, sp.beams)
        bm.free_sequence(root)
    for n, s in enumerate(beams):
        for _ in range(int(sp.suffix_lens[n])):
            _, pair = bm.append_slot(s)
            if pair is not None:
                cow.append(pair)
    bm.check_invariants()
    lens = np.array([bm.seq_len(s) for s in beams], np.int32)
    tables = bm.tables_array(beams)
    keys = np.concatenate([np.concatenate([sp.prompt_keys[n // sp.beams], sp.suffix_keys[n]]) for n in range(sp.num_seqs)])
    values = np.concatenate([np.concatenate([sp.prompt_values[n // sp.beams], sp.suffix_values[n]])
                             for n in range(sp.num_seqs)])
    offsets = np.zeros(sp.num_seqs + 1, np.int64)
    offsets[1:] = np.cumsum(lens.astype(np.int64))
    slots = np.concatenate([tables[i, np.arange(t) // B].astype(np.int64) * B + np.arange(t) % B
                            for i, t in enumerate(lens)])
    spare = np.arange(live, live + len(cow), dtype=np.int64)
    pairs = np.stack([np.array([c[0] for c in cow], np.int64), spare], axis=1) if cow else np.zeros((0, 2), np.int64)
    return DecodeWorkload(
        name=f"shared_prefix_{prompt_len}", seed=seed, kv_dtype=sp.kv_dtype, q_dtype=sp.q_dtype,
        num_seqs=sp.num_seqs, num_heads=sp.num_heads, num_kv_heads=sp.num_kv_heads, head_dim=sp.head_dim,
        block_size=B, num_blocks=live + len(cow), partition_size=partition_size, scale=sp.scale, seq_lens=lens,
        block_tables=tables, token_offsets=offsets, keys=keys, values=values, slots=slots, q=sp.q, k_scale=None,
        v_scale=None, copy_pairs=pairs)


def unique_kv_bytes(wl):
    """K+V bytes of the distinct cached tokens (a slot shared by several
    sequences counts once)."""
    return len(np.unique(wl.slots)) * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes


def swap_bandwidth(mib, steps):
    """Host-link rate of pa_swap_blocks: the gqa block shape (8 kv heads x
    16 rows x 128 bf16, 64 KiB of K+V per block), `mib` MiB of blocks moved
    device -> pinned host and back, in a seeded random block order."""
    import torch
    import paged_kv_cache_142_amd as pa
    per_block = 2 * 8 * 16 * 128 * 2
    n = max(1, mib * (1 << 20) // per_block)
    shape = (n, 8, 16, 128)
    kc = torch.randn(shape, device="cuda").to(torch.bfloat16)
    vc = torch.randn(shape, device="cuda").to(torch.bfloat16)
    hk = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    rng = np.random.default_rng(0)
    out_pairs = torch.from_numpy(np.stack([rng.permutation(n), rng.permutation(n)], 1).astype(np.int64)).cuda()
    in_pairs = out_pairs.flip(1).contiguous()
    times = {}
    for name, args in (("out", (kc, vc, hk, hv, out_pairs)), ("in", (hk, hv, kc, vc, in_pairs))):
        pa.pa_swap_blocks(*args)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            pa.pa_swap_blocks(*args)
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / steps * 1e-3
    byts = n * per_block
    print(json.dumps({"swap_blocks": n, "bytes_per_direction": byts,
                      "swap_out_GBs": round(byts / times["out"] / 1e9, 2),
                      "swap_in_GBs": round(byts / times["in"] / 1e9, 2),
                      "swap_out_ms": round(times["out"] * 1e3, 3), "swap_in_ms": round(times["in"] * 1e3, 3)}))


def prefill_flops(wl):
    """Algorithmic flops of one prefill step: for every query row at position
    p and query head, 2 d for the scores and 2 d for the values against each
    of the p + 1 keys it may see."""
    c = wl.cache
    total = 0
    for T, Q in zip(c.seq_lens.astype(np.int64), wl.query_lens.astype(np.int64)):
        first = T - Q + 1  # keys seen by the first query row
        total += (first + T) * Q // 2
    return int(total) * c.num_heads * 4 * c.head_dim


def run_prefill(args):
    """The prefill step: scatter of the chunk tokens' K/V, then pa_prefill."""
    import torch
    import paged_kv_cache_142_amd as pa
    import workloads
    chunk = None if args.config == "prefill" else 512
    wl = workloads.prefill(args.seed, chunk=chunk)
    c = wl.cache
    view = {"f16": torch.float16, "bf16": torch.bfloat16}

    def up(raw, fmt):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(view[fmt]).cuda()

    kc = torch.zeros(c.pool_shape(), dtype=view[c.kv_dtype], device="cuda")
    vc = torch.zeros_like(kc)
    keys, values = up(c.keys, c.kv_dtype), up(c.values, c.kv_dtype)
    slots = torch.from_numpy(c.slots).cuda()
    ctx = torch.from_numpy(wl.context_rows()).cuda()
    if len(ctx):
        pa.pa_reshape_and_cache(keys[ctx].contiguous(), values[ctx].contiguous(), kc, vc, slots[ctx].contiguous())
    ch = torch.from_numpy(wl.chunk_rows()).cuda()
    ck, cv, cs = keys[ch].contiguous(), values[ch].contiguous(), slots[ch].contiguous()
    del keys, values
    q = up(wl.q, c.q_dtype)
    out = torch.empty((wl.total_q, c.num_heads, c.head_dim), dtype=torch.float32, device="cuda")
    qs = torch.from_numpy(wl.query_start).cuda()
    tables = torch.from_numpy(c.block_tables).cuda()
    lens = torch.from_numpy(c.seq_lens).cuda()
    calls = [pa.prepared("pa_reshape_and_cache", ck, cv, kc, vc, cs),
             pa.prepared("pa_prefill", out, q, qs, kc, vc, tables, lens, c.max_seq_len, int(wl.query_lens.max()),
                         float(c.scale))]
    for _ in range(args.warmup):
        for call in calls:
            call()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        for call in calls:
            call()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    scatter_us = back_to_back(torch, calls[:1], args.steps)
    prefill_us = back_to_back(torch, calls[1:], args.steps)
    flops = prefill_flops(wl)
    tflops = flops / (prefill_us * 1e-6) / 1e12
    line = {
        "metric": "paged prefill attn: algorithmic TFLOP/s (causal), query tokens/s",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": c.kv_dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {c.num_seqs} seqs, sum T={int(c.seq_lens.sum())} (max {c.max_seq_len}), "
                               f"{wl.total_q} query tokens, {c.num_heads}/{c.num_kv_heads} heads, d={c.head_dim}, "
                               f"B={c.block_size}, {c.kv_dtype} K/V/q, f32 out; step = scatter of the query "
                               f"tokens' K/V + pa_prefill", "seed": wl.cache.seed,
                   "flops_per_step": flops, "query_tokens": wl.total_q},
        "query_tokens_per_s": round(wl.total_q / (ms * 1e-3), 1),
        "kernels_us": {"reshape_and_cache": round(scatter_us, 2), "prefill": round(prefill_us, 2)},
        "kernels_timing": "each call alone, back to back between one event pair",
        "roofline": {"kernel": "pa_prefill", "bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "note": "bf16 dense matrix-core peak; the kernel issues 34 matrix products per 32 "
                             "algorithmic ones (2 accrue the column sums of the rounded weights) and computes "
                             "the masked keys of the diagonal steps"},
    }
    print(json.dumps(line), flush=True)


def _workload(name, seed, partition_size):
    import workloads
    if partition_size is None:
        partition_size = {"gqa": 832, "shared_prefix_grouped": 256, "shared_prefix_cow_grouped": 256,
                          "shared_prefix_long_grouped": 1024}.get(name, 512)
    if name.startswith("shared_prefix_cow"):
        return shared_prefix_step(seed, partition_size, 1032)
    if name.startswith("shared_prefix_long"):
        return shared_prefix_step(seed, partition_size, LONG_PROMPT)
    if name.startswith("shared_prefix"):
        return shared_prefix_step(seed, partition_size, 1024)
    if name == "gqa":
        return workloads.gqa(seed, partition_size=partition_size)
    if name == "mha":
        return workloads.mha(seed, partition_size=partition_size)
    if name == "long_fp8":
        return workloads.long_fp8(seed, block_size=16, partition_size=partition_size)
    if name == "long_fp8_b32":
        return workloads.long_fp8(seed, block_size=32, partition_size=partition_size)
    return workloads.tiny(seed)


def _describe(wl):
    return (f"{wl.name}: {wl.num_seqs} seqs, sum T={int(wl.seq_lens.sum())} (max {wl.max_seq_len}), "
            f"{wl.num_heads}/{wl.num_kv_heads} heads, d={wl.head_dim}, B={wl.block_size}, {wl.kv_dtype} KV, "
            f"{wl.q_dtype} q, f32 out and accumulation, P={wl.partition_size}; step = copy of "
            f"{len(wl.copy_pairs)} blocks + store of {wl.num_seqs} new tokens"
            f"{' (bf16, quantized on write)' if wl.step_keys_src is not None else ''} + split-KV decode")


def _first_per_slot(slots, rows):
    """The rows, keeping the first of those that name the same slot."""
    _, first = np.unique(slots[rows], return_index=True)
    return rows[np.sort(first)]


class Device:
    """The workload resident on the GPU and the step's prepared calls.

    pools > 1 keeps that many copies of the K/V pool; step i runs on copy
    i % pools, so that back-to-back steps do not find the previous step's
    K/V in the 256 MB Infinity Cache (MALL) once the copies together exceed it.
    """

    def __init__(self, wl, pools=1, groups=None, separate_cow=False):
        import torch
        import paged_kv_cache_142_amd as pa
        self.pa, self.torch, self.wl = pa, torch, wl
        dev = "cuda"
        view = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}

        def up(raw, fmt):
            raw = np.ascontiguousarray(raw)
            if fmt in ("f16", "bf16"):
                return torch.from_numpy(raw.view(np.int16)).view(view[fmt]).to(dev)
            return torch.from_numpy(raw).to(dev)

        self.fp8 = wl.kv_dtype == "fp8_e4m3"
        self.k_cache = torch.zeros(wl.pool_shape(), dtype=view[wl.kv_dtype], device=dev)
        self.v_cache = torch.zeros(wl.pool_shape(), dtype=view[wl.kv_dtype], device=dev)
        keys, values = up(wl.keys, wl.kv_dtype), up(wl.values, wl.kv_dtype)
        slots = torch.from_numpy(wl.slots).to(dev)
        # one row per slot: sequences that share a block (shared prefixes)
        # list its rows once each, with identical contents
        pre = torch.from_numpy(_first_per_slot(wl.slots, wl.prefill_rows())).to(dev)
        step = torch.from_numpy(_first_per_slot(wl.slots, wl.step_rows())).to(dev)
        kv = "fp8_e4m3" if self.fp8 else None
        pa.pa_reshape_and_cache(keys[pre].contiguous(), values[pre].contiguous(), self.k_cache, self.v_cache,
                                slots[pre].contiguous(), kv_dtype=kv)
        # fp8 pools: the step's new tokens arrive in bf16 and are quantized on write
        self.quantize_step = wl.step_keys_src is not None
        if self.quantize_step:
            self.step_keys = up(wl.step_keys_src, "bf16")
            self.step_values = up(wl.step_values_src, "bf16")
        else:
            self.step_keys = keys[step].contiguous()
            self.step_values = values[step].contiguous()
        self.step_slots = slots[step].contiguous()
        del keys, values
        self.pairs = torch.from_numpy(wl.copy_pairs).to(dev)
        self.q = up(wl.q, wl.q_dtype)
        self.out = torch.empty((wl.num_seqs, wl.num_heads, wl.head_dim), dtype=torch.float32, device=dev)
        self.tables = torch.from_numpy(wl.block_tables).to(dev)
        self.lens = torch.from_numpy(wl.seq_lens).to(dev)
        self.k_scale = torch.from_numpy(wl.k_scale).to(dev) if self.fp8 else None
        self.v_scale = torch.from_numpy(wl.v_scale).to(dev) if self.fp8 else None
        n = pa.pa_decode_workspace_size(wl.num_seqs, wl.num_heads, wl.head_dim, wl.max_seq_len, wl.partition_size)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        self.kv = kv
        dargs = dict(out=self.out, q=self.q, k_cache=self.k_cache, v_cache=self.v_cache,
                          block_tables=self.tables, seq_lens=self.lens, max_seq_len=wl.max_seq_len,
                          scale=float(wl.scale), partition_size=wl.partition_size, workspace=self.ws,
                          k_scale=self.k_scale, v_scale=self.v_scale, kv_dtype=kv)
        self.dargs = dargs
        # beam groups: decode through pa_decode_shared_prefix, which reads the
        # shared prompt partitions once per group
        self.groups = None
        if groups is not None:
            starts, prefix = groups
            self.groups = dict(group_start=torch.from_numpy(starts).to(dev),
                               group_prefix=torch.from_numpy(prefix).to(dev),
                               max_group_size=int(np.diff(starts).max()), max_prefix_len=int(prefix.max()))
        self.pools = [(self.k_cache, self.v_cache)] + [(self.k_cache.clone(), self.v_cache.clone())
                                                        for _ in range(pools - 1)]
        # The timed step stores the new tokens inside the decode call
        # (pa_decode_append: copy-on-write copies first, then one call) where
        # that call applies; the per-call timing loop keeps the four separate
        # launches (scatter, copy, partition, reduce).
        self.append_fused = not self.quantize_step and self.step_keys.shape[0] == wl.num_seqs
        # the copy-on-write copies inside that call (pa_decode_append_cow), or
        # as a launch of their own before it
        self.separate_cow = separate_cow
        # identical calls every step: marshal the C arguments once per pool copy
        self.call_sets = [self._step_calls(kc, vc) for kc, vc in self.pools]
        self.part_sets = [self._make_calls(kc, vc) for kc, vc in self.pools]
        self.decode_calls = [self._decode_call(kc, vc) for kc, vc in self.pools]
        # decode with append alone (no copies), for the per-call times
        self.append_calls = ([self.pa.prepared("pa_decode_append", **dict(self.dargs, k_cache=kc, v_cache=vc),
                                               key=self.step_keys, value=self.step_values) for kc, vc in self.pools]
                             if self.append_fused and self.groups is None else [])
        self.calls = self.call_sets[0]
        torch.cuda.synchronize()

    def _decode_call(self, kc, vc):
        dargs = dict(self.dargs, k_cache=kc, v_cache=vc)
        if self.groups is not None:
            return self.pa.prepared("pa_decode_shared_prefix", **dargs, **self.groups)
        return self.pa.prepared("pa_decode", **dargs)

    def _step_calls(self, k_cache=None, v_cache=None):
        """The timed step's calls.  FP8 pools: the quantize-on-write scatter,
        then the copies and the decode in one call given no tokens."""
        if self.quantize_step and not self.separate_cow and self.groups is None and self.pairs.numel():
            calls = self._make_calls(k_cache, v_cache)
            kc = self.k_cache if k_cache is None else k_cache
            vc = self.v_cache if v_cache is None else v_cache
            return [calls[0], self.pa.prepared("pa_decode_append_cow", **dict(self.dargs, k_cache=kc, v_cache=vc),
                                               key=None, value=None, block_pairs=self.pairs)]
        return self._make_calls(k_cache, v_cache, fused=self.append_fused)

    def _make_calls(self, k_cache=None, v_cache=None, fused=False):
        pa, kv = self.pa, self.kv
        kc = self.k_cache if k_cache is None else k_cache
        vc = self.v_cache if v_cache is None else v_cache
        dargs = dict(self.dargs, k_cache=kc, v_cache=vc)
        if fused:
            copy = pa.prepared("pa_copy_blocks", kc, vc, self.pairs, kv_dtype=kv) if self.pairs.numel() else (
                lambda: None)
            if self.groups is not None:
                return [copy, pa.prepared("pa_decode_shared_prefix", **dargs, **self.groups, key=self.step_keys,
                                          value=self.step_values)]
            if self.separate_cow:
                return [copy, pa.prepared("pa_decode_append", **dargs, key=self.step_keys, value=self.step_values)]
            return [pa.prepared("pa_decode_append_cow", **dargs, key=self.step_keys, value=self.step_values,
                                block_pairs=self.pairs)]
        scatter = (pa.prepared("pa_reshape_and_cache_fp8", self.step_keys, self.step_values, kc, vc,
                               self.k_scale, self.v_scale, self.step_slots)
                   if self.quantize_step else
                   pa.prepared("pa_reshape_and_cache", self.step_keys, self.step_values, kc, vc,
                               self.step_slots, kv_dtype=kv))
        copy = pa.prepared("pa_copy_blocks", kc, vc, self.pairs, kv_dtype=kv) if self.pairs.numel() else (lambda: None)
        if self.groups is not None:  # one call: prefix states, partitions, reduce
            return [scatter, copy, self._decode_call(kc, vc), lambda: None]
        return [
            scatter,
            copy,
            pa.prepared("pa_decode_partition", **dargs),
            pa.prepared("pa_decode_reduce", **dargs),
        ]

    def capture(self):
        """Capture one step (four launches, no memsets) into a HIP graph."""
        import torch
        pa, wl = self.pa, self.wl
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                calls = self._step_calls()
                for call in calls:
                    call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        return g

    def step(self, i=0):
        for call in self.call_sets[i % len(self.call_sets)]:
            call()


def settle(run, min_ms):
    """Untimed steps until at least min_ms of wall time has passed (the GPU
    raises its clocks over the first hundreds of milliseconds of load);
    returns (steps, seconds)."""
    import torch
    if min_ms <= 0:
        return 0, 0.0
    t0 = time.perf_counter()
    k = 0
    while True:
        for _ in range(10):
            run(k)
            k += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return k, time.perf_counter() - t0


def back_to_back(torch, calls, n):
    """Mean microseconds per call of n calls issued back to back (call i
    is calls[i % len(calls)]), between one event pair, after a few untimed
    ones."""
    for i in range(min(n, 4)):
        calls[i % len(calls)]()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        calls[i % len(calls)]()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def identity_tables(wl):
    """The same workload with every sequence's blocks in consecutive
    physical blocks: the physical ids are relabelled so that the blocks the
    tables name, in table order, become 0, 1, 2, ... and the rest follow.
    Contents, lengths and copy pairs are the same up to the relabelling."""
    B = wl.block_size
    named = wl.block_tables[wl.block_tables >= 0]
    _, first = np.unique(named, return_index=True)
    used = named[np.sort(first)].astype(np.int64)
    rest = np.setdiff1d(np.arange(wl.num_blocks, dtype=np.int64), used)
    new_id = np.empty(wl.num_blocks, np.int64)
    new_id[np.concatenate([used, rest])] = np.arange(wl.num_blocks, dtype=np.int64)
    tables = np.where(wl.block_tables >= 0, new_id[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    slots = new_id[wl.slots // B] * B + wl.slots % B
    pairs = new_id[wl.copy_pairs] if len(wl.copy_pairs) else wl.copy_pairs
    return dataclasses.replace(wl, block_tables=tables, slots=slots.astype(np.int64),
                               copy_pairs=pairs.astype(np.int64).reshape(-1, 2))


def paging_ab(args):
    """pa_decode on the same workload with shuffled and with identity block
    tables, alternating batches of back-to-back calls between the two in one
    process: the cost of the block-table indirection on this hardware."""
    import torch
    wl = _workload(args.config, args.seed, args.partition_size)
    devs = {"shuffled": Device(wl, pools=args.pools), "identity": Device(identity_tables(wl), pools=args.pools)}
    settle(devs["shuffled"].step, args.settle_ms)
    times = {k: [] for k in devs}
    for _ in range(args.ab_rounds):
        for name, d in devs.items():
            times[name].append(back_to_back(torch, d.decode_calls, args.steps))
    med = {k: float(np.median(v)) for k, v in times.items()}
    print(json.dumps({
        "paging_ab": _describe(wl), "rounds": args.ab_rounds, "calls_per_round": args.steps,
        "pa_decode_us_median": {k: round(v, 2) for k, v in med.items()},
        "pa_decode_us_p10_p90": {k: [round(float(np.percentile(v, 10)), 2), round(float(np.percentile(v, 90)), 2)]
                                 for k, v in times.items()},
        "shuffled_over_identity": round(med["shuffled"] / med["identity"], 4)}), flush=True)


def partition_algorithmic_bytes(wl):
    """Bytes the partition kernel must move: every K/V row of every sequence
    once, each kv-head workgroup's block-table entries, the queries and the
    sequence lengths.  (Partition states written for the reduce are
    overhead, not algorithmic bytes.)"""
    B = wl.block_size
    lens = wl.seq_lens.astype(np.int64)
    q_bytes = {"f32": 4, "f16": 2, "bf16": 2}[wl.q_dtype]
    blocks = int(((lens + B - 1) // B).sum())
    return (wl.kv_bytes() + 4 * wl.num_kv_heads * blocks + wl.num_seqs * wl.num_heads * wl.head_dim * q_bytes
            + 4 * wl.num_seqs)


def _source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(wl):
    """HBM bytes per partition launch from committed rocprofv3 counters, when
    they were taken on the current kernel source and this workload."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != _source_hash() or rec.get("workload") != wl.name or \
            rec.get("seed") != wl.seed or rec.get("partition_size") != wl.partition_size:
        return None
    return rec.get("hbm_bytes_per_launch")


def _oracle_pools(wl):
    """The oracle's K/V pools of the workload (its scatter of every token)."""
    import oracle
    kc = np.zeros(wl.pool_shape(), wl.keys.dtype)
    vc = np.zeros(wl.pool_shape(), wl.keys.dtype)
    oracle.reshape_and_cache(kc, vc, wl.keys, wl.values, wl.slots, wl.block_size)
    return kc, vc


def _oracle_rows(wl, kc, vc, first, stride, budget_s):
    """Run the oracle on rows first, first + stride, ... (wrapping around)
    until budget_s of its own time is spent; returns (rows, tokens, seconds)."""
    import oracle
    done, tokens, elapsed, i = 0, 0, 0.0, first % wl.num_seqs
    while elapsed < budget_s:
        t0 = time.perf_counter()
        oracle.paged_decode(wl.q, wl.q_dtype, kc, vc, wl.kv_dtype, wl.block_tables, wl.seq_lens,
                            wl.block_size, float(wl.scale), wl.k_scale, wl.v_scale, rows=[i])
        elapsed += time.perf_counter() - t0
        done += 1
        tokens += int(wl.seq_lens[i])
        i = (i + stride) % wl.num_seqs
    return done, tokens, elapsed


def _oracle_worker(job):
    """One worker process of the all-cores baseline: the pools come from a
    shared file, the rest of the workload from the arguments."""
    wl, pool_file, first, stride, budget_s = job
    pools = np.load(pool_file, mmap_mode="r")
    return _oracle_rows(wl, pools[0], pools[1], first, stride, budget_s)


def _cpu_share():
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # one GPU's share of a shared host: at most 16 workers
    return max(1, min(avail, 16)), avail


def cpu_baseline(wl, budget_s):
    """The float64 oracle, as it stands, over a bounded sample of the same
    workload: its sequences in order, starting over after the last one, for
    about budget_s seconds.  Run twice: on one thread, and on all the host
    cores this GPU's job may use (one spawned worker process per core, each
    on its own share of the sequences, BLAS limited to one thread per
    worker, the pools shared through a file in memory).  The worker
    processes are fresh interpreters that never touch the GPU."""
    import tempfile
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing
    from threadpoolctl import threadpool_limits

    kc, vc = _oracle_pools(wl)
    kv_per_token = 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes
    with threadpool_limits(limits=1):
        done, tokens, elapsed = _oracle_rows(wl, kc, vc, 0, 1, budget_s)
    one = {"value": round(tokens * kv_per_token / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} sequences in order ({done / wl.num_seqs:.2f} passes over the {wl.num_seqs}; "
                     f"{tokens} tokens, {tokens * kv_per_token / 1e6:.1f} MB of KV), float64 NumPy, "
                     f"BLAS limited to 1 thread, {elapsed:.1f} s",
           "seconds": round(elapsed, 2), "us_per_seq": round(elapsed / done * 1e6, 1)}
    workers, avail = _cpu_share()
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    fd, pool_file = tempfile.mkstemp(suffix=".npy", dir=shm)
    os.close(fd)
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        np.save(pool_file, np.stack([kc, vc]))
        del kc, vc
        os.environ.update({k: "1" for k in saved})  # inherited by the spawned workers
        # the workers need the queries, tables and lengths, not the token rows
        slim = dataclasses.replace(wl, keys=wl.keys[:0], values=wl.values[:0], slots=wl.slots[:0],
                                   step_keys_src=None, step_values_src=None)
        jobs = [(slim, pool_file, w, workers, budget_s) for w in range(workers)]
        t0 = time.perf_counter()
        with ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("spawn")) as ex:
            parts = list(ex.map(_oracle_worker, jobs))
        wall = time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        os.unlink(pool_file)
    done_all = sum(p[0] for p in parts)
    tok_all = sum(p[1] for p in parts)
    busy = max(p[2] for p in parts)
    return {"value": round(tok_all * kv_per_token / busy / 1e9, 4), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{done_all} sequences ({done_all / wl.num_seqs:.2f} passes over the {wl.num_seqs}; "
                      f"{tok_all} tokens, {tok_all * kv_per_token / 1e6:.1f} MB of KV), float64 NumPy, "
                      f"{workers} worker processes with 1 BLAS thread each, about {busy:.1f} s each",
            "os_cpu_count": os.cpu_count(), "cores_available": avail, "blas_threads_per_worker": 1,
            "seconds": round(busy, 2), "wall_s_with_start_up": round(wall, 2),
            "single_thread": one}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the paged decode path here is a single-GPU build "
              "(sharding across GPUs is described, not implemented).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, args.steps)
        return
    if args.swap_mib:
        swap_bandwidth(args.swap_mib, args.steps)
        return
    if args.config.startswith("prefill"):
        run_prefill(args)
        return
    if args.paging_ab:
        paging_ab(args)
        return
    wl = _workload(args.config, args.seed, args.partition_size)
    if args.identity_tables:
        wl = identity_tables(wl)
    if args.graph and args.pools != 1:
        print("--graph replays one captured step and cannot rotate pool copies; use --pools 1", file=sys.stderr)
        sys.exit(2)
    groups = None
    if args.config.endswith("_grouped"):  # 8 prompts x 6 beams, consecutive; the prompt's whole blocks are shared
        beams = 6
        starts = np.arange(0, wl.num_seqs + 1, beams, dtype=np.int32)
        prompt_len = (1032 if args.config.startswith("shared_prefix_cow") else
                      LONG_PROMPT if args.config.startswith("shared_prefix_long") else 1024)
        # the prompt's whole blocks, and never a member's newest token (which
        # the step stores into the member's own block): a beam with no suffix
        # yet shares one block less
        B = wl.block_size
        shared = np.array([min(prompt_len // B * B, int((wl.seq_lens[a:b] - 1).min()) // B * B)
                           for a, b in zip(starts[:-1], starts[1:])], np.int32)
        groups = (starts, shared)
    dev = Device(wl, pools=args.pools, groups=groups, separate_cow=args.separate_cow)
    graph = None
    if args.graph:  # one eager step first (one-time kernel attribute setup), then capture
        dev.step()
        torch.cuda.synchronize()
        graph = dev.capture()
    run = (lambda i: graph.replay()) if graph is not None else dev.step
    settle_steps, settle_s = settle(run, args.settle_ms)
    for i in range(args.warmup):
        run(settle_steps + i)
    torch.cuda.synchronize()
    # timed region: exactly K steps between one event pair; events at batch
    # boundaries (none inside a batch) give the distribution over batches
    nb = min(args.steps, 10)
    bounds = np.linspace(0, args.steps, nb + 1).round().astype(int)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for b in range(nb):
        for i in range(bounds[b], bounds[b + 1]):
            run(i)
        evs[b + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = gpu_ms / args.steps
    batch_us = [evs[b].elapsed_time(evs[b + 1]) / (bounds[b + 1] - bounds[b]) * 1e3 for b in range(nb)]

    # each call alone, `steps` times back to back between one event pair (no
    # marker between the launches), alternating the pool copies as the step does
    n = args.steps
    decode_alone_us = back_to_back(torch, dev.decode_calls, n)
    k_us = {"reshape_and_cache": back_to_back(torch, [c[0] for c in dev.part_sets], n),
            "copy_blocks": back_to_back(torch, [c[1] for c in dev.part_sets], n)}
    if groups is None:
        k_us["decode_partition"] = back_to_back(torch, [c[2] for c in dev.part_sets], n)
        k_us["decode_reduce"] = back_to_back(torch, [c[3] for c in dev.part_sets], n)
    k_us["decode"] = decode_alone_us
    if dev.quantize_step and len(dev.call_sets[0]) == 2:  # the copies and the decode in one call
        k_us["decode_cow"] = back_to_back(torch, [c[1] for c in dev.call_sets], n)
    if dev.append_calls:
        k_us["decode_append"] = back_to_back(torch, dev.append_calls, n)
        if not dev.separate_cow:
            k_us["decode_append_cow"] = back_to_back(torch, [c[0] for c in dev.call_sets], n)
    kv_bytes = wl.kv_bytes()
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    if groups is not None:
        # the call's launches together against the distinct bytes they must read
        part_bytes = unique_kv_bytes(wl)
        achieved = part_bytes / (k_us["decode"] * 1e-6) / 1e9
        roof_kernel = ("pa_decode_shared_prefix (its launches together, called back to back) over the distinct "
                       "K/V bytes")
        traffic = None
    else:
        part_bytes = partition_algorithmic_bytes(wl)
        achieved = part_bytes / (k_us["decode_partition"] * 1e-6) / 1e9
        roof_kernel = ("decode partition kernel: pa_decode_partition called back to back between one event pair "
                       "(one launch per call up to 64 sequences; above that a plan kernel precedes it)")
        traffic = _traffic(wl)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.kv_dtype, "data": "synthetic",
        "config": {"workload": _describe(wl), "seed": wl.seed, "num_seqs": wl.num_seqs,
                   "sum_seq_len": int(wl.seq_lens.sum()), "max_seq_len": wl.max_seq_len,
                   "num_heads": wl.num_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, "partition_size": wl.partition_size, "kv_dtype": wl.kv_dtype,
                   "q_dtype": wl.q_dtype, "accum": "f32", "kv_bytes_per_step": kv_bytes},
        "us_per_step": round(ms_per_step * 1e3, 2),
        "seqs_per_s": round(wl.num_seqs / (ms_per_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_alone_us": round(decode_alone_us, 2),
        "decode_alone_GBs": round(kv_bytes / (decode_alone_us * 1e-6) / 1e9, 2),
        "decode_alone_hbm_frac": round(kv_bytes / (decode_alone_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "step_us_median": round(float(np.median(batch_us)), 2),
        "step_us_p10_p90": [round(float(np.percentile(batch_us, 10)), 2),
                            round(float(np.percentile(batch_us, 90)), 2)],
        "step_batches": f"{nb} batches of {args.steps // nb}-{-(-args.steps // nb)} steps inside the timed region",
        "kernels_us": {k: round(v, 2) for k, v in k_us.items()},
        "kernels_timing": "each call alone, back to back between one event pair",
        "settle": {"untimed_steps": settle_steps, "seconds": round(settle_s, 3), "min_ms": args.settle_ms,
                   "why": "untimed steps before --warmup until the GPU clocks have risen from idle"},
        "host_wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "step_mode": "hip_graph" if graph is not None else "eager",
        "step_calls": ((["pa_copy_blocks", "pa_decode_shared_prefix (with the new tokens)"] if groups is not None
                        else ["pa_copy_blocks", "pa_decode_append"] if dev.separate_cow
                        else ["pa_decode_append_cow (the copies and the new tokens' store in the decode launch, "
                              "but for the FP8 matrix-core shape: there pa_copy_blocks, then pa_decode_append)"]) if dev.append_fused else
                       ["pa_reshape_and_cache_fp8", "pa_decode_append_cow (no tokens: the copies in the "
                        "matrix-core partition launch, then the reduce)"] if len(dev.call_sets[0]) == 2 else
                       ["pa_reshape_and_cache" + ("_fp8" if dev.quantize_step else ""), "pa_copy_blocks",
                        "pa_decode_shared_prefix" if groups is not None else "pa_decode_partition",
                        *([] if groups is not None else ["pa_decode_reduce"])]),
        "pool_copies": args.pools,
        "block_tables": ("identity: each sequence's blocks are consecutive physical blocks" if args.identity_tables
                         else "shuffled: blocks drawn from a seeded permutation of the pool"),
        "roofline": {"kernel": roof_kernel, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": part_bytes},
    }
    if wl.name.startswith("shared_prefix"):
        line["config"]["unique_kv_bytes_per_step"] = unique_kv_bytes(wl)
        distinct = unique_kv_bytes(wl) * args.pools
        line["config"]["cache_assisted"] = (
            "prompt blocks are shared by 6 beams: the logical KV bytes are read from far fewer distinct bytes"
            + (", which fit in the 256 MB Infinity Cache" if distinct < 256e6 else
               f" ({distinct / 1e6:.0f} MB over the pool copies, more than the 256 MB Infinity Cache)"))
        line["unique_kv_GBs"] = round(unique_kv_bytes(wl) / (ms_per_step * 1e-3) / 1e9, 2)
        if groups is not None:
            line["config"]["decode"] = ("pa_decode_shared_prefix: groups of 6 beams, the prompt's whole blocks "
                                        f"({int(groups[1][0])} tokens) shared")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
