"""Seeded generators for the five decode workloads (no method arithmetic).

Every array is produced from ``numpy.random.SeedSequence([seed, tag])``:
normals are drawn in float32 in fixed-size chunks, each chunk from its own
spawned PCG64 stream, so the bytes do not depend on the number of threads.
Values are then rounded to the stored format:

* fp32 -- the float32 draw itself;
* fp16 -- NumPy ``astype(float16)`` (round to nearest even);
* bf16 -- PyTorch ``to(torch.bfloat16)`` (round to nearest even);
* fp8 E4M3 -- per kv head a float32 scale ``amax / 448`` (keys and values
  separately), then PyTorch ``to(torch.float8_e4m3fn)`` of the clipped
  quotient (round to nearest even, saturated at +-448).

Raw storage arrays are ``float32`` (fp32), ``uint16`` bit patterns (fp16,
bf16) and ``uint8`` codes (fp8).

Structure of a ``DecodeWorkload``: sequence ``i`` holds ``seq_lens[i]`` tokens
including the token of the current step (its last one).  Physical blocks are
handed out as consecutive chunks of one seeded permutation of the pool, in
sequence order; unused table entries are ``-1``.  ``slots[r]`` is the physical
slot (``block * B + row``) of token row ``r``; token rows are stored in
logical order, sequence after sequence.  ``copy_pairs`` name
``(source, destination)`` blocks for the step's block copy: sources are
blocks in use, destinations are spare blocks that no table references.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8_e4m3": np.uint8}
FP8_MAX = 448.0
_CHUNK_ELEMS = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------ low level


def _seed(seed, tag):
    return np.random.SeedSequence([int(seed), int(tag)])


def round_to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the raw storage of ``dtype`` (not fp8)."""
    if dtype == "f32":
        return np.asarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"no plain rounding for {dtype!r}")


def quantize_e4m3(x32: np.ndarray, head_scale: np.ndarray) -> np.ndarray:
    """fp8 E4M3FN codes of ``x / scale`` (per kv head on axis -2)."""
    q = np.asarray(x32, dtype=np.float32) / head_scale.astype(np.float32)[:, None]
    q = np.clip(q, -FP8_MAX, FP8_MAX)
    return torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _row_chunks(num_rows, row_elems):
    per = max(1, _CHUNK_ELEMS // row_elems)
    return [(s, min(num_rows, s + per)) for s in range(0, num_rows, per)]


def _token_rows(seed_seq, num_rows, heads, dim, dtype):
    """``[num_rows][heads][dim]`` N(0,1) rows rounded to ``dtype``.

    Returns ``(raw, head_scale)``; ``head_scale`` is ``None`` except for fp8.
    """
    chunks = _row_chunks(num_rows, heads * dim)
    children = seed_seq.spawn(len(chunks))

    def draw(k):
        lo, hi = chunks[k]
        rng = np.random.default_rng(children[k])
        return rng.standard_normal((hi - lo, heads, dim), dtype=np.float32)

    out = np.empty((num_rows, heads, dim), dtype=STORAGE[dtype])
    if dtype != "fp8_e4m3":
        def fill(k):
            lo, hi = chunks[k]
            out[lo:hi] = round_to_storage(draw(k), dtype)
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(len(chunks))))
        return out, None

    def amax(k):
        return np.abs(draw(k)).max(axis=(0, 2))
    with ThreadPoolExecutor(_THREADS) as ex:
        head_amax = np.max(np.stack(list(ex.map(amax, range(len(chunks))))), axis=0)
    head_scale = (head_amax.astype(np.float32) / np.float32(FP8_MAX)).astype(np.float32)

    def fill8(k):
        lo, hi = chunks[k]
        out[lo:hi] = quantize_e4m3(draw(k), head_scale)
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill8, range(len(chunks))))
    return out, head_scale


def _query(seed_seq, num_seqs, heads, dim, dtype):
    rng = np.random.default_rng(seed_seq)
    return round_to_storage(rng.standard_normal((num_seqs, heads, dim), dtype=np.float32), dtype)


# ------------------------------------------------------------ workloads


@dataclass
class DecodeWorkload:
    name: str
    seed: int
    kv_dtype: str
    q_dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    partition_size: int
    scale: np.float32
    seq_lens: np.ndarray        # int32 [N], including the current token
    block_tables: np.ndarray    # int32 [N][max_blocks], -1 where unused
    token_offsets: np.ndarray   # int64 [N+1], rows of sequence i: offsets[i]..offsets[i+1]
    keys: np.ndarray            # raw [sum T][H_kv][d], logical order
    values: np.ndarray          # raw [sum T][H_kv][d]
    slots: np.ndarray           # int64 [sum T]
    q: np.ndarray               # raw [N][H_q][d]
    k_scale: Optional[np.ndarray]  # float32 [H_kv] for fp8, else None
    v_scale: Optional[np.ndarray]
    copy_pairs: np.ndarray      # int64 [n][2]
    # fp8 pools only: the step's new tokens as bf16 rows [N][H_kv][d] (raw
    # bits), quantized on write instead of copied from keys/values
    step_keys_src: Optional[np.ndarray] = None
    step_values_src: Optional[np.ndarray] = None

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    @property
    def elem_bytes(self):
        return ELEM_BYTES[self.kv_dtype]

    def prefill_rows(self):
        """Token rows already cached before the step (all but each last)."""
        keep = np.ones(len(self.slots), dtype=bool)
        last = self.token_offsets[1:] - 1
        keep[last[self.seq_lens > 0]] = False
        return np.nonzero(keep)[0]

    def step_rows(self):
        """The current token of every non-empty sequence (one per sequence)."""
        last = self.token_offsets[1:] - 1
        return last[self.seq_lens > 0]

    def pool_shape(self):
        return (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)

    def kv_bytes(self):
        """K+V bytes the step must read: ``sum_i T_i * 2 * H_kv * d * b``."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * self.elem_bytes


def _tables(perm, need, block_size):
    width = max(1, max(need) if len(need) else 1)
    tables = np.full((len(need), width), -1, dtype=np.int32)
    start = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[start:start + n]
        start += n
    return tables


def _slots(tables, seq_lens, block_size):
    out = []
    for i, t in enumerate(seq_lens):
        pos = np.arange(int(t), dtype=np.int64)
        out.append(tables[i, pos // block_size].astype(np.int64) * block_size + pos % block_size)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def build_decode_workload(name, seed, *, seq_lens, num_heads, num_kv_heads, head_dim, block_size,
                          kv_dtype, q_dtype, spare_blocks, num_copy_pairs, partition_size,
                          pool_size=None):
    """Assemble a ``DecodeWorkload`` from lengths and shapes (seeded)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = [-(-int(t) // block_size) for t in seq_lens]
    used = sum(need)
    num_blocks = pool_size if pool_size is not None else used + spare_blocks
    num_copy_pairs = min(num_copy_pairs, used, num_blocks - used)
    perm = np.random.default_rng(_seed(seed, 1)).permutation(num_blocks).astype(np.int64)
    tables = _tables(perm, need, block_size)
    offsets = np.zeros(len(seq_lens) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(seq_lens.astype(np.int64))
    total = int(offsets[-1])
    keys, k_scale = _token_rows(_seed(seed, 2), total, num_kv_heads, head_dim, kv_dtype)
    values, v_scale = _token_rows(_seed(seed, 3), total, num_kv_heads, head_dim, kv_dtype)
    q = _query(_seed(seed, 4), len(seq_lens), num_heads, head_dim, q_dtype)
    rng = np.random.default_rng(_seed(seed, 5))
    in_use = perm[:used]
    spare = perm[used:]
    src = rng.choice(in_use, size=num_copy_pairs, replace=False) if num_copy_pairs else np.zeros(0, np.int64)
    dst = rng.choice(spare, size=num_copy_pairs, replace=False) if num_copy_pairs else np.zeros(0, np.int64)
    pairs = np.stack([src, dst], axis=1).astype(np.int64).reshape(-1, 2)
    step_src = (None, None)
    if kv_dtype == "fp8_e4m3":
        n_step = int((seq_lens > 0).sum())
        step_src = (_token_rows(_seed(seed, 6), n_step, num_kv_heads, head_dim, "bf16")[0],
                    _token_rows(_seed(seed, 7), n_step, num_kv_heads, head_dim, "bf16")[0])
    return DecodeWorkload(
        step_keys_src=step_src[0], step_values_src=step_src[1],
        name=name, seed=seed, kv_dtype=kv_dtype, q_dtype=q_dtype, num_seqs=len(seq_lens),
        num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=num_blocks, partition_size=partition_size,
        scale=np.float32(1.0 / math.sqrt(head_dim)), seq_lens=seq_lens, block_tables=tables,
        token_offsets=offsets, keys=keys, values=values, slots=_slots(tables, seq_lens, block_size),
        q=q, k_scale=k_scale, v_scale=v_scale, copy_pairs=pairs)


def tiny(seed=0):
    """fp32, lengths 1/17/40/100, 4 heads = 4 kv heads, d=64, B=16, pool 32, 3 copy pairs."""
    return build_decode_workload("tiny", seed, seq_lens=[1, 17, 40, 100], num_heads=4, num_kv_heads=4,
                                 head_dim=64, block_size=16, kv_dtype="f32", q_dtype="f32",
                                 spare_blocks=0, num_copy_pairs=3, partition_size=512, pool_size=32)


def gqa(seed=0, num_seqs=64, max_len=4096, partition_size=832):
    """bf16, 32 query / 8 kv heads, d=128, B=16, lengths uniform on 1..4096,
    split-KV partitions of 832 tokens (the benchmarked configuration)."""
    lens = np.random.default_rng(_seed(seed, 0)).integers(1, max_len + 1, size=num_seqs)
    return build_decode_workload("gqa", seed, seq_lens=lens, num_heads=32, num_kv_heads=8, head_dim=128,
                                 block_size=16, kv_dtype="bf16", q_dtype="bf16", spare_blocks=16,
                                 num_copy_pairs=16, partition_size=partition_size)


def mha(seed=0, num_seqs=256, max_len=2048, partition_size=512):
    """fp16, 40 heads = 40 kv heads, d=128, B=16, lengths uniform on 1..2048."""
    lens = np.random.default_rng(_seed(seed, 0)).integers(1, max_len + 1, size=num_seqs)
    return build_decode_workload("mha", seed, seq_lens=lens, num_heads=40, num_kv_heads=40, head_dim=128,
                                 block_size=16, kv_dtype="f16", q_dtype="f16", spare_blocks=16,
                                 num_copy_pairs=16, partition_size=partition_size)


def long_fp8(seed=0, block_size=16, num_seqs=16, seq_len=32768, partition_size=512):
    """fp8 E4M3 KV with per-kv-head scales, bf16 q, 64/8 heads, d=128."""
    return build_decode_workload(f"long_fp8_b{block_size}", seed, seq_lens=[seq_len] * num_seqs,
                                 num_heads=64, num_kv_heads=8, head_dim=128, block_size=block_size,
                                 kv_dtype="fp8_e4m3", q_dtype="bf16", spare_blocks=16,
                                 num_copy_pairs=16, partition_size=partition_size)


@dataclass
class SharedPrefixWorkload:
    """Prompts shared by beams; the assembly into blocks is left to the caller.

    ``prompt_keys[k]``: raw ``[prompt_len][H_kv][d]`` of prompt ``k``;
    ``suffix_keys[s]``: raw ``[suffix_lens[s]][H_kv][d]`` of sequence
    ``s = k * beams + b``.  Sequence ``s`` attends to its prompt followed by its
    own suffix (``prompt_len + suffix_lens[s]`` tokens).  ``extreme[s]`` marks
    the sequences whose query was rescaled so that their largest logit
    magnitude is ``logit_target``.
    """
    seed: int
    num_prompts: int
    beams: int
    prompt_len: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str
    q_dtype: str
    scale: np.float32
    suffix_lens: np.ndarray
    prompt_keys: np.ndarray
    prompt_values: np.ndarray
    suffix_keys: list
    suffix_values: list
    q: np.ndarray
    extreme: np.ndarray
    logit_target: float

    @property
    def num_seqs(self):
        return self.num_prompts * self.beams

    def seq_lens(self):
        return (self.prompt_len + self.suffix_lens).astype(np.int32)

    def logical_rows(self, s, which):
        """Raw logical ``[T][H_kv][d]`` keys (``which='k'``) or values of sequence ``s``."""
        k = s // self.beams
        if which == "k":
            return np.concatenate([self.prompt_keys[k], self.suffix_keys[s]], axis=0)
        return np.concatenate([self.prompt_values[k], self.suffix_values[s]], axis=0)


def shared_prefix(seed=0, prompt_len=1032, num_prompts=8, beams=6, max_suffix=256, logit_target=80.0):
    """8 prompts x 6 beams, GQA 32/8, d=128, bf16, B=16; odd sequences get
    queries rescaled so that their largest |logit| equals ``logit_target``.

    The rescale is input construction: for each (sequence, head) the float32
    draw of ``q`` is multiplied by ``logit_target / max_j |scale * k_j . q|``
    over that sequence's (bf16-rounded) keys, then rounded to bf16.
    """
    H, Hkv, d, B = 32, 8, 128, 16
    rng = np.random.default_rng(_seed(seed, 10))
    suffix = rng.integers(0, max_suffix + 1, size=num_prompts * beams)
    pk, _ = _token_rows(_seed(seed, 11), num_prompts * prompt_len, Hkv, d, "bf16")
    pv, _ = _token_rows(_seed(seed, 12), num_prompts * prompt_len, Hkv, d, "bf16")
    pk = pk.reshape(num_prompts, prompt_len, Hkv, d)
    pv = pv.reshape(num_prompts, prompt_len, Hkv, d)
    total_suffix = int(suffix.sum())
    sk, _ = _token_rows(_seed(seed, 13), total_suffix, Hkv, d, "bf16")
    sv, _ = _token_rows(_seed(seed, 14), total_suffix, Hkv, d, "bf16")
    cut = np.concatenate([[0], np.cumsum(suffix)])
    suffix_keys = [sk[cut[s]:cut[s + 1]] for s in range(len(suffix))]
    suffix_values = [sv[cut[s]:cut[s + 1]] for s in range(len(suffix))]
    scale = np.float32(1.0 / math.sqrt(d))
    q32 = np.random.default_rng(_seed(seed, 15)).standard_normal((num_prompts * beams, H, d), dtype=np.float32)
    extreme = (np.arange(num_prompts * beams) % 2) == 1
    group = H // Hkv
    for s in np.nonzero(extreme)[0]:
        keys = np.concatenate([pk[s // beams], suffix_keys[s]], axis=0)
        kf = torch.from_numpy(keys.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        for h in range(H):
            mag = np.abs(kf[:, h // group, :] @ q32[s, h].astype(np.float64)).max() * float(scale)
            q32[s, h] = (q32[s, h].astype(np.float64) * (logit_target / mag)).astype(np.float32)
    q = round_to_storage(q32, "bf16")
    return SharedPrefixWorkload(
        seed=seed, num_prompts=num_prompts, beams=beams, prompt_len=prompt_len, num_heads=H,
        num_kv_heads=Hkv, head_dim=d, block_size=B, kv_dtype="bf16", q_dtype="bf16", scale=scale,
        suffix_lens=suffix.astype(np.int32), prompt_keys=pk, prompt_values=pv, suffix_keys=suffix_keys,
        suffix_values=suffix_values, q=q, extreme=extreme, logit_target=logit_target)


@dataclass
class PrefillWorkload:
    """A multi-query (prefill) step over paged K/V.

    ``cache`` holds every sequence's ``T_i = cache.seq_lens[i]`` tokens (its
    keys, values, block tables and slots); the step's query rows are the last
    ``query_lens[i]`` tokens of each sequence, packed: sequence ``i`` owns rows
    ``query_start[i] .. query_start[i+1] - 1`` of ``q`` (raw ``[total_q][H][d]``).
    Before the step the cache holds each sequence's earlier tokens; the step
    writes the chunk's keys and values, then attends.
    """
    cache: DecodeWorkload
    query_lens: np.ndarray   # int32 [N]
    query_start: np.ndarray  # int32 [N+1]
    q: np.ndarray            # raw [total_q][H][d]

    @property
    def name(self):
        return self.cache.name

    @property
    def total_q(self):
        return int(self.query_start[-1])

    def chunk_rows(self):
        """Rows of ``cache.keys`` written by the step (each sequence's last Q_i)."""
        off = self.cache.token_offsets
        return np.concatenate([np.arange(off[i + 1] - self.query_lens[i], off[i + 1], dtype=np.int64)
                               for i in range(len(self.query_lens))]) if len(self.query_lens) else \
            np.zeros(0, np.int64)

    def context_rows(self):
        """Rows cached before the step."""
        keep = np.ones(len(self.cache.slots), dtype=bool)
        keep[self.chunk_rows()] = False
        return np.nonzero(keep)[0]


def build_prefill_workload(name, seed, *, seq_lens, query_lens, num_heads, num_kv_heads, head_dim, block_size,
                           kv_dtype, q_dtype, spare_blocks=0, logit_target=None):
    """Assemble a ``PrefillWorkload``: the cache as for decode (seeded), plus
    N(0, 1) query rows for each sequence's last ``query_lens[i]`` tokens.

    With ``logit_target``, each query row (token, head) is rescaled, before
    rounding to ``q_dtype``, so that its largest ``|scale * q . k|`` over the
    keys it sees (the sequence's keys up to its own position) equals the
    target: an extreme-logit stress input."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    if np.any(query_lens < 0) or np.any(query_lens > seq_lens):
        raise ValueError("query_lens must lie in [0, seq_lens]")
    cache = build_decode_workload(name, seed, seq_lens=seq_lens, num_heads=num_heads, num_kv_heads=num_kv_heads,
                                  head_dim=head_dim, block_size=block_size, kv_dtype=kv_dtype, q_dtype=q_dtype,
                                  spare_blocks=spare_blocks, num_copy_pairs=0, partition_size=512)
    start = np.zeros(len(query_lens) + 1, dtype=np.int32)
    start[1:] = np.cumsum(query_lens)
    rng = np.random.default_rng(_seed(seed, 20))
    q32 = rng.standard_normal((int(start[-1]), num_heads, head_dim), dtype=np.float32)
    if logit_target is not None:
        group = num_heads // num_kv_heads
        for i, (T, Q) in enumerate(zip(seq_lens.astype(np.int64), query_lens.astype(np.int64))):
            if Q == 0:
                continue
            raw = cache.keys[cache.token_offsets[i]:cache.token_offsets[i + 1]]
            kf = torch.from_numpy(raw.view(np.int16)).view(
                torch.bfloat16 if kv_dtype == "bf16" else torch.float16).to(torch.float64).numpy()
            rows = q32[start[i]:start[i + 1]].astype(np.float64)       # [Q][H][d]
            for h in range(num_heads):
                logit = np.abs(rows[:, h, :] @ kf[:, h // group, :].T) * float(cache.scale)  # [Q][T]
                visible = np.arange(T)[None, :] <= (T - Q + np.arange(Q))[:, None]
                mag = np.where(visible, logit, 0.0).max(axis=1)
                q32[start[i]:start[i + 1], h, :] = (rows[:, h, :] * (logit_target / mag)[:, None]).astype(np.float32)
    q = round_to_storage(q32, q_dtype)
    return PrefillWorkload(cache=cache, query_lens=query_lens, query_start=start, q=q)


def prefill(seed=0, num_seqs=16, max_len=2048, chunk=None, kv_dtype="bf16", num_heads=32, num_kv_heads=8,
            head_dim=128, block_size=16):
    """bf16, 32/8 heads, d=128, B=16, context lengths uniform on 1..max_len;
    full prefill (every token a query) or, with ``chunk``, the last
    ``min(chunk, T)`` tokens of each sequence."""
    lens = np.random.default_rng(_seed(seed, 21)).integers(1, max_len + 1, size=num_seqs)
    qlens = lens if chunk is None else np.minimum(lens, chunk)
    return build_prefill_workload(f"prefill{'' if chunk is None else f'_chunk{chunk}'}", seed, seq_lens=lens,
                                  query_lens=qlens, num_heads=num_heads, num_kv_heads=num_kv_heads,
                                  head_dim=head_dim, block_size=block_size, kv_dtype=kv_dtype,
                                  q_dtype="bf16" if kv_dtype == "fp8_e4m3" else kv_dtype)


def make(name, seed=0, **kw):
    """Workload by name: tiny, gqa, mha, shared_prefix, long_fp8, prefill."""
    return {"tiny": tiny, "gqa": gqa, "mha": mha, "shared_prefix": shared_prefix,
            "long_fp8": long_fp8, "prefill": prefill}[name](seed=seed, **kw)
