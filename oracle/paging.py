"""Physical KV pool, scatter through a slot mapping, block copy, gather.

Test infrastructure only (see the package docstring).

Pool layout (a reading: the pages describe logical blocks of ``B`` tokens
mapped to physical blocks but give no memory layout):
``cache[num_blocks][H_kv][B][d]`` for K and the same for V, so that one
(physical block, kv head) tile of ``B*d`` elements is contiguous.

Addressing (0h-n0.github.io, "論文解説: Efficient Memory Management for Large
Language Model Serving with PagedAttention", section "PagedAttentionのメモリ
管理": logical block ``k`` of a sequence holds its tokens ``k*B .. k*B+B-1``
and the block table maps logical block numbers to physical block numbers):
token ``t`` of sequence ``i`` lives in physical block ``table[i][t // B]`` at
row ``t % B``.  A slot is the flat index ``physical_block * B + row``.

All functions copy raw stored elements unchanged (any dtype), so they are
exact; they work on NumPy arrays in host memory.
"""

from __future__ import annotations

import numpy as np


def reshape_and_cache(k_cache, v_cache, key, value, slot_mapping, block_size):
    """Write each new token's K/V rows into its slot, in place.

    ``key``/``value``: ``[num_tokens][H_kv][d]``; ``slot_mapping``:
    ``[num_tokens]`` integers; a negative slot means "no write" for that token
    (a reading: padding tokens in a batch).  Storing the new token's K and V
    so that later steps reuse them is the point of the KV cache (youngju.dev,
    "KVキャッシュとPagedAttention — 推論メモリのすべて", section "核心原理:
    KVキャッシュとは何か"); one block is added at a time as tokens accumulate
    (same page, "PagedAttention: OS仮想メモリ式の管理").

    Parity: pinned by the paged-versus-contiguous round trip in the oracle
    tests (scatter every token, gather every sequence, compare with the
    contiguous arrays bit for bit).
    """
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block, row = divmod(slot, block_size)
        k_cache[block, :, row, :] = key[t]
        v_cache[block, :, row, :] = value[t]


def copy_blocks(k_cache, v_cache, block_pairs):
    """Copy whole physical blocks ``src -> dst`` (K and V, every head), in place.

    This is the block copy that copy-on-write performs before a sequence
    writes into a block it shares (0h-n0.github.io explainer, section
    "Copy-on-Write（CoW）によるメモリ共有": when the reference count exceeds
    one a new block is allocated, the old block's contents copied into it and
    the table remapped).  Every pair reads the contents from before the call
    (a reading for batches of pairs): sources are snapshotted first.

    Parity: pinned in the oracle tests by comparing the gathered logical
    contents of a copied sequence with the original and by checking that
    untouched blocks are unchanged.
    """
    pairs = np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    k_src = {int(s): k_cache[int(s)].copy() for s, _ in pairs}
    v_src = {int(s): v_cache[int(s)].copy() for s, _ in pairs}
    for s, d in pairs:
        k_cache[int(d)] = k_src[int(s)]
        v_cache[int(d)] = v_src[int(s)]


def swap_blocks(src_k, src_v, dst_k, dst_v, block_pairs):
    """Copy whole blocks from one pool into another: ``dst[d] = src[s]`` (K
    and V, every head and row) for each pair ``(s, d)``.

    This is the transfer of preemption by swapping (0h-n0.github.io
    explainer, section "プリエンプション戦略", strategy 1): a preempted
    sequence's physical blocks move to a pool in CPU memory and later back
    into free GPU blocks; the block tables are remapped on the host.  Pairs
    naming a block outside either pool are skipped (a reading: the same rule
    as for slots).

    Parity: pinned in the oracle tests by a round trip through a second pool
    that restores every sequence's gathered contents, and by untouched
    destination blocks staying unchanged.
    """
    pairs = np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    for s, d in pairs:
        s, d = int(s), int(d)
        if 0 <= s < src_k.shape[0] and 0 <= d < dst_k.shape[0]:
            dst_k[d] = src_k[s]
            dst_v[d] = src_v[s]


def gather_sequence(cache, table_row, seq_len, block_size):
    """Logical rows ``[H_kv][seq_len][d]`` of one sequence, via its table row.

    Concatenates, in logical block order, the tiles ``cache[table_row[k]]``
    for ``k = 0 .. ceil(seq_len/B)-1`` and keeps the first ``seq_len`` rows;
    the unused rows of the last block are never read (dihengye.cn,
    "PagedAttention", section "分块 Attention 计算": block ``j`` stores keys and
    values ``(j-1)B+1 .. jB`` in 1-based numbering).

    Parity: pinned by the paged-versus-contiguous round trip and by the
    printed block-table examples in ``tests/golden/``.
    """
    num_logical = -(-int(seq_len) // block_size)
    tiles = [cache[int(table_row[k])] for k in range(num_logical)]
    if not tiles:
        h, _, d = cache.shape[1:]
        return np.zeros((h, 0, d), dtype=cache.dtype)
    rows = np.concatenate(tiles, axis=1)  # [H_kv][num_logical*B][d]
    return rows[:, : int(seq_len), :]


def quantize_reshape_and_cache(k_cache, v_cache, key32, value32, k_scale, v_scale, slot_mapping, block_size):
    """Quantize float32 K/V rows to E4M3FN codes and scatter them, in place.

    ``key32``/``value32``: ``[num_tokens][H_kv][d]`` float32 values (the new
    tokens' K and V widened exactly from their stored format); head ``h`` is
    divided by ``k_scale[h]`` (``v_scale[h]``) in float32 and encoded with
    ``formats.e4m3fn_encode``.  FP8 KV storage with a scale: youngju.dev,
    "KVキャッシュとPagedAttention — 推論メモリのすべて", section "KV量子化:
    FP8とINT8".

    Parity: the whole call is pinned against a reference built from torch
    alone (float32 division by each head's own K or V scale, clamp to +-448,
    torch's float8_e4m3fn rounding, scatter by advanced indexing), on inputs
    chosen so that a float64 division, a neighbouring head's scale or the
    other tensor's scale each change a stored code; the encoder is also
    pinned on its own.
    """
    from .formats import quantize_to_e4m3fn
    key32 = np.asarray(key32, dtype=np.float32)
    value32 = np.asarray(value32, dtype=np.float32)
    kcodes = np.stack([quantize_to_e4m3fn(key32[:, h], np.float32(k_scale[h])) for h in range(key32.shape[1])], axis=1)
    vcodes = np.stack([quantize_to_e4m3fn(value32[:, h], np.float32(v_scale[h])) for h in range(value32.shape[1])],
                      axis=1)
    reshape_and_cache(k_cache, v_cache, kcodes, vcodes, slot_mapping, block_size)
