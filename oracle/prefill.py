"""Multi-query (prefill / chunked prefill) attention over paged K/V, float64.

Test infrastructure only (see the package docstring).

A prefill step runs attention for many new tokens of a sequence at once.
Their keys and values are written into the sequence's blocks first (the
same scatter as decode), and each new token's query attends to every cached
token up to and including its own position: the plain scaled-dot-product
attention ``softmax(q K^T * scale) V`` of the explainer (0h-n0.github.io,
"論文解説: Efficient Memory Management for Large Language Model Serving with
PagedAttention", section "Attention計算") restricted, for the query at
position ``p``, to keys ``0 .. p``.  The pages contrast the two workloads:
prefill and decode steps have different computational shapes (auturnal.com,
"メモリ予算内での言語モデルのサービング", section 7), and long prefills
dominate some workloads (same page, section 1); the block tables and the
pool are the same ones decode reads.

Readings (the pages leave these open):

* the ``Q_i`` query rows of sequence ``i`` are its last ``Q_i`` tokens: row
  ``j`` sits at position ``T_i - Q_i + j`` where ``T_i = seq_lens[i]`` counts
  every cached token including the chunk (``Q_i == T_i`` is a full prefill,
  ``Q_i < T_i`` a chunk appended to an existing context);
* the query rows of all sequences are packed: sequence ``i`` owns rows
  ``query_start[i] .. query_start[i+1] - 1`` of ``q`` and of the output;
* GQA mapping, ``d_v = d_k``, the float32 scale and FP8 dequantisation are as
  for decode (``attention`` module).

``paged_prefill`` is that definition, one matrix product per (sequence,
head) with the causal mask applied before a max-subtracted softmax.
``paged_prefill_rowwise`` computes the same rows one at a time with
``dense_attention`` over the truncated key list; it exists to pin the first.

Parity: pinned in ``tests/test_oracle_prefill.py`` against the row-by-row
form, against decode (the last row of a chunk is the decode output), against
``torch.nn.functional.scaled_dot_product_attention`` in float64 with a causal
mask, and on extreme logits.
"""

from __future__ import annotations

import numpy as np

from .attention import _dequantized_rows, dense_attention
from .formats import decode_elements


def _positions(seq_len, num_rows):
    return np.arange(int(seq_len) - int(num_rows), int(seq_len), dtype=np.int64)


def paged_prefill(q, q_dtype, query_start, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                  block_size, scale, k_scale=None, v_scale=None, seqs=None):
    """Output ``[total_q][H_q][d]`` (float64): causal attention of every
    packed query row over its sequence's paged K/V.

    ``q``: raw ``[total_q][H_q][d]`` of format ``q_dtype``; ``query_start``:
    ``[N+1]``; ``k_cache``/``v_cache``: raw pools; ``seq_lens``: ``[N]``.
    With ``seqs`` given, only those sequences' rows are computed (others stay
    zero).
    """
    qf = decode_elements(np.asarray(q), q_dtype)
    total_q, num_heads, d = qf.shape
    num_kv_heads = k_cache.shape[1]
    group = num_heads // num_kv_heads
    out = np.zeros((total_q, num_heads, d), dtype=np.float64)
    for i in (range(len(seq_lens)) if seqs is None else seqs):
        r0, r1 = int(query_start[i]), int(query_start[i + 1])
        if r1 == r0:
            continue
        T = int(seq_lens[i])
        keys = _dequantized_rows(k_cache, block_tables[i], T, block_size, kv_dtype, k_scale)
        values = _dequantized_rows(v_cache, block_tables[i], T, block_size, kv_dtype, v_scale)
        pos = _positions(T, r1 - r0)
        masked = np.arange(T)[None, :] > pos[:, None]  # key after the query's position
        for h in range(num_heads):
            s = (qf[r0:r1, h, :] @ keys[h // group].T) * float(scale)
            s[masked] = -np.inf
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[r0:r1, h, :] = (w / w.sum(axis=1, keepdims=True)) @ values[h // group]
    return out


def paged_prefill_rowwise(q, q_dtype, query_start, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                          block_size, scale, k_scale=None, v_scale=None):
    """The same rows one at a time: ``dense_attention`` of each query over
    the keys and values at positions ``0 .. p``."""
    qf = decode_elements(np.asarray(q), q_dtype)
    total_q, num_heads, d = qf.shape
    group = num_heads // k_cache.shape[1]
    out = np.zeros((total_q, num_heads, d), dtype=np.float64)
    for i in range(len(seq_lens)):
        r0, r1 = int(query_start[i]), int(query_start[i + 1])
        T = int(seq_lens[i])
        keys = _dequantized_rows(k_cache, block_tables[i], T, block_size, kv_dtype, k_scale)
        values = _dequantized_rows(v_cache, block_tables[i], T, block_size, kv_dtype, v_scale)
        for j, p in enumerate(_positions(T, r1 - r0)):
            for h in range(num_heads):
                out[r0 + j, h] = dense_attention(qf[r0 + j, h], keys[h // group][: p + 1],
                                                 values[h // group][: p + 1], scale)
    return out
