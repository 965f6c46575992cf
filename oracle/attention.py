"""Single-query attention over paged K/V, in float64.

Test infrastructure only (see the package docstring).

The result the method must reach is plain scaled-dot-product attention of
the current token's query against every cached key and value of its
sequence: ``softmax(q K^T * scale) V`` with ``q`` of shape ``1 x d``, ``K``
and ``V`` of shape ``n x d`` (0h-n0.github.io, "論文解説: Efficient Memory
Management for Large Language Model Serving with PagedAttention", section
"Attention計算"; youngju.dev, "KVキャッシュとPagedAttention — 推論メモリのす
べて", section "核心原理: KVキャッシュとは何か").  Paging only changes where
the rows live: the explainer's same section computes per-block scores
``A_j = q K_j^T * scale`` over the blocks the table names and applies one
softmax over their concatenation, which equals the plain definition after
the gather.

``dense_attention`` is that definition and ``paged_decode`` applies it after
gathering each sequence through its table.  ``online_softmax_attention`` is
the block recurrence of auturnal.com, "メモリ予算内での言語モデルのサービン
グ", equation (4), and ``split_kv_attention``/``lse_merge`` apply the same
recurrence to partition states; those two exist to pin the oracle and to
state what the GPU's split-KV path must reproduce.

Readings (the pages leave these open):

* query head ``h`` reads kv head ``h // G`` with ``G = H_q / H_kv``
  (consecutive query heads share a kv head; youngju.dev section "GQAとMQA"
  only says query heads are grouped);
* ``d_v = d_k = d``;
* ``scale`` is the float32 value handed to the GPU, widened exactly;
* an empty sequence (``seq_len == 0``) produces a zero row.
"""

from __future__ import annotations

import numpy as np

from .formats import decode_elements
from .paging import gather_sequence


def dense_attention(q, keys, values, scale):
    """``softmax(keys @ q * scale) @ values`` for one query, float64.

    ``q``: ``[d]``; ``keys``/``values``: ``[n][d]``.  The softmax subtracts the
    maximum score before exponentiating, which leaves the result unchanged and
    keeps ``exp`` finite for large logits (the auturnal.com review, section 6,
    asks for extreme-logit checks for exactly this reason).

    Parity: pinned against ``torch.nn.functional.scaled_dot_product_attention``
    in float64, and by closed forms (one token, equal scores, two tokens, a
    dominant logit).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    scores = (keys @ q) * float(scale)
    weights = np.exp(scores - scores.max())
    return (weights / weights.sum()) @ values


def _dequantized_rows(cache, table_row, seq_len, block_size, kv_dtype, head_scale):
    rows = decode_elements(gather_sequence(cache, table_row, seq_len, block_size), kv_dtype)
    if head_scale is not None:
        rows = rows * np.asarray(head_scale, dtype=np.float32).astype(np.float64)[:, None, None]
    return rows  # [H_kv][seq_len][d]


def paged_decode_row(q_row, q_dtype, k_cache, v_cache, kv_dtype, table_row, seq_len,
                     block_size, scale, k_scale=None, v_scale=None):
    """Output ``[H_q][d]`` (float64) of one sequence.

    ``q_row``: raw ``[H_q][d]`` query elements of format ``q_dtype``;
    ``k_cache``/``v_cache``: raw pools ``[num_blocks][H_kv][B][d]``;
    ``table_row``: the sequence's block-table row; ``k_scale``/``v_scale``:
    float32 per-kv-head scales for ``fp8_e4m3`` storage (``None`` otherwise).

    Steps: gather the sequence's K and V through the table, widen (and
    dequantize) to float64, then apply ``dense_attention`` per query head on
    kv head ``h // G``.
    """
    q = decode_elements(q_row, q_dtype)
    num_heads = q.shape[0]
    num_kv_heads = k_cache.shape[1]
    group = num_heads // num_kv_heads
    keys = _dequantized_rows(k_cache, table_row, seq_len, block_size, kv_dtype, k_scale)
    values = _dequantized_rows(v_cache, table_row, seq_len, block_size, kv_dtype, v_scale)
    out = np.zeros(q.shape, dtype=np.float64)
    for h in range(num_heads):
        out[h] = dense_attention(q[h], keys[h // group], values[h // group], scale)
    return out


def paged_decode(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                 block_size, scale, k_scale=None, v_scale=None, rows=None):
    """Output ``[N][H_q][d]`` (float64) for every sequence, or for ``rows``.

    With ``rows`` given, only those sequences are computed and the result has
    ``len(rows)`` entries in that order.
    """
    indices = range(len(seq_lens)) if rows is None else rows
    return np.stack([
        paged_decode_row(q[i], q_dtype, k_cache, v_cache, kv_dtype, block_tables[i],
                         int(seq_lens[i]), block_size, scale, k_scale, v_scale)
        for i in indices
    ])


def online_softmax_attention(q, keys, values, scale, block_size, return_state=False):
    """Attention by the block recurrence of equation (4), float64.

    Scores are visited ``block_size`` at a time in token order.  The state
    starts at ``m = -inf, l = 0, acc = 0`` (a reading: the equation gives only
    the update); for a block with scores ``s_j`` and value rows ``v_j``::

        m'   = max(m, max_j s_j)
        l'   = exp(m - m') * l   + sum_j exp(s_j - m')
        acc' = exp(m - m') * acc + sum_j exp(s_j - m') * v_j

    The value accumulator is rescaled by the same factor as ``l`` (the
    review's note under equation (4)).  The result is ``acc / l``.  With
    ``return_state`` the unnormalised ``(m, l, acc)`` is returned instead.

    Parity: pinned against ``dense_attention`` (max abs difference <= 1e-12)
    at block sizes 1, 2, 3, 7, 16, 32, 512 and n.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m = -np.inf
    l = 0.0
    acc = np.zeros(values.shape[1], dtype=np.float64)
    for start in range(0, keys.shape[0], block_size):
        s = (keys[start:start + block_size] @ q) * float(scale)
        v = values[start:start + block_size]
        m_new = max(m, float(s.max()))
        alpha = np.exp(m - m_new)  # exp(-inf) = 0 on the first block
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        acc = alpha * acc + p @ v
        m = m_new
    if return_state:
        return m, l, acc
    if l == 0.0:
        return np.zeros_like(acc)
    return acc / l


def lse_merge(ms, ls, accs):
    """Merge partition states ``(m_p, l_p, acc_p)`` into one output row.

    This is equation (4) applied with each partition's state as one "block":
    ``M = max_p m_p``, ``L = sum_p exp(m_p - M) l_p``,
    ``A = sum_p exp(m_p - M) acc_p``, result ``A / L``, summed in partition
    order.

    Parity: pinned through ``split_kv_attention`` against ``dense_attention``.
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    big_m = ms.max()
    w = np.exp(ms - big_m)
    return (w[:, None] * accs).sum(axis=0) / (w * ls).sum()


def split_kv_attention(q, keys, values, scale, block_size, partition_size):
    """Attention with tokens split into partitions of ``partition_size``.

    Partition ``p`` covers tokens ``[p*P, min((p+1)*P, n))`` (a reading;
    ``P`` a multiple of ``block_size`` so partitions hold whole blocks and no
    partition is empty).  Each partition runs the block recurrence from the
    initial state; the states are merged by ``lse_merge``.
    """
    n = keys.shape[0]
    states = [
        online_softmax_attention(q, keys[s:s + partition_size], values[s:s + partition_size],
                                 scale, block_size, return_state=True)
        for s in range(0, n, partition_size)
    ]
    ms, ls, accs = zip(*states)
    return lse_merge(ms, ls, np.stack(accs))
