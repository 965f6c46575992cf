"""KV byte accounting and page-tail waste, exact integer/rational arithmetic.

Test infrastructure only (see the package docstring).  Follows auturnal.com,
"メモリ予算内での言語モデルのサービング：注意機構、ページング、スケジューリ
ング", equations (1)-(3) and sections 3 and 5, and youngju.dev,
"KVキャッシュとPagedAttention — 推論メモリのすべて", sections
"KVキャッシュはなぜメモリを消費するのか" and "断片化の問題".
"""

from __future__ import annotations

from fractions import Fraction


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes):
    """Uncompressed K+V bytes held per token: ``2 * L * H_kv * d * b``.

    The factor two counts keys and values (equation (1) without the sum).
    """
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def kv_bytes(seq_lens, num_layers, num_kv_heads, head_dim, elem_bytes):
    """Equation (1): ``M_KV = 2 L H_kv d b * sum_i T_i``."""
    return kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes) * sum(
        int(t) for t in seq_lens)


def blocks_needed(seq_len, block_size):
    """Pages a request of ``seq_len`` tokens occupies: ``ceil(T / B)``."""
    return -(-int(seq_len) // block_size)


def tail_waste(seq_lens, block_size):
    """Equation (2): ``W = sum_i (B * ceil(T_i / B) - T_i)`` in token slots."""
    return sum(block_size * blocks_needed(t, block_size) - int(t) for t in seq_lens)


def tail_waste_bound(num_requests, block_size):
    """Right-hand side of equation (2) for non-empty requests: ``N (B - 1)``."""
    return num_requests * (block_size - 1)


def mean_tail_waste_uniform(block_size, max_len):
    """Exact mean tail waste for lengths uniform on ``1..max_len``.

    Computed by enumeration with rationals, not from the closed form, so that
    equation (3) (``(B-1)/2`` when ``max_len`` is a positive multiple of
    ``B``) can be checked against it.
    """
    total = sum(tail_waste([t], block_size) for t in range(1, max_len + 1))
    return Fraction(total, max_len)


def mean_reservation_waste_uniform(reserved, max_len):
    """Mean unused slots when every request reserves ``reserved`` slots and
    lengths are uniform on ``1..max_len`` (section 5's comparison), exact."""
    total = sum(reserved - t for t in range(1, max_len + 1))
    return Fraction(total, max_len)


def reservation_waste(reserved, used):
    """Slots left unused by a contiguous reservation of ``reserved`` slots
    of which ``used`` are filled (youngju.dev section "断片化の問題")."""
    return reserved - used
