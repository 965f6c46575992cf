"""Float64 CPU oracle for paged single-query decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, header, table or helper with the
HIP library; both sides receive the same raw input arrays from the seeded
generators in ``workloads/`` and compute independently.

What it computes, and the passage each function follows:

* ``formats``   -- exact widening of stored K/V/q elements (fp32, fp16, bf16)
  and the 256-entry OCP E4M3FN decode table written from the format's
  sign/exponent/mantissa definition.  FP8 KV storage with a scale is named on
  youngju.dev, "KVキャッシュとPagedAttention — 推論メモリのすべて", section
  "KV量子化: FP8とINT8" (one byte per element; a scale is needed).
* ``paging``    -- the physical pool ``[num_blocks][H_kv][B][d]``, the scatter
  of new tokens through a slot mapping, the block copy used by copy-on-write,
  the block transfer between pools of preemption by swapping (section
  "プリエンプション戦略" of the explainer below), and the gather of a
  sequence's logical K/V through its block table
  (0h-n0.github.io, "論文解説: Efficient Memory Management for Large Language
  Model Serving with PagedAttention", sections "PagedAttentionのメモリ管理"
  and "Copy-on-Write（CoW）によるメモリ共有"; dihengye.cn, "PagedAttention",
  section "Block Table 结构").
* ``attention`` -- the plain definition softmax(q K^T * scale) V for one
  query row over the gathered keys (0h-n0.github.io explainer, section
  "Attention計算"), the block-by-block online-softmax recurrence of
  auturnal.com, "メモリ予算内での言語モデルのサービング", equation (4), and
  the log-sum-exp merge of per-partition partial states that the same
  recurrence implies.
* ``prefill``   -- multi-query (prefill / chunked prefill) attention over the
  same paged K/V: each new token's query attends causally to the cached
  tokens up to its own position (the explainer's attention definition,
  restricted; auturnal.com review, sections 1 and 7, on prefill versus
  decode shapes).
* ``accounting`` -- KV bytes per token (equation (1) of the auturnal.com
  review; youngju.dev section "KVキャッシュはなぜメモリを消費するのか"),
  page-tail waste and its bound (equation (2)), the exact mean tail waste for
  uniform lengths (equation (3)) and the reservation comparison of section 5.

Every floating-point result is computed in float64.  Parity status of each
function is listed in its docstring; all are pinned by ``tests/test_oracle*.py``
against closed forms, printed worked examples, library routines or brute force.
"""

from . import accounting, attention, formats, paging, prefill  # noqa: F401
from .attention import (  # noqa: F401
    dense_attention,
    lse_merge,
    online_softmax_attention,
    paged_decode,
    paged_decode_row,
    split_kv_attention,
)
from .prefill import paged_prefill, paged_prefill_rowwise  # noqa: F401
from .formats import decode_elements, e4m3fn_encode, e4m3fn_table, quantize_to_e4m3fn  # noqa: F401
from .paging import (  # noqa: F401
    copy_blocks,
    gather_sequence,
    quantize_reshape_and_cache,
    reshape_and_cache,
    swap_blocks,
)
