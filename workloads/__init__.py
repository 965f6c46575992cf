"""Seeded synthetic inputs for paged decode attention.

This module is shared by the GPU path's tests and benchmark and by the
oracle's callers; it holds no step of the method's arithmetic.  It only
draws random numbers (NumPy PCG64, seeded), rounds them to the stored
formats with library casts (PyTorch/NumPy), and lays out the block-table
structure of each workload: which physical blocks each sequence owns, the
slot of every token, and which block pairs a copy step uses.

The five workloads are synthetic stand-ins for the serving traces the pages
measure on (the pages' datasets are not used):

* ``tiny``           -- fp32, 4 sequences of 1/17/40/100 tokens, 4 heads, d=64
* ``gqa``            -- bf16, 64 sequences, lengths uniform on 1..4096, 32/8 heads
* ``mha``            -- fp16, 256 sequences, lengths uniform on 1..2048, 40/40 heads
* ``shared_prefix``  -- bf16, 8 prompts x 6 beams sharing the prompt's blocks
* ``long_fp8``       -- fp8 E4M3 KV with per-kv-head scales, 16 x 32768 tokens, 64/8 heads

and, for multi-query attention over the same pool, ``prefill`` -- bf16,
16 sequences of 1..2048 tokens, 32/8 heads, every token (or the last chunk of
each sequence) a query.
"""

from .generators import (  # noqa: F401
    DecodeWorkload,
    PrefillWorkload,
    SharedPrefixWorkload,
    build_decode_workload,
    build_prefill_workload,
    gqa,
    long_fp8,
    make,
    mha,
    prefill,
    shared_prefix,
    tiny,
)
