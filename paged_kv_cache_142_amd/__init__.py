"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libpagedattn.so``
(``include/pagedattn.h``): the functions below carry the C names and only
marshal arguments (device pointers of torch tensors, sizes, dtype codes and
the current HIP stream).  Every step of the computation runs in the HIP
kernels; PyTorch is used for device memory and streams only.

``BlockManager`` (``blocks.py``) is the host-side block allocator with
reference counts and copy-on-write that produces block tables, slot mappings
and copy pairs for these calls.
"""

from __future__ import annotations

import torch

from . import _lib
from .blocks import BlockManager, PoolExhausted  # noqa: F401

PA_DTYPE_F32, PA_DTYPE_F16, PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODES = {"f32": PA_DTYPE_F32, "f16": PA_DTYPE_F16, "bf16": PA_DTYPE_BF16,
               "fp8_e4m3": PA_DTYPE_FP8_E4M3}
_TORCH_CODES = {torch.float32: PA_DTYPE_F32, torch.float16: PA_DTYPE_F16, torch.bfloat16: PA_DTYPE_BF16,
                torch.float8_e4m3fn: PA_DTYPE_FP8_E4M3, torch.uint8: PA_DTYPE_FP8_E4M3}


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = _lib.load().pa_status_string(status).decode()
        super().__init__(f"{call} failed: {msg} ({status})")


def dtype_code(t: torch.Tensor, override=None) -> int:
    """Element-format code of a tensor (``override`` may name it: 'bf16', ...)."""
    if override is not None:
        return DTYPE_CODES[override] if isinstance(override, str) else int(override)
    try:
        return _TORCH_CODES[t.dtype]
    except KeyError:
        raise ValueError(f"no element format for {t.dtype}; pass it explicitly") from None


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpagedattn must be contiguous")
    return t.data_ptr()


def _stream(stream, device):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return torch.cuda.current_stream(device).cuda_stream


def _check(status, call):
    if status != 0:
        raise PagedAttnError(status, call)


def pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, kv_dtype=None, stream=None):
    """Scatter ``key``/``value`` ``[T][H_kv][d]`` into the pools at ``slot_mapping``."""
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    _check(_lib.load().pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), int(slot_mapping.numel()),
        num_kv_heads, head_dim, block_size, num_blocks, dtype_code(k_cache, kv_dtype),
        _stream(stream, k_cache.device)), "pa_reshape_and_cache")


def pa_reshape_and_cache_fp8(key, value, k_cache, v_cache, k_scale, v_scale, slot_mapping, src_dtype=None,
                             stream=None):
    """Quantize ``key``/``value`` (fp32/fp16/bf16) to E4M3 codes with per-head
    scales and scatter them into the fp8 pools at ``slot_mapping``."""
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    _check(_lib.load().pa_reshape_and_cache_fp8(
        _ptr(key), _ptr(value), dtype_code(key, src_dtype), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(slot_mapping), int(slot_mapping.numel()), num_kv_heads, head_dim, block_size,
        num_blocks, _stream(stream, k_cache.device)), "pa_reshape_and_cache_fp8")


def pa_copy_blocks(k_cache, v_cache, block_pairs, kv_dtype=None, stream=None):
    """Copy whole blocks for each ``(src, dst)`` row of ``block_pairs`` (int64, device)."""
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    _check(_lib.load().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), int(block_pairs.numel() // 2), num_kv_heads, head_dim,
        block_size, num_blocks, dtype_code(k_cache, kv_dtype), _stream(stream, k_cache.device)),
        "pa_copy_blocks")


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, block_pairs, kv_dtype=None, stream=None):
    """Copy whole blocks ``src[s] -> dst[d]`` for each ``(s, d)`` row of
    ``block_pairs`` between two pools, one of them in pinned host memory
    (swap-out: device -> host; swap-in: host -> device)."""
    src_blocks, num_kv_heads, block_size, head_dim = src_k.shape
    dst_blocks = dst_k.shape[0]
    if tuple(dst_k.shape[1:]) != (num_kv_heads, block_size, head_dim):
        raise ValueError("source and destination pools differ in block shape")
    for t in (src_k, src_v, dst_k, dst_v):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError("pa_swap_blocks: host pools must be pinned memory (pin_memory=True)")
    device = src_k.device if src_k.is_cuda else dst_k.device
    _check(_lib.load().pa_swap_blocks(
        _ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(block_pairs), int(block_pairs.numel() // 2),
        num_kv_heads, head_dim, block_size, src_blocks, dst_blocks, dtype_code(src_k, kv_dtype),
        _stream(stream, device)), "pa_swap_blocks")


def pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_seq_len, partition_size) -> int:
    return int(_lib.load().pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_seq_len, partition_size))


def _decode_argv(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, partition_size,
                 workspace, k_scale=None, v_scale=None, kv_dtype=None, q_dtype=None, out_dtype=None, stream=None):
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    num_seqs, num_heads, _ = q.shape
    return (_ptr(out), dtype_code(out, out_dtype), _ptr(q), dtype_code(q, q_dtype), _ptr(k_cache), _ptr(v_cache),
            dtype_code(k_cache, kv_dtype), _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens),
            int(max_seq_len), num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, float(scale),
            _ptr(k_scale), _ptr(v_scale), int(partition_size), _ptr(workspace),
            int(workspace.numel() * workspace.element_size()) if workspace is not None else 0,
            _stream(stream, q.device))


def _prefill_argv(out, q, query_start, k_cache, v_cache, block_tables, seq_lens, max_seq_len, max_query_len,
                  scale, kv_dtype=None, q_dtype=None, out_dtype=None, stream=None):
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    total_q, num_heads, _ = q.shape
    return (_ptr(out), dtype_code(out, out_dtype), _ptr(q), dtype_code(q, q_dtype), _ptr(query_start), total_q,
            int(max_query_len), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache, kv_dtype), _ptr(block_tables),
            int(block_tables.shape[1]), _ptr(seq_lens), int(max_seq_len), int(seq_lens.numel()), num_heads,
            num_kv_heads, head_dim, block_size, num_blocks, float(scale), _stream(stream, q.device))


def pa_prefill(*args, **kw):
    """Causal multi-query attention of packed query rows over paged K/V.

    Arguments: ``out, q, query_start, k_cache, v_cache, block_tables,
    seq_lens, max_seq_len, max_query_len, scale``; see ``include/pagedattn.h``.
    """
    _check(_lib.load().pa_prefill(*_prefill_argv(*args, **kw)), "pa_prefill")


def prepared(name, *args, **kw):
    """A zero-argument callable that issues the C call ``name`` with these
    arguments, marshalled once (for loops that repeat an identical call).

    The tensors must stay alive and in place while the callable is used.
    """
    lib = _lib.load()
    fn = getattr(lib, name)
    if name in ("pa_decode", "pa_decode_partition", "pa_decode_reduce"):
        argv = _decode_argv(*args, **kw)
    elif name == "pa_decode_append":
        key, value = kw.pop("key"), kw.pop("value")
        argv = _decode_argv(*args, **kw) + _append_argv(key, value, args, kw)
    elif name == "pa_decode_append_cow":
        key, value, pairs = kw.pop("key"), kw.pop("value"), kw.pop("block_pairs")
        argv = _decode_argv(*args, **kw) + _append_argv_opt(key, value, args, kw) + _pairs_argv(pairs)
    elif name == "pa_decode_shared_prefix":
        gs, gp, mgs, mpl = (kw.pop(k) for k in ("group_start", "group_prefix", "max_group_size", "max_prefix_len"))
        key, value = kw.pop("key", None), kw.pop("value", None)
        argv = (_decode_argv(*args, **kw) + _group_argv(gs, gp, mgs, mpl)
                + (_append_argv(key, value, args, kw) if key is not None else (None, None)))
    elif name == "pa_prefill":
        argv = _prefill_argv(*args, **kw)
    elif name == "pa_reshape_and_cache":
        key, value, k_cache, v_cache, slot_mapping = args
        nb, hkv, bs, d = k_cache.shape
        argv = (_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), int(slot_mapping.numel()),
                hkv, d, bs, nb, dtype_code(k_cache, kw.get("kv_dtype")), _stream(kw.get("stream"), k_cache.device))
    elif name == "pa_reshape_and_cache_fp8":
        key, value, k_cache, v_cache, k_scale, v_scale, slot_mapping = args
        nb, hkv, bs, d = k_cache.shape
        argv = (_ptr(key), _ptr(value), dtype_code(key, kw.get("src_dtype")), _ptr(k_cache), _ptr(v_cache),
                _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping), int(slot_mapping.numel()), hkv, d, bs, nb,
                _stream(kw.get("stream"), k_cache.device))
    elif name == "pa_copy_blocks":
        k_cache, v_cache, block_pairs = args
        nb, hkv, bs, d = k_cache.shape
        argv = (_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), int(block_pairs.numel() // 2), hkv, d, bs, nb,
                dtype_code(k_cache, kw.get("kv_dtype")), _stream(kw.get("stream"), k_cache.device))
    else:
        raise ValueError(name)
    c_args = [t(a) if a is not None else None for t, a in zip(fn.argtypes, argv)]

    def call():
        status = fn(*c_args)
        if status != 0:
            raise PagedAttnError(status, name)
    return call


def _decode_call(name, *args, **kw):
    _check(getattr(_lib.load(), name)(*_decode_argv(*args, **kw)), name)


def pa_decode(*args, **kw):
    """``out[i][h] = softmax(scale * K_i q[i][h]) V_i`` over each sequence's paged K/V.

    Arguments: ``out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len,
    scale, partition_size, workspace`` and, for FP8 pools, ``k_scale`` and
    ``v_scale``; see ``include/pagedattn.h``.
    """
    _decode_call("pa_decode", *args, **kw)


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, partition_size,
                      k_scale=None, v_scale=None, kv_dtype=None, q_dtype=None, out_dtype=None, stream=None):
    """``pa_decode`` with the split-KV workspace in the library's static
    device array (no workspace argument; the call allocates nothing)."""
    argv = _decode_argv(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, partition_size,
                        None, k_scale=k_scale, v_scale=v_scale, kv_dtype=kv_dtype, q_dtype=q_dtype,
                        out_dtype=out_dtype, stream=stream)
    _check(_lib.load().pa_decode_noalloc(*argv[:21], argv[23]), "pa_decode_noalloc")


def _append_argv(key, value, args, kw):
    q = kw["q"] if "q" in kw else args[1]
    k_cache = kw["k_cache"] if "k_cache" in kw else args[2]
    want = (q.shape[0], k_cache.shape[1], k_cache.shape[3])
    if tuple(key.shape) != want or tuple(value.shape) != want:
        raise ValueError(f"key and value must be [num_seqs, num_kv_heads, head_dim] = {list(want)}")
    if key.dtype != k_cache.dtype or value.dtype != k_cache.dtype:
        raise ValueError("key and value must be in the pool's element format")
    return (_ptr(key), _ptr(value))


def _append_argv_opt(key, value, args, kw):
    """The new rows, or two null pointers when neither is given."""
    if key is None and value is None:
        return (None, None)
    if key is None or value is None:
        raise ValueError("give both key and value, or neither")
    return _append_argv(key, value, args, kw)


def pa_decode_append(*args, key, value, **kw):
    """``pa_decode`` that first stores each sequence's newest token
    (``key``/``value`` ``[num_seqs][num_kv_heads][head_dim]``) at position
    ``seq_lens - 1``; the other arguments are ``pa_decode``'s."""
    argv = _decode_argv(*args, **kw) + _append_argv(key, value, args, kw)
    _check(_lib.load().pa_decode_append(*argv), "pa_decode_append")


def pa_decode_append_cow(*args, key, value, block_pairs, **kw):
    """``pa_copy_blocks`` with ``block_pairs`` (int64 ``[P][2]`` (source,
    destination), device), then ``pa_decode_append``; one launch where the
    partition kernel stores the new tokens.  ``key=None, value=None``: the
    copies, then ``pa_decode`` (one launch for the FP8 matrix-core shape)."""
    argv = _decode_argv(*args, **kw) + _append_argv_opt(key, value, args, kw) + _pairs_argv(block_pairs)
    _check(_lib.load().pa_decode_append_cow(*argv), "pa_decode_append_cow")


def _pairs_argv(block_pairs):
    if block_pairs is None:
        return (None, 0)
    if block_pairs.dtype != torch.int64 or block_pairs.numel() % 2:
        raise ValueError("block_pairs must be int64 (source, destination) pairs")
    return (_ptr(block_pairs), int(block_pairs.numel() // 2))


def pa_decode_shared_prefix(*args, group_start, group_prefix, max_group_size, max_prefix_len, key=None, value=None,
                            **kw):
    """``pa_decode`` reading each group's shared prompt partitions once.

    ``group_start`` (int32, ``[G+1]``) and ``group_prefix`` (int32, ``[G]``
    shared tokens) are device tensors; the other arguments are ``pa_decode``'s.
    """
    argv = (_decode_argv(*args, **kw) + _group_argv(group_start, group_prefix, max_group_size, max_prefix_len)
            + (_append_argv(key, value, args, kw) if key is not None else (None, None)))
    _check(_lib.load().pa_decode_shared_prefix(*argv), "pa_decode_shared_prefix")


def _group_argv(group_start, group_prefix, max_group_size, max_prefix_len):
    if group_start.numel() != group_prefix.numel() + 1:
        raise ValueError("group_start needs one entry more than group_prefix")
    if group_start.dtype != torch.int32 or group_prefix.dtype != torch.int32:
        raise ValueError("group_start and group_prefix must be int32")
    return (_ptr(group_start), _ptr(group_prefix), int(group_prefix.numel()), int(max_group_size),
            int(max_prefix_len))


def pa_decode_partition(*args, **kw):
    """First launch of ``pa_decode`` (partition states into the workspace)."""
    _decode_call("pa_decode_partition", *args, **kw)


def pa_decode_reduce(*args, **kw):
    """Second launch of ``pa_decode`` (merge of the partition states)."""
    _decode_call("pa_decode_reduce", *args, **kw)
