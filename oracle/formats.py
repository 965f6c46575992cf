"""Exact float64 values of the stored element formats.

Test infrastructure only (see the package docstring).

Stored formats and how they widen to float64:

* ``"f32"``  -- IEEE binary32, given as a ``float32`` array; the cast is exact.
* ``"f16"``  -- IEEE binary16, given as its raw ``uint16`` bit patterns; the cast
  through ``numpy.float16`` is exact.
* ``"bf16"`` -- bfloat16, given as raw ``uint16`` bit patterns.  A bfloat16 is
  the upper half of a binary32 with the same sign and exponent fields, so the
  value is the binary32 whose high 16 bits are the pattern and whose low 16
  bits are zero.
* ``"fp8_e4m3"`` -- the OCP 8-bit float E4M3FN, given as raw ``uint8`` codes,
  decoded by a 256-entry table built below from the field definition.  The
  pages name FP8 KV storage (one byte per element, roughly half of FP16) but
  not the exact encoding (youngju.dev, "KVキャッシュとPagedAttention — 推論メモ
  リのすべて", section "KV量子化: FP8とINT8"); E4M3FN is the reading taken here
  because it is the FP8 format of the target hardware's conversion
  instructions.  Its stored value is multiplied by a float32 per-kv-head scale
  (``value = code_value * scale``), which the same section says an 8-bit KV
  format needs.
"""

from __future__ import annotations

import numpy as np

KV_DTYPES = ("f32", "f16", "bf16", "fp8_e4m3")


def e4m3fn_table() -> np.ndarray:
    """Float64 value of every E4M3FN code 0..255.

    Field layout of a code: bit 7 sign, bits 6..3 a biased exponent (bias 7),
    bits 2..0 a mantissa.  Exponent field 0 encodes subnormals
    ``mantissa/8 * 2**(1-7)``; fields 1..15 encode ``(1 + mantissa/8) *
    2**(exponent-7)``, except that exponent 15 with mantissa 7 is NaN (the
    "FN" variant has no infinities, so the largest finite magnitude is
    ``1.75 * 2**8 = 448``).

    Parity: pinned exhaustively against ``torch.float8_e4m3fn`` and at
    hand-checked codes (0, smallest subnormal, 1.0, 448, NaN).
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exponent = (code >> 3) & 0xF
        mantissa = code & 0x7
        if exponent == 0xF and mantissa == 0x7:
            table[code] = np.nan
        elif exponent == 0:
            table[code] = sign * (mantissa / 8.0) * 2.0 ** (1 - 7)
        else:
            table[code] = sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)
    return table


_E4M3FN = e4m3fn_table()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (``uint16``) as float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return as_f32.astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of binary16 bit patterns (``uint16``) as float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def e4m3fn_encode(x) -> np.ndarray:
    """E4M3FN codes of float values: nearest code, ties to the even code,
    saturated at +-448; NaN gives 0x7F.

    The nearest code is found by comparing against every finite code value
    (exact in float64).  On a tie the even code wins, which is the code whose
    mantissa field is even (round to nearest even).  Values beyond the
    largest finite magnitude, infinities included, become +-448, the
    saturating reading of storing a value too large for the format.

    Parity: pinned against torch's float8_e4m3fn conversion on every
    bfloat16 value inside the format's range and on dense float32 samples,
    and against hand-picked ties, subnormals and overflow cases.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.array([c for c in range(256) if not np.isnan(_E4M3FN[c])], dtype=np.int64)
    values = _E4M3FN[finite]
    out = np.empty(x.shape, dtype=np.uint8)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    for n, v in enumerate(flat):
        if np.isnan(v):
            res[n] = 0x7F
            continue
        v = min(max(v, -448.0), 448.0)
        dist = np.abs(values - v)
        best = np.flatnonzero(dist == dist.min())
        codes = finite[best]
        if len(codes) > 1:  # tie between two neighbours (or +0/-0)
            same_sign = codes[(codes >= 0x80) == bool(np.signbit(v))]
            codes = same_sign if len(same_sign) else codes
            even = codes[(codes & 1) == 0]
            codes = even if len(even) else codes
        res[n] = codes[0]
    return out


def quantize_to_e4m3fn(x32, scale32) -> np.ndarray:
    """Codes of ``x / scale``: the quotient is the IEEE float32 division of
    the float32 value by the float32 scale, then ``e4m3fn_encode``."""
    q = np.asarray(x32, dtype=np.float32) / np.asarray(scale32, dtype=np.float32)
    return e4m3fn_encode(q.astype(np.float32))


def decode_elements(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Float64 values of stored elements of format ``dtype`` (no scale)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return f16_bits_to_f64(raw)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "fp8_e4m3":
        return _E4M3FN[np.asarray(raw, dtype=np.uint8)]
    raise ValueError(f"unknown element format {dtype!r}")
