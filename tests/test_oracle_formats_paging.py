"""Pins for the oracle's element formats and paging (CPU only).

Each check ties the oracle to something other than itself: a library
conversion routine, hand-decoded codes, the block-table examples the pages
print (``tests/golden/block_tables.json``), or a contiguous round trip.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats, paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------- formats


def test_e4m3fn_table_matches_torch_exhaustively():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.e4m3fn_table()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    finite = ~np.isnan(ref)
    assert np.array_equal(ours[finite], ref[finite])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0),
])
def test_e4m3fn_hand_decoded_codes(code, value):
    assert formats.e4m3fn_table()[code] == value


def test_e4m3fn_nan_codes_and_negative_zero():
    t = formats.e4m3fn_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert int(np.isnan(t).sum()) == 2
    assert t[0x80] == 0.0 and np.signbit(t[0x80])


def test_bf16_widening_matches_torch_exhaustively():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = formats.bf16_bits_to_f64(bits)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_f16_widening_matches_torch_exhaustively():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    ours = formats.f16_bits_to_f64(bits)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_bf16_known_patterns():
    assert formats.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert formats.bf16_bits_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert formats.bf16_bits_to_f64(np.array([0x3F81], np.uint16))[0] == 1.0 + 2.0 ** -7


# ----------------------------------------------------------------- paging


def _tagged_pool(num_blocks, heads, block_size, dim):
    """Pool whose element (b, h, r, c) encodes its own coordinates."""
    b, h, r, c = np.meshgrid(np.arange(num_blocks), np.arange(heads), np.arange(block_size),
                             np.arange(dim), indexing="ij")
    return (b * 1_000_000 + h * 10_000 + r * 100 + c).astype(np.int64)


@pytest.mark.parametrize("example", _golden("block_tables.json")["examples"], ids=lambda e: e["name"])
def test_gather_follows_printed_block_tables(example):
    B = example["block_size"]
    pool = _tagged_pool(16, 2, B, 3)
    rows = paging.gather_sequence(pool, example["table"], example["seq_len"], B)
    assert rows.shape == (2, example["seq_len"], 3)
    for t in range(example["seq_len"]):
        want_block = example["table"][t // B]
        assert rows[1, t, 2] == want_block * 1_000_000 + 1 * 10_000 + (t % B) * 100 + 2
    if "tokens_per_block" in example:
        counts = [min(B, example["seq_len"] - k * B) for k in range(len(example["table"]))]
        assert counts == example["tokens_per_block"]
    if "token_blocks" in example:
        for first, last, phys in example["token_blocks"]:
            assert rows[0, first, 0] // 1_000_000 == phys
            assert rows[0, last, 0] // 1_000_000 == phys


def _contiguous_case(rng, seq_lens, heads, dim, block_size, spare=5):
    """Contiguous K/V per sequence, random physical tables, slot mapping."""
    need = [-(-t // block_size) for t in seq_lens]
    pool_size = sum(need) + spare
    perm = rng.permutation(pool_size)
    tables, start = [], 0
    for n in need:
        tables.append(perm[start:start + n])
        start += n
    keys = [rng.standard_normal((t, heads, dim)) for t in seq_lens]
    values = [rng.standard_normal((t, heads, dim)) for t in seq_lens]
    slots = [np.array([tab[t // block_size] * block_size + t % block_size for t in range(T)], np.int64)
             for tab, T in zip(tables, seq_lens)]
    return pool_size, tables, keys, values, slots


@pytest.mark.parametrize("block_size", [1, 3, 16, 32])
def test_scatter_then_gather_round_trips_bitwise(block_size):
    rng = np.random.default_rng(11)
    B = block_size
    seq_lens = [1, B - 1 if B > 1 else 1, B, B + 1, 3 * B + 2, 100]
    heads, dim = 3, 8
    pool_size, tables, keys, values, slots = _contiguous_case(rng, seq_lens, heads, dim, B)
    kc = np.full((pool_size, heads, B, dim), np.nan)
    vc = np.full((pool_size, heads, B, dim), np.nan)
    for k, v, s in zip(keys, values, slots):
        paging.reshape_and_cache(kc, vc, k, v, s, B)
    for i, T in enumerate(seq_lens):
        gk = paging.gather_sequence(kc, tables[i], T, B)
        gv = paging.gather_sequence(vc, tables[i], T, B)
        assert np.array_equal(gk, keys[i].transpose(1, 0, 2))
        assert np.array_equal(gv, values[i].transpose(1, 0, 2))


def test_scatter_skips_negative_slots_and_touches_nothing_else():
    kc = np.zeros((4, 2, 4, 3))
    vc = np.zeros((4, 2, 4, 3))
    key = np.ones((3, 2, 3))
    value = 2 * np.ones((3, 2, 3))
    paging.reshape_and_cache(kc, vc, key, value, np.array([5, -1, 14]), 4)
    assert np.all(kc[1, :, 1] == 1) and np.all(vc[1, :, 1] == 2)
    assert np.all(kc[3, :, 2] == 1) and np.all(vc[3, :, 2] == 2)
    assert kc.sum() == 2 * 2 * 3 and vc.sum() == 2 * 2 * 2 * 3


def test_copy_blocks_copies_whole_blocks_and_leaves_the_rest():
    kc = _tagged_pool(8, 2, 4, 3).astype(np.float64)
    vc = -kc
    k0, v0 = kc.copy(), vc.copy()
    paging.copy_blocks(kc, vc, np.array([[1, 6], [3, 7], [1, 5]]))
    for s, d in [(1, 6), (3, 7), (1, 5)]:
        assert np.array_equal(kc[d], k0[s]) and np.array_equal(vc[d], v0[s])
    for b in [0, 1, 2, 3, 4]:
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])


def test_copy_blocks_reads_contents_from_before_the_call():
    kc = _tagged_pool(4, 1, 2, 1).astype(np.float64)
    vc = kc.copy()
    k0 = kc.copy()
    # block 1 is both a destination and (later in the list) a source
    paging.copy_blocks(kc, vc, np.array([[0, 1], [1, 2]]))
    assert np.array_equal(kc[1], k0[0]) and np.array_equal(kc[2], k0[1])


def test_copy_on_write_copy_preserves_logical_contents():
    """A sequence remapped to a copied block reads the same logical rows."""
    rng = np.random.default_rng(3)
    B, heads, dim = 4, 2, 5
    pool_size, tables, keys, values, slots = _contiguous_case(rng, [10], heads, dim, B, spare=3)
    kc = np.zeros((pool_size, heads, B, dim))
    vc = np.zeros((pool_size, heads, B, dim))
    paging.reshape_and_cache(kc, vc, keys[0], values[0], slots[0], B)
    used = set(int(x) for x in tables[0])
    spare = [b for b in range(pool_size) if b not in used]
    table = tables[0].copy()
    paging.copy_blocks(kc, vc, np.array([[table[2], spare[0]]]))
    table[2] = spare[0]
    assert np.array_equal(paging.gather_sequence(kc, table, 10, B), keys[0].transpose(1, 0, 2))
    assert np.array_equal(paging.gather_sequence(vc, table, 10, B), values[0].transpose(1, 0, 2))


def test_package_exports():
    for name in ["dense_attention", "paged_decode", "online_softmax_attention", "split_kv_attention",
                 "lse_merge", "reshape_and_cache", "copy_blocks", "gather_sequence", "e4m3fn_table"]:
        assert callable(getattr(oracle, name))


# --------------------------------------------------------- fp8 encoder


def test_e4m3fn_encode_round_trips_every_finite_code():
    t = formats.e4m3fn_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(formats.e4m3fn_encode(t[codes]), codes)


def test_e4m3fn_encode_matches_torch_on_all_bf16_values_in_range():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = formats.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    vals = vals[keep]
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.e4m3fn_encode(vals), ref)


def test_e4m3fn_encode_matches_torch_on_float32_samples():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.uniform(-448, 448, 5000),
                        rng.standard_normal(5000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.e4m3fn_encode(x.astype(np.float64)), ref)


@pytest.mark.parametrize("value,code", [
    (2.0 ** -10, 0x00),            # half the smallest subnormal: tie, even code 0
    (1.5 * 2.0 ** -9, 0x02),       # tie between codes 1 and 2
    (2.5 * 2.0 ** -9, 0x02),       # tie between codes 2 and 3
    (1.0 + 2.0 ** -4, 0x38),       # tie between 1.0 (0x38) and 1.125 (0x39)
    (1.0 + 3 * 2.0 ** -4, 0x3A),   # tie between 1.125 and 1.25: even 0x3A
    (440.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E),
    (-464.0, 0xFE), (-np.inf, 0xFE), (-0.0, 0x80), (np.nan, 0x7F),
])
def test_e4m3fn_encode_hand_cases(value, code):
    assert formats.e4m3fn_encode(np.array([value]))[0] == code


def test_quantize_uses_float32_division():
    x = np.array([1.0, 3.0, -7.5], np.float32)
    s = np.float32(0.1)
    want = formats.e4m3fn_encode((x / s).astype(np.float64))
    assert np.array_equal(formats.quantize_to_e4m3fn(x, s), want)
    assert formats.e4m3fn_table()[formats.quantize_to_e4m3fn(np.array([448 * 0.1], np.float32), s)[0]] == 448.0


# ------------------------------------------- quantize-on-write, pinned to torch
#
# FP8 KV storage keeps a scale beside the 8-bit codes (youngju.dev,
# "KVキャッシュとPagedAttention — 推論メモリのすべて", section "KV量子化: FP8と
# INT8").  The reference below is built from torch alone: the IEEE float32
# quotient of each element by its own kv head's scale (K and V scales apart),
# clamped to the format's range (torch turns out-of-range values into NaN
# rather than saturating), converted by torch's float8_e4m3fn rounding, and
# scattered by advanced indexing.  It shares no step with the oracle.


def _e4m3_neighbours():
    """Pairs (lo, hi, code_lo, code_hi) of neighbouring positive finite
    E4M3FN values, from torch's decoding of the codes."""
    codes = torch.arange(0x00, 0x7F, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return [(vals[c], vals[c + 1], c, c + 1) for c in range(len(vals) - 1)]


def _division_sensitive_inputs(scales):
    """float32 x per scale s whose E4M3 code differs between the float32
    quotient x/s (the stated reading) and the exact quotient.

    Each x is a float32 neighbour of mid * s, mid halfway between two codes.
    The float32 quotient (torch's IEEE division) and the exact quotient
    (float64 division, exact to well below a float32 ulp here) are compared
    with mid in float64: they pick different codes when they fall on
    opposite sides of it, or when the float32 one lands on it exactly (ties
    go to the even code) and the exact one lies on the odd code's side.
    torch's own float64 -> float8 conversion rounds through float32, so it
    cannot stand in for the exact side.
    """
    picked = {}
    for h, s in enumerate(scales):
        xs = []
        for lo, hi, c_lo, _ in _e4m3_neighbours()[::5]:
            mid = (lo + hi) / 2
            x0 = np.float32(mid * np.float64(s))
            for k in range(-3, 4):
                x = x0
                for _ in range(abs(k)):
                    x = np.nextafter(x, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
                q32 = float((torch.tensor([x]) / torch.tensor([s])).item())
                q64 = float(np.float64(x) / np.float64(s))
                side32 = np.sign(q32 - mid)
                side64 = np.sign(q64 - mid)
                odd_side = -1.0 if c_lo % 2 else 1.0
                if (side32 * side64 < 0) or (side32 == 0 and side64 == odd_side):
                    xs.append(x)
        picked[h] = np.array(xs, np.float32)
    return picked


def _torch_quantized_pool(pool_shape, key32, value32, k_scale, v_scale, slots, block_size):
    kx = torch.from_numpy(key32)
    vx = torch.from_numpy(value32)
    ks = torch.from_numpy(k_scale)[None, :, None]
    vs = torch.from_numpy(v_scale)[None, :, None]
    kc = (kx / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (vx / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    kp = torch.full(pool_shape, 0xA5, dtype=torch.uint8)
    vp = torch.full(pool_shape, 0xA5, dtype=torch.uint8)
    s = torch.from_numpy(slots)
    keep = s >= 0
    blk, row = s[keep] // block_size, s[keep] % block_size
    kp[blk, :, row, :] = kc[keep]
    vp[blk, :, row, :] = vc[keep]
    return kp.numpy(), vp.numpy()


def _quantize_case(seed=23):
    rng = np.random.default_rng(seed)
    num_tokens, hkv, d, bs, nb = 24, 4, 64, 16, 5
    k_scale = np.array([0.1, 0.3, 0.07, 1 / 3], np.float32)
    v_scale = np.array([0.013, 0.9, 0.41, 0.05], np.float32)
    key32 = (rng.standard_normal((num_tokens, hkv, d)) * 4).astype(np.float32)
    value32 = (rng.standard_normal((num_tokens, hkv, d)) * 4).astype(np.float32)
    # plant the division-sensitive values of each head's own scale, and
    # out-of-range values that must saturate
    for arr, scales in ((key32, k_scale), (value32, v_scale)):
        for h, xs in _division_sensitive_inputs(scales).items():
            flat = arr[:, h, :].reshape(-1)
            idx = rng.choice(flat.size, size=len(xs), replace=False)
            flat[idx] = xs * rng.choice([-1, 1], size=len(xs))
            arr[:, h, :] = flat.reshape(num_tokens, d)
        arr[0, :, 0] = 1e6
        arr[1, :, 1] = -np.inf
    slots = rng.permutation(nb * bs)[:num_tokens].astype(np.int64)
    slots[5] = -1  # a skipped token
    return key32, value32, k_scale, v_scale, slots, bs, (nb, hkv, bs, d)


def test_quantize_reshape_and_cache_matches_torch_per_head():
    key32, value32, k_scale, v_scale, slots, bs, shape = _quantize_case()
    kp = np.full(shape, 0xA5, np.uint8)
    vp = np.full(shape, 0xA5, np.uint8)
    oracle.quantize_reshape_and_cache(kp, vp, key32, value32, k_scale, v_scale, slots, bs)
    want_k, want_v = _torch_quantized_pool(shape, key32, value32, k_scale, v_scale, slots, bs)
    assert np.array_equal(kp, want_k)
    assert np.array_equal(vp, want_v)


def test_quantize_pin_discriminates_plausible_oracle_mistakes(monkeypatch):
    """The inputs above separate the stated reading from its near misses.
    Each mistake is planted in the oracle (on the CPU) and must change at
    least one stored code: dividing in float64, taking a neighbouring head's
    scale, or taking the V scale for K."""
    key32, value32, k_scale, v_scale, slots, bs, shape = _quantize_case()
    for h, xs in _division_sensitive_inputs(k_scale).items():
        assert len(xs) >= 3, f"too few division-sensitive values for head {h}"
    want_k, want_v = _torch_quantized_pool(shape, key32, value32, k_scale, v_scale, slots, bs)

    def run(ks, vs):
        kp = np.full(shape, 0xA5, np.uint8)
        vp = np.full(shape, 0xA5, np.uint8)
        oracle.quantize_reshape_and_cache(kp, vp, key32, value32, ks, vs, slots, bs)
        return kp, vp

    kp, vp = run(k_scale, v_scale)
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)
    for ks, vs in ((np.roll(k_scale, 1), v_scale), (v_scale, v_scale), (k_scale, np.roll(v_scale, -1))):
        kp, vp = run(ks, vs)
        assert not (np.array_equal(kp, want_k) and np.array_equal(vp, want_v))
    with monkeypatch.context() as m:
        m.setattr(formats, "quantize_to_e4m3fn",
                  lambda x, s: formats.e4m3fn_encode(np.asarray(x, np.float64) / np.float64(s)))
        kp, vp = run(k_scale, v_scale)
    assert not np.array_equal(kp, want_k)
    assert not np.array_equal(vp, want_v)
