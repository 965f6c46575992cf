"""Quantize-on-write scatter (pa_reshape_and_cache_fp8) against the oracle's
E4M3FN encoder, byte for byte over the whole pool."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_142_amd as pa
from gpu_util import poison_device, poison_host, to_device, to_host_raw
from workloads.generators import round_to_storage

pytestmark = pytest.mark.gpu


def _edge_values():
    t = oracle.e4m3fn_table()
    finite = np.sort(np.unique(t[~np.isnan(t)]))
    mids = (finite[:-1] + finite[1:]) / 2  # exact ties at scale 1
    special = np.array([0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 480.0, 1e4, -1e4, np.inf, -np.inf, np.nan,
                        2.0 ** -10, 2.0 ** -12, -(2.0 ** -10)])
    return np.concatenate([finite, mids, special])


@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("dim,block", [(128, 16), (64, 32)])
def test_quantize_on_write_is_bit_exact(src, dim, block):
    rng = np.random.default_rng(hash((src, dim, block)) % 2 ** 32)
    heads, num_blocks = 4, 24
    edge = _edge_values()
    n_tok = 40
    vals = rng.standard_normal((n_tok, heads, dim)) * rng.choice([0.3, 1.0, 30.0, 300.0], size=(n_tok, heads, 1))
    flat = vals.reshape(-1)
    flat[:len(edge)] = edge  # head 0 of the first tokens: ties, saturation, zeros, NaN
    with np.errstate(over="ignore"):  # fp16 overflows to inf, which must saturate to 448
        raw_k = round_to_storage(vals.astype(np.float32), src)
        raw_v = round_to_storage((-vals).astype(np.float32), src)
    k_scale = np.array([1.0, 0.5, 0.0123, 3.0], np.float32)
    v_scale = np.array([0.25, 1.0, 7.0, 0.001], np.float32)
    slots = rng.permutation(num_blocks * block)[:n_tok].astype(np.int64)
    slots[5] = -1  # skipped token
    shape = (num_blocks, heads, block, dim)
    kc, vc = poison_device(shape, "fp8_e4m3"), poison_device(shape, "fp8_e4m3")
    pa.pa_reshape_and_cache_fp8(to_device(raw_k, src), to_device(raw_v, src), kc, vc,
                                torch.from_numpy(k_scale).cuda(), torch.from_numpy(v_scale).cuda(),
                                torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    hk, hv = poison_host(shape, "fp8_e4m3"), poison_host(shape, "fp8_e4m3")
    k32 = oracle.decode_elements(raw_k, src).astype(np.float32)
    v32 = oracle.decode_elements(raw_v, src).astype(np.float32)
    oracle.quantize_reshape_and_cache(hk, hv, k32, v32, k_scale, v_scale, slots, block)
    gk, gv = to_host_raw(kc, "fp8_e4m3"), to_host_raw(vc, "fp8_e4m3")
    bad = np.flatnonzero(gk.reshape(-1) != hk.reshape(-1))
    assert bad.size == 0, f"{bad.size} K codes differ, e.g. gpu {gk.reshape(-1)[bad[:5]]} oracle {hk.reshape(-1)[bad[:5]]}"
    assert np.array_equal(gv, hv)
