"""The hot-path step captured in a HIP graph and replayed gives exactly the
eager result on every replay (no memset nodes are recorded: the library
launches kernels only)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_142_amd as pa
import workloads
from gpu_util import TOL, DeviceCase, assert_close, oracle_out, oracle_pools, out_as_f64

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    wl = workloads.gqa(8, num_seqs=12, max_len=2500)
    case = DeviceCase(wl)
    case.run_step()
    torch.cuda.synchronize()
    eager = case.out.clone()
    pools = (case.k_cache.clone(), case.v_cache.clone())
    args = case.decode_args()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            calls = [pa.prepared("pa_reshape_and_cache", case.step_keys, case.step_values, case.k_cache,
                                 case.v_cache, case.step_slots),
                     pa.prepared("pa_copy_blocks", case.k_cache, case.v_cache, case.pairs),
                     pa.prepared("pa_decode_partition", **args),
                     pa.prepared("pa_decode_reduce", **args)]
            for call in calls:
                call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        case.out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(case.out.view(torch.int32), eager.view(torch.int32)), f"replay {rep} differs"
        assert torch.equal(case.k_cache.view(torch.int16), pools[0].view(torch.int16))
        assert torch.equal(case.v_cache.view(torch.int16), pools[1].view(torch.int16))
    kc, vc = oracle_pools(wl)
    assert_close(out_as_f64(case.out), oracle_out(wl, kc, vc), TOL["bf16"], "graph replay")


def _capture(make_calls):
    """Capture the calls make_calls() marshals (on a side stream) in a graph."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for call in make_calls():
                call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def _replays_match(g, out, eager, what, reps=4):
    for rep in range(reps):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"{what}: replay {rep} differs"


@pytest.mark.parametrize("kind", ["fp8_quantize", "plan_kernel", "append"])
def test_graph_other_decode_paths(kind):
    """The FP8 step (quantize-on-write scatter, matrix-core decode), a batch
    of more than 64 sequences (work order from the plan kernel), and the
    step as copies plus decode with append."""
    if kind == "fp8_quantize":
        wl = workloads.long_fp8(8, num_seqs=3, seq_len=1500, partition_size=512)
    else:
        wl = workloads.gqa(9, num_seqs=80, max_len=700, partition_size=256)
    print(f"[case] graph {kind}: {wl.name} N={wl.num_seqs}", flush=True)
    case = DeviceCase(wl)
    case.run_step()
    torch.cuda.synchronize()
    eager = case.out.clone()
    args = case.decode_args()

    def calls():
        if kind == "append":
            return [pa.prepared("pa_copy_blocks", case.k_cache, case.v_cache, case.pairs),
                    pa.prepared("pa_decode_append", **args, key=case.step_keys, value=case.step_values)]
        if case.quantize_step:
            first = pa.prepared("pa_reshape_and_cache_fp8", case.step_keys, case.step_values, case.k_cache,
                                case.v_cache, case.k_scale, case.v_scale, case.step_slots)
        else:
            first = pa.prepared("pa_reshape_and_cache", case.step_keys, case.step_values, case.k_cache,
                                case.v_cache, case.step_slots)
        return [first, pa.prepared("pa_copy_blocks", case.k_cache, case.v_cache, case.pairs,
                                   kv_dtype=wl.kv_dtype if wl.kv_dtype == "fp8_e4m3" else None),
                pa.prepared("pa_decode", **args)]

    g = _capture(calls)
    _replays_match(g, case.out, eager, kind)
    kc, vc = oracle_pools(wl)
    assert_close(out_as_f64(case.out), oracle_out(wl, kc, vc), TOL[wl.kv_dtype], f"graph replay {kind}")


def test_graph_shared_prefix_and_prefill():
    from test_gpu_prefill import PrefillCase
    from test_gpu_shared_prefix import _grouped_case
    from gpu_util import poison_device, to_device

    P = 256
    groups = [(2 * P, [2 * P + 5, 2 * P + 90, 2 * P]), (P + 16, [P + 16, P + 100])]
    lens, tables, starts, prefixes, hk, hv, q = _grouped_case(12, num_heads=32, num_kv_heads=8, head_dim=128,
                                                              block_size=16, fmt="bf16", groups=groups)
    print("[case] graph shared-prefix decode", flush=True)
    msl = int(lens.max())
    dev = dict(out=poison_device(q.shape, "f32"), q=to_device(q, "bf16"), k_cache=to_device(hk, "bf16"),
               v_cache=to_device(hv, "bf16"), block_tables=torch.from_numpy(tables).cuda(),
               seq_lens=torch.from_numpy(lens).cuda(), max_seq_len=msl, scale=0.088, partition_size=P,
               workspace=torch.empty(pa.pa_decode_workspace_size(q.shape[0], q.shape[1], q.shape[2], msl, P),
                                     dtype=torch.uint8, device="cuda"))
    grp = dict(group_start=torch.from_numpy(starts).cuda(), group_prefix=torch.from_numpy(prefixes).cuda(),
               max_group_size=3, max_prefix_len=int(prefixes.max()))
    pa.pa_decode_shared_prefix(**dev, **grp)
    torch.cuda.synchronize()
    eager = dev["out"].clone()
    g = _capture(lambda: [pa.prepared("pa_decode_shared_prefix", **dev, **grp)])
    _replays_match(g, dev["out"], eager, "shared-prefix decode")

    print("[case] graph prefill", flush=True)
    pwl = workloads.prefill(12, num_seqs=4, max_len=400, chunk=60, kv_dtype="bf16")
    case = PrefillCase(pwl)
    case.run()
    eager = case.out.clone()
    c = pwl.cache
    pargs = dict(out=case.out, q=case.q, query_start=case.query_start, k_cache=case.k_cache, v_cache=case.v_cache,
                 block_tables=case.tables, seq_lens=case.lens, max_seq_len=c.max_seq_len,
                 max_query_len=int(pwl.query_lens.max()), scale=float(c.scale))
    g = _capture(lambda: [pa.prepared("pa_prefill", **pargs)])
    _replays_match(g, case.out, eager, "prefill")
