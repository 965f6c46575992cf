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
