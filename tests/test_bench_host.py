"""Host logic of bench.py, on the CPU: the identity block-table relabelling
keeps every sequence's contents and the oracle's result, and the oracle
baselines (one thread, all cores) run and report what they used."""

import numpy as np

import bench
import oracle
import workloads


def _oracle_result(wl):
    kc = np.zeros(wl.pool_shape(), wl.keys.dtype)
    vc = np.zeros(wl.pool_shape(), wl.keys.dtype)
    oracle.reshape_and_cache(kc, vc, wl.keys, wl.values, wl.slots, wl.block_size)
    oracle.copy_blocks(kc, vc, wl.copy_pairs)
    return kc, vc, oracle.paged_decode(wl.q, wl.q_dtype, kc, vc, wl.kv_dtype, wl.block_tables, wl.seq_lens,
                                       wl.block_size, float(wl.scale), wl.k_scale, wl.v_scale)


def test_identity_tables_are_consecutive_and_keep_contents():
    wl = workloads.gqa(5, num_seqs=9, max_len=700)
    ident = bench.identity_tables(wl)
    nxt = 0
    for i, t in enumerate(ident.seq_lens):
        n = -(-int(t) // wl.block_size)
        assert np.array_equal(ident.block_tables[i, :n], np.arange(nxt, nxt + n))
        assert (ident.block_tables[i, n:] == -1).all()
        nxt += n
    kc0, vc0, out0 = _oracle_result(wl)
    kc1, vc1, out1 = _oracle_result(ident)
    assert np.array_equal(out0, out1)  # the same rows in the same order: bitwise
    for i, t in enumerate(wl.seq_lens):
        for pool0, pool1 in ((kc0, kc1), (vc0, vc1)):
            a = oracle.gather_sequence(pool0, wl.block_tables[i], t, wl.block_size)
            b = oracle.gather_sequence(pool1, ident.block_tables[i], t, wl.block_size)
            assert np.array_equal(a, b)
    # copy pairs move to the relabelled blocks: the copied tiles are the same
    for (s0, d0), (s1, d1) in zip(wl.copy_pairs, ident.copy_pairs):
        assert np.array_equal(kc0[d0], kc1[d1])


def test_cpu_baselines_report_their_cores():
    wl = workloads.tiny(0)
    res = bench.cpu_baseline(wl, 0.3)
    assert res["kind"] == "oracle" and res["value"] > 0 and res["unit"] == "GB/s"
    workers, avail = bench._cpu_share()
    assert res["cores"] == workers <= 16 and res["cores_available"] == avail
    assert res["blas_threads_per_worker"] == 1
    assert res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0
