"""The threaded driver of the oracle (oracle/parallel.py) returns exactly what
one sequential call returns: it only cuts the batch into parts."""
import numpy as np

import oracle
from oracle.parallel import (decode_fp8_par, decode_par, host_threads, prefill_fp8_rows_par,
                             prefill_rows_par)
from paged_kv_cache_71_amd import workloads as W


def test_decode_par_is_bit_identical():
    b = W.decode_batch(3, [0, 1, 17, 300, 45, 999, 16, 2], 8, 2, 64, 4, "bf16")
    k, v, tables = b.compact_pool()
    want = oracle.decode(b.q, k, v, b.dtype, tables, b.context_lens, b.scale)
    for threads in (1, 3, 8):
        assert np.array_equal(decode_par(b.q, k, v, b.dtype, tables, b.context_lens, b.scale,
                                         threads=threads), want)
    seqs = [5, 0, 3]
    assert np.array_equal(decode_par(b.q, k, v, b.dtype, tables, b.context_lens, b.scale,
                                     seqs=seqs, threads=2), want[seqs])


def test_decode_fp8_par_is_bit_identical():
    b = W.decode_batch(4, [1, 40, 300, 7, 0], 8, 2, 64, 16, "f16")
    f = W.fp8_pools(b, 3)
    _, _, tables = b.compact_pool(extra_poison_blocks=0)
    want = oracle.decode_fp8(b.q, b.dtype, f.k_blocks, f.v_blocks, f.k_scale, f.v_scale, tables,
                             b.context_lens, b.scale)
    got = decode_fp8_par(b.q, b.dtype, f.k_blocks, f.v_blocks, f.k_scale, f.v_scale, tables,
                         b.context_lens, b.scale, threads=4)
    assert np.array_equal(got, want)


def test_prefill_rows_par_is_bit_identical():
    b = W.varlen_prefill(5, [0, 30, 7], [9, 40, 1], 8, 2, 64, 8, "bf16")
    k, v, tables = b.compact_pool()
    want = oracle.prefill(b.q, b.cu_seqlens_q, k, v, b.dtype, tables, b.context_lens, b.scale)
    rows = W.strided_chunk_rows(b.cu_seqlens_q, 3)
    assert rows[0] == 0 and 8 in rows and 48 in rows and 49 in rows   # chunk ends included
    got = prefill_rows_par(b.q, b.cu_seqlens_q, k, v, b.dtype, tables, b.context_lens, b.scale,
                           rows[::-1], threads=3)
    assert np.array_equal(got, want[rows[::-1]])
    f = W.fp8_pools(b, 1)
    _, _, t0 = b.compact_pool(extra_poison_blocks=0)
    want8 = oracle.prefill_fp8(b.q, b.dtype, b.cu_seqlens_q, f.k_blocks, f.v_blocks, f.k_scale,
                               f.v_scale, t0, b.context_lens, b.scale)
    got8 = prefill_fp8_rows_par(b.q, b.dtype, b.cu_seqlens_q, f.k_blocks, f.v_blocks, f.k_scale,
                                f.v_scale, t0, b.context_lens, b.scale, rows, threads=5)
    assert np.array_equal(got8, want8[rows])


def test_host_threads_is_the_affinity_mask():
    import os
    assert host_threads(10**6) == len(os.sched_getaffinity(0))
    assert host_threads(1) == 1
