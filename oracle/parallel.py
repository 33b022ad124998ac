"""Run the fp64 oracle over disjoint parts of a batch on several host threads
-- TEST INFRASTRUCTURE ONLY (tests, ``__graft_entry__.smoke()`` and the CPU
baseline of ``bench.py``).

Nothing here computes attention: every part is one call of the functions in
``oracle/__init__.py`` (plain fp64 C) on a subset of the sequences or query
rows, and the parts are stitched back together.  Each output element comes
from exactly the same C code path and inputs as in a single call, so the
result is bit-for-bit that of the sequential oracle.  ctypes releases the GIL
for the duration of each C call and the C oracle keeps no global state, so
the threads run in parallel.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import _load, decode, decode_fp8, prefill, prefill_fp8


def host_threads(cap: int = 16) -> int:
    """Cores in this process's affinity mask (at most ``cap``)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def _balanced_parts(weights: np.ndarray, n_parts: int) -> list[np.ndarray]:
    """Split indices 0..len(weights)-1 into about n_parts lists of similar total
    weight (longest first, each to the lightest part so far)."""
    order = np.argsort(-np.asarray(weights, np.int64), kind="stable")
    loads = np.zeros(n_parts, np.int64)
    parts: list[list[int]] = [[] for _ in range(n_parts)]
    for i in order:
        j = int(np.argmin(loads))
        parts[j].append(int(i))
        loads[j] += int(weights[i]) + 1
    return [np.array(sorted(p), np.int64) for p in parts if p]


def _run(tasks, threads):
    _load()  # build / load the C library once, before the threads start
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda f: f(), tasks))


def decode_par(q, k_cache, v_cache, dtype: str, block_tables, context_lens, scale: float,
               seqs=None, threads: int | None = None) -> np.ndarray:
    """oracle.decode over the sequences ``seqs`` (default: all), in parallel.
    Returns [len(seqs), Hq, D] fp64."""
    threads = threads or host_threads()
    sel = np.arange(q.shape[0]) if seqs is None else np.asarray(seqs, np.int64)
    lens = np.asarray(context_lens)[sel]
    parts = _balanced_parts(lens, 4 * threads)
    out = np.empty((sel.size,) + tuple(q.shape[1:]), np.float64)

    def task(p):
        s = sel[p]
        return lambda: (p, decode(q[s], k_cache, v_cache, dtype, block_tables[s],
                                  np.asarray(context_lens)[s], scale))
    for p, r in _run([task(p) for p in parts], threads):
        out[p] = r
    return out


def decode_fp8_par(q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, block_tables,
                   context_lens, scale: float, seqs=None, threads: int | None = None) -> np.ndarray:
    """oracle.decode_fp8 over the sequences ``seqs`` (default: all), in parallel."""
    threads = threads or host_threads()
    sel = np.arange(q.shape[0]) if seqs is None else np.asarray(seqs, np.int64)
    lens = np.asarray(context_lens)[sel]
    parts = _balanced_parts(lens, 4 * threads)
    out = np.empty((sel.size,) + tuple(q.shape[1:]), np.float64)

    def task(p):
        s = sel[p]
        return lambda: (p, decode_fp8(q[s], q_dtype, k_cache, v_cache, k_scale, v_scale,
                                      block_tables[s], np.asarray(context_lens)[s], scale))
    for p, r in _run([task(p) for p in parts], threads):
        out[p] = r
    return out


def _prefill_tasks(cu_seqlens_q, rows, threads):
    """(sequence, rows of it) work items: each sequence's wanted rows cut into
    pieces so that every thread gets several."""
    cu = np.asarray(cu_seqlens_q, np.int64)
    rows = np.asarray(rows, np.int64)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    per_seq = [rows[seq_of == s] for s in range(cu.size - 1)]
    n_items = max(1, sum(r.size > 0 for r in per_seq))
    pieces = max(1, (4 * threads + n_items - 1) // n_items)
    items = []
    for r in per_seq:
        if r.size:
            items += [c for c in np.array_split(r, min(pieces, r.size)) if c.size]
    return items


def prefill_rows_par(q, cu_seqlens_q, k_cache, v_cache, dtype: str, block_tables, context_lens,
                     scale: float, rows, threads: int | None = None) -> np.ndarray:
    """oracle.prefill for the query rows ``rows`` only, in parallel.
    Returns [len(rows), Hq, D] fp64 in the order of ``rows``."""
    threads = threads or host_threads()
    rows = np.asarray(rows, np.int64)
    pos = {int(r): i for i, r in enumerate(rows)}
    out = np.empty((rows.size,) + tuple(q.shape[1:]), np.float64)

    def task(r):
        return lambda: (r, prefill(q, cu_seqlens_q, k_cache, v_cache, dtype, block_tables,
                                   context_lens, scale, rows=r)[r])
    for r, res in _run([task(r) for r in _prefill_tasks(cu_seqlens_q, rows, threads)], threads):
        out[[pos[int(x)] for x in r]] = res
    return out


def prefill_fp8_rows_par(q, q_dtype: str, cu_seqlens_q, k_cache, v_cache, k_scale, v_scale,
                         block_tables, context_lens, scale: float, rows,
                         threads: int | None = None) -> np.ndarray:
    """oracle.prefill_fp8 for the query rows ``rows`` only, in parallel."""
    threads = threads or host_threads()
    rows = np.asarray(rows, np.int64)
    pos = {int(r): i for i, r in enumerate(rows)}
    out = np.empty((rows.size,) + tuple(q.shape[1:]), np.float64)

    def task(r):
        return lambda: (r, prefill_fp8(q, q_dtype, cu_seqlens_q, k_cache, v_cache, k_scale,
                                       v_scale, block_tables, context_lens, scale, rows=r)[r])
    for r, res in _run([task(r) for r in _prefill_tasks(cu_seqlens_q, rows, threads)], threads):
        out[[pos[int(x)] for x in r]] = res
    return out
