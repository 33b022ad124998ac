"""Mixed decode + prefill batches on the GPU: one call for decode rows and
chunk rows.  Every row must equal the standalone decode / prefill result bit
for bit, and the fp64 oracle (a decode row is a chunk of one token) within
tolerance."""
import numpy as np
import pytest
import torch

import oracle
from oracle.parallel import prefill_rows_par
from gpu_util import TOL, DevBatch, max_abs
from paged_kv_cache_71_amd import workloads as W

pytestmark = pytest.mark.gpu


def run_mixed(pkv, db: DevBatch, out_dtype="f32"):
    b = db.b
    out = db.out(out_dtype)
    maxq = int(np.max(np.diff(b.cu_seqlens_q)))
    pkv.paged_attention_mixed(out, db.q, db.cu_seqlens_q, b.meta["num_decode"], maxq, db.k_cache,
                              db.v_cache, db.block_tables, db.context_lens, b.max_context_len,
                              b.scale)
    torch.cuda.synchronize()
    return out


def run_separate(pkv, db: DevBatch, out_dtype="f32"):
    """The decode rows through paged_attention_decode, the chunks through
    paged_attention_prefill (its own batch of the chunk sequences)."""
    b = db.b
    nd = b.meta["num_decode"]
    out = db.out(out_dtype)
    if nd:
        pkv.paged_attention_decode(out[:nd], db.q[:nd], db.k_cache, db.v_cache,
                                   db.block_tables[:nd].contiguous(), db.context_lens[:nd].contiguous(),
                                   b.max_context_len, b.scale)
    if nd < b.S:
        cu = db.cu_seqlens_q[nd:] - nd
        maxq = int(np.max(np.diff(b.cu_seqlens_q[nd:])))
        pkv.paged_attention_prefill(out[nd:], db.q[nd:].contiguous(), cu.contiguous(), maxq,
                                    db.k_cache, db.v_cache, db.block_tables[nd:].contiguous(),
                                    db.context_lens[nd:].contiguous(), b.max_context_len, b.scale)
    torch.cuda.synchronize()
    return out


def check(pkv, b, rows=None):
    print(f"[mixed] {b.name} S={b.S} decodes={b.meta['num_decode']} Tq={b.q.shape[0]} "
          f"Hq={b.Hq} Hkv={b.Hkv} D={b.D} B={b.B} {b.dtype}", flush=True)
    db = DevBatch(b)
    mixed = run_mixed(pkv, db)
    sep = run_separate(pkv, db)
    assert torch.equal(mixed, sep)
    k, v, tables = b.compact_pool()
    rows = np.arange(b.q.shape[0]) if rows is None else np.asarray(rows)
    ref = prefill_rows_par(b.q, b.cu_seqlens_q, k, v, b.dtype, tables, b.context_lens, b.scale,
                           rows)
    err = max_abs(mixed[torch.as_tensor(rows).cuda()], ref)
    assert err <= TOL[b.dtype], f"max abs err {err}"
    return mixed


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D,B,Hq,Hkv", [(128, 16, 32, 8), (64, 4, 8, 2), (128, 8, 8, 8)])
def test_mixed_matches_separate_calls_and_oracle(gpu_lib, dtype, D, B, Hq, Hkv):
    rng = np.random.default_rng(D + B + Hq)
    dl = rng.integers(1, 700, 9)
    b = W.mixed_batch(D * 3 + B, dl, [300, 0, 1000], [70, 33, 128], Hq, Hkv, D, B, dtype)
    check(gpu_lib, b)


@pytest.mark.parametrize("nd,chunks", [(0, [40, 17]), (6, []), (1, [1]), (5, [200])])
def test_mixed_edge_layouts(gpu_lib, nd, chunks):
    """No decodes, no chunks, a one-token chunk, one decode."""
    dl = list(range(5, 5 + 37 * nd, 37))
    b = W.mixed_batch(nd + 7, dl, [64 * (i + 1) for i in range(len(chunks))], chunks, 16, 4, 128, 16,
                      "bf16")
    check(gpu_lib, b)


def test_mixed_llama3_8b_batch(gpu_lib):
    """The benchmarked mix: 256 Llama-3-8B decodes and one 512-token chunk after
    8192 cached tokens; every output row against the oracle, then again with
    peaked weights (queries scaled by 6)."""
    b = W.llama3_8b_mixed_bf16(0)
    check(gpu_lib, b)
