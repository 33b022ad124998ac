"""paged_attention_decode on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle.parallel import decode_par
from gpu_util import TOL, TORCH_DT, DevBatch, max_abs, to_dev, to_host_bits
from paged_kv_cache_71_amd import workloads as W

pytestmark = pytest.mark.gpu


def gpu_decode(pkv, db: DevBatch, out_dtype="f32", workspace=None):
    b = db.b
    out = db.out(out_dtype)
    pkv.paged_attention_decode(out, db.q, db.k_cache, db.v_cache, db.block_tables,
                               db.context_lens, b.max_context_len, b.scale, workspace=workspace)
    torch.cuda.synchronize()
    return out


def oracle_decode(b: W.PagedBatch, seqs=None):
    k, v, tables = b.compact_pool()
    return decode_par(b.q, k, v, b.dtype, tables, b.context_lens, b.scale, seqs=seqs)


def check(pkv, b, seqs=None, out_dtype="f32"):
    print(f"[decode] {b.name} S={b.S} Hq={b.Hq} Hkv={b.Hkv} D={b.D} B={b.B} {b.dtype} "
          f"maxL={b.max_context_len}", flush=True)
    db = DevBatch(b)
    out = gpu_decode(pkv, db, out_dtype)
    ref = oracle_decode(b, seqs)
    got = out if seqs is None else out[torch.as_tensor(np.asarray(seqs)).cuda()]
    err = max_abs(got, ref)
    assert err <= TOL[b.dtype], f"max abs err {err}"
    return out, ref


def test_tiny_f32(gpu_lib):
    check(gpu_lib, W.tiny_f32(0))


def test_opt13b_f16_reduced(gpu_lib):
    check(gpu_lib, W.opt13b_f16(0, S=10, NB=3000))


def test_llama3_8b_bf16_reduced(gpu_lib):
    check(gpu_lib, W.llama3_8b_bf16(0, S=24, NB=30000))


@pytest.mark.parametrize("prompt_len", [2000, 1999])
def test_shared_prefix_reduced(gpu_lib, prompt_len):
    b = W.shared_prefix_bf16(0, prompts=3, n=4, prompt_len=prompt_len, NB=3000)
    check(gpu_lib, b)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_dtype_headdim_block_sweep(gpu_lib, dtype, D, B):
    lengths = [1, B, B + 1, 37, 300, 513, 1100]
    check(gpu_lib, W.decode_batch(B * 7 + D, lengths, 8, 2, D, B, dtype))


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 4), (32, 8), (64, 4), (12, 4), (6, 2), (5, 1)])
def test_group_sizes(gpu_lib, Hq, Hkv):
    check(gpu_lib, W.decode_batch(Hq * Hkv, [3, 64, 700, 1500], Hq, Hkv, 128, 16, "bf16"))


def test_partition_boundaries_and_edges(gpu_lib):
    lengths = [0, 1, 15, 16, 17, 511, 512, 513, 1023, 1024, 1025, 4096, 8192, 0, 1]
    b = W.decode_batch(11, lengths, 32, 8, 128, 16, "bf16")
    out, ref = check(gpu_lib, b)
    assert torch.all(out[0] == 0) and torch.all(out[13] == 0)        # empty context -> zeros


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_long_rows_span_many_waves(gpu_lib, dtype):
    """One 8192-token sequence: each of its 8 rows (KV heads) is cut across
    about a hundred waves, so the merge runs many batches of partial states."""
    check(gpu_lib, W.decode_batch(5, [8192], 32, 8, 128, 16, dtype))


def test_context_of_131072_tokens(gpu_lib):
    """A 131,072-token sequence (8,192 blocks, 512 MiB of bf16 K+V) beside a
    short and a 70,000-token one: rows cut across the whole wave set, block
    offsets past 2^31 bytes in the pool."""
    b = W.decode_batch(7, [131072, 5, 70000], 32, 8, 128, 16, "bf16", NB=70000)
    check(gpu_lib, b)


def test_more_sequences_than_one_launch(gpu_lib):
    """4100 short sequences (some empty): more than one split + merge launch pair."""
    lengths = np.random.default_rng(3).integers(0, 40, 4100)
    out, _ = check(gpu_lib, W.decode_batch(6, lengths, 8, 2, 64, 4, "f32"))
    assert torch.all(out[torch.from_numpy(lengths == 0).cuda()] == 0)


def test_single_token_context_returns_value_exactly(gpu_lib):
    b = W.decode_batch(3, [1, 1, 1], 8, 2, 128, 16, "bf16")
    db = DevBatch(b)
    out = gpu_decode(gpu_lib, db)
    v = W.storage_to_f32(b.v_blocks, "bf16")
    for s in range(3):
        blk = int(np.where(b.block_ids == b.block_tables[s, 0])[0][0])
        for h in range(8):
            assert np.array_equal(out[s, h].cpu().numpy(), v[blk, 0, h // 4])


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_low_precision_output_within_one_ulp(gpu_lib, out_dtype):
    b = W.llama3_8b_bf16(2, S=8, NB=12000)
    db = DevBatch(b)
    out = gpu_decode(gpu_lib, db, out_dtype)
    ref = oracle_decode(b)
    ref_t = torch.from_numpy(ref).to(TORCH_DT[out_dtype])     # RNE of the exact result
    def ordered(bits):   # sign-magnitude bits -> integers ordered like the values
        bits = bits.astype(np.int32)
        return np.where(bits & 0x8000, -(bits & 0x7FFF), bits)
    diff = ordered(to_host_bits(out)) - ordered(to_host_bits(ref_t.cuda()))
    # within one ulp of the correctly rounded result, except near zero where the
    # fp32 accumulation error (<= 2e-5 here) is larger than an ulp
    near_zero = np.abs(out.float().cpu().numpy() - ref) <= 2e-5
    assert np.all((np.abs(diff) <= 1) | near_zero)
    assert np.mean(np.abs(diff) <= 1) > 0.999


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("dtype,D,B,Hq,Hkv", [("bf16", 128, 16, 32, 8), ("bf16", 128, 16, 64, 4),
                                               ("f16", 64, 4, 8, 2), ("f32", 64, 8, 4, 4)])
def test_low_precision_output_is_the_rounded_fp32_output(gpu_lib, out_dtype, dtype, D, B, Hq, Hkv):
    """Rows finished inside one wave, rows merged across waves and empty
    contexts: a 16-bit output holds exactly the fp32 output rounded to nearest
    even (the same fp32 value is computed on either path), on the matrix-core
    and the vector path."""
    lengths = [0, 1, 17, 300, 4100, 0, 2000, 65]
    b = W.decode_batch(D + B + Hq, lengths, Hq, Hkv, D, B, dtype)
    out32, _ = check(gpu_lib, b)
    out16 = gpu_decode(gpu_lib, DevBatch(b), out_dtype)
    want = out32.to(TORCH_DT[out_dtype])
    assert torch.equal(out16.view(torch.int16), want.view(torch.int16))
    assert torch.all(out16[0] == 0) and torch.all(out16[5] == 0)


def _relayout(b: W.PagedBatch, seed: int, alias_copies: bool = False) -> W.PagedBatch:
    """Same logical contents, different physical blocks (a fresh permutation of
    the pool); optionally give every aliased block a private copy."""
    rng = np.random.default_rng(seed)
    k, v, tables = b.compact_pool(extra_poison_blocks=0)
    n = k.shape[0]
    if alias_copies:
        nb = -(-b.context_lens // b.B)
        holders = [(s, j) for s in range(b.S) for j in range(nb[s])]
        k = np.concatenate([k[tables[s, j]][None] for s, j in holders])
        v = np.concatenate([v[tables[s, j]][None] for s, j in holders])
        tables = np.full_like(tables, -1)
        for i, (s, j) in enumerate(holders):
            tables[s, j] = i
        n = k.shape[0]
    NB = n + 50
    perm = rng.permutation(NB)[:n]
    new_tables = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    import dataclasses
    last = np.maximum(b.context_lens.astype(np.int64) - 1, 0)
    keep = b.context_lens > 0
    slots = (new_tables[np.arange(b.S), last // b.B].astype(np.int64) * b.B + last % b.B)[keep]
    return dataclasses.replace(b, NB=NB, block_tables=new_tables, block_ids=perm.astype(np.int64),
                               k_blocks=k, v_blocks=v, new_slots=slots)


def test_bit_exact_under_physical_permutation(gpu_lib):
    b = W.llama3_8b_bf16(4, S=16, NB=20000)
    outs = [gpu_decode(gpu_lib, DevBatch(x)) for x in (b, _relayout(b, 1), _relayout(b, 2))]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_aliased_prefix_equals_private_copies_bit_exact(gpu_lib):
    b = W.shared_prefix_bf16(1, prompts=2, n=4, prompt_len=1999, NB=3000)
    shared = gpu_decode(gpu_lib, DevBatch(b))
    private = gpu_decode(gpu_lib, DevBatch(_relayout(b, 3, alias_copies=True)))
    assert torch.equal(shared, private)


def test_workspace_too_small_is_rejected(gpu_lib):
    b = W.decode_batch(1, [2000, 30], 8, 2, 128, 16, "bf16")
    db = DevBatch(b)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.PkvError, match="WORKSPACE"):
        gpu_decode(gpu_lib, db, workspace=ws)


# ---------------------------------------------------------------- full-size workloads
def test_llama3_8b_full_size(gpu_lib):
    """The benchmarked workload (256 sequences, 12 GB pool): every output
    element of every sequence against the oracle."""
    check(gpu_lib, W.llama3_8b_bf16(0))


def test_llama3_8b_tp8_shard_full_size(gpu_lib):
    """One GPU's share of the benchmarked batch at tensor parallelism 8 (4 query
    heads over 1 KV head of every block, same lengths and block placement):
    every output element against the oracle."""
    check(gpu_lib, W.llama3_8b_tp8_shard(0))


def test_opt13b_full_size(gpu_lib):
    check(gpu_lib, W.opt13b_f16(0))


def test_shared_prefix_full_size(gpu_lib):
    """The shared-prefix batch (64 prompts x 4 samples aliasing 125 blocks):
    every output element against the oracle."""
    check(gpu_lib, W.shared_prefix_bf16(0))


def test_concurrent_host_threads(gpu_lib):
    """Four host threads call decode at once, each on its own stream with its own
    workspace (the library's caches are shared): every result equals the same
    call made alone, bit for bit."""
    import threading
    batches = [W.decode_batch(300 + i, [5, 700, 1500, 33, 2048], 32, 8, 128, 16, "bf16") for i in range(4)]
    devs = [DevBatch(b) for b in batches]
    alone = [gpu_decode(gpu_lib, d).clone() for d in devs]
    outs = [None] * 4
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                b, d = batches[i], devs[i]
                n = gpu_lib.decode_workspace_size(b.S, b.Hq, b.Hkv, b.D, b.B, b.max_context_len)
                ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
                out = d.out("f32")
                for _ in range(5):
                    gpu_lib.paged_attention_decode(out, d.q, d.k_cache, d.v_cache, d.block_tables,
                                                   d.context_lens, b.max_context_len, b.scale,
                                                   workspace=ws)
                s.synchronize()
                outs[i] = out
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(4):
        assert torch.equal(outs[i], alone[i])
