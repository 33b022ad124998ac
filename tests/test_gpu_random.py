"""Seeded random sweep against the fp64 oracle: every case draws its own
shape (head dim, KV heads, group size, block size), dtype, length mix (empty
contexts, contexts shorter than a block, long ones), chunk layout and softmax
scale, for decode, prefill, mixed batches, cascade (shared-prefix) decode and
the FP8 variants.  Each case
prints its parameters before it runs, so a failure names the draw.  The
fixed-shape tests cover the named configurations; this sweep covers the
combinations between them."""
import numpy as np
import pytest

from paged_kv_cache_71_amd import workloads as W
from test_gpu_cascade import check as check_cascade
from test_gpu_decode import check as check_decode
from test_gpu_fp8 import check as check_decode_fp8
from test_gpu_fp8 import check_prefill as check_prefill_fp8
from test_gpu_mixed import check as check_mixed
from test_gpu_prefill import check as check_prefill

pytestmark = pytest.mark.gpu

# oracle work per prefill-like case (multiply-adds of q.k and p.v), so a case
# finishes within about two seconds on the CPU
PREFILL_BUDGET = 1.5e9


def _heads(rng, d_choices=(64, 128)):
    D = int(rng.choice(d_choices))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    while Hkv * G > 64:
        Hkv //= 2
    return Hkv * G, max(Hkv, 1), D


def _lengths(rng, S, hi):
    kind = rng.random(S)
    short = rng.integers(1, 40, S)
    long = rng.integers(40, hi + 1, S)
    return np.where(kind < 0.1, 0, np.where(kind < 0.45, short, long)).astype(np.int32)


def _scale(rng, D):
    return float(rng.choice([1.0, 1.0, -0.7, 2.5, 0.0])) / np.sqrt(D)


def _prefill_layout(rng, S, Hq, D, max_chunk, max_prior):
    """Chunk and prior lengths within the oracle budget (chunks >= 1)."""
    while True:
        chunks = rng.integers(1, max_chunk + 1, S)
        prior = np.where(rng.random(S) < 0.25, 0, rng.integers(0, max_prior + 1, S))
        work = float(np.sum(chunks * (prior + chunks))) * Hq * D * 2
        if work <= PREFILL_BUDGET:
            return prior.astype(np.int32), chunks.astype(np.int32)
        max_chunk = max(1, max_chunk // 2)
        max_prior = max(1, max_prior // 2)


@pytest.mark.parametrize("case", range(80))
def test_random_decode(gpu_lib, case):
    rng = np.random.default_rng(1000 + case)
    Hq, Hkv, D = _heads(rng)
    B = int(rng.choice([1, 2, 4, 8, 16, 32]))
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    S = int(rng.integers(1, 13))
    lengths = _lengths(rng, S, 3000)
    print(f"[random decode {case}] Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} lengths={lengths.tolist()}",
          flush=True)
    b = W.decode_batch(2000 + case, lengths, Hq, Hkv, D, B, dtype)
    b.scale = _scale(rng, D)
    check_decode(gpu_lib, b)


@pytest.mark.parametrize("case", range(60))
def test_random_prefill(gpu_lib, case):
    rng = np.random.default_rng(3000 + case)
    Hq, Hkv, D = _heads(rng)
    B = int(rng.choice([1, 2, 4, 8, 16, 16, 32, 32]))
    dtype = str(rng.choice(["f32", "f16", "bf16", "bf16"]))
    S = int(rng.integers(1, 7))
    prior, chunks = _prefill_layout(rng, S, Hq, D, 300, 6000)
    print(f"[random prefill {case}] Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} prior={prior.tolist()} "
          f"chunks={chunks.tolist()}", flush=True)
    b = W.varlen_prefill(4000 + case, prior, chunks, Hq, Hkv, D, B, dtype)
    b.scale = _scale(rng, D)
    check_prefill(gpu_lib, b)


@pytest.mark.parametrize("case", range(24))
def test_random_mixed(gpu_lib, case):
    rng = np.random.default_rng(5000 + case)
    Hq, Hkv, D = _heads(rng)
    B = int(rng.choice([4, 8, 16, 16, 32]))
    dtype = str(rng.choice(["f32", "f16", "bf16", "bf16"]))
    nd = int(rng.integers(0, 10))
    dl = rng.integers(1, 1500, nd)
    nc = int(rng.integers(0 if nd else 1, 4))
    prior, chunks = _prefill_layout(rng, nc, Hq, D, 128, 2000)
    print(f"[random mixed {case}] Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} decodes={dl.tolist()} "
          f"prior={prior.tolist()} chunks={chunks.tolist()}", flush=True)
    b = W.mixed_batch(6000 + case, dl, prior, chunks, Hq, Hkv, D, B, dtype)
    b.scale = _scale(rng, D)
    check_mixed(gpu_lib, b)


@pytest.mark.parametrize("case", range(24))
def test_random_decode_fp8(gpu_lib, case):
    rng = np.random.default_rng(7000 + case)
    Hq, Hkv, D = _heads(rng)
    B = int(rng.choice([1, 4, 8, 16, 32]))
    q_dtype = str(rng.choice(["f16", "bf16"]))
    S = int(rng.integers(1, 13))
    lengths = _lengths(rng, S, 3000)
    print(f"[random fp8 decode {case}] Hq={Hq} Hkv={Hkv} D={D} B={B} q={q_dtype} "
          f"lengths={lengths.tolist()}", flush=True)
    b = W.decode_batch(8000 + case, lengths, Hq, Hkv, D, B, q_dtype)
    b.scale = _scale(rng, D)
    check_decode_fp8(gpu_lib, b, seed=case)


@pytest.mark.parametrize("case", range(24))
def test_random_prefill_fp8(gpu_lib, case):
    rng = np.random.default_rng(9000 + case)
    Hq, Hkv, D = _heads(rng)
    B = int(rng.choice([16, 32]))
    q_dtype = str(rng.choice(["f16", "bf16"]))
    S = int(rng.integers(1, 6))
    prior, chunks = _prefill_layout(rng, S, Hq, D, 300, 6000)
    print(f"[random fp8 prefill {case}] Hq={Hq} Hkv={Hkv} D={D} B={B} q={q_dtype} "
          f"prior={prior.tolist()} chunks={chunks.tolist()}", flush=True)
    b = W.varlen_prefill(10000 + case, prior, chunks, Hq, Hkv, D, B, q_dtype)
    b.scale = _scale(rng, D)
    check_prefill_fp8(gpu_lib, b, seed=case)


@pytest.mark.parametrize("case", range(24))
def test_random_cascade(gpu_lib, case):
    rng = np.random.default_rng(11000 + case)
    Hq, Hkv, D = _heads(rng)
    B = int(rng.choice([1, 2, 4, 8, 16, 32]))
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    sizes = [int(x) for x in rng.integers(1, 6, int(rng.integers(1, 5)))]
    pblocks = [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(0, 1500 // B + 1, len(sizes))]
    suffix = np.where(rng.random(sum(sizes)) < 0.2, 0, rng.integers(0, 400, sum(sizes)))
    print(f"[random cascade {case}] Hq={Hq} Hkv={Hkv} D={D} B={B} {dtype} groups={sizes} "
          f"prefix_blocks={pblocks} suffixes={suffix.tolist()}", flush=True)
    b = W.grouped_batch(12000 + case, sizes, pblocks, suffix, Hq, Hkv, D, B, dtype)
    b.scale = _scale(rng, D)
    check_cascade(gpu_lib, b)
