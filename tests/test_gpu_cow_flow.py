"""Copy-on-write decode step driven by the host block manager, on the GPU:
fork -> append (CoW pairs) -> copy_blocks -> reshape_and_cache -> decode,
compared with the oracle doing the same steps on the host."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_71_amd as pkv
from gpu_util import TOL, max_abs, to_dev, to_host_bits
from paged_kv_cache_71_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("prompt_len,expect_pairs", [(1999, 3), (2000, 0), (37, 3)])
def test_cow_step(gpu_lib, prompt_len, expect_pairs):
    print(f"[cow] prompt_len={prompt_len}", flush=True)
    rng = np.random.default_rng(prompt_len)
    B, Hq, Hkv, D, n, prompts = 16, 32, 8, 128, 4, 3
    NB = 3 * (prompt_len // B + 8) * n
    bm = pkv.BlockManager(NB, B, free_order=rng.permutation(NB))
    seqs = []
    for _ in range(prompts):
        parent = bm.add_seq(prompt_len)
        seqs += [parent] + [bm.fork(parent) for _ in range(n - 1)]
    # prompt K/V for every allocated block (host copy = oracle's pool)
    k_host = np.full((NB, B, Hkv, D), W.NAN_BITS["bf16"], np.uint16)
    v_host = k_host.copy()
    for p in range(prompts):
        for blk in bm.table(seqs[p * n]):
            k_host[blk] = W.to_storage(rng.standard_normal((B, Hkv, D), dtype=np.float32), "bf16")
            v_host[blk] = W.to_storage(rng.standard_normal((B, Hkv, D), dtype=np.float32), "bf16")
    # each sample appends its first generated token
    slots, pairs = [], []
    for s in seqs:
        slot, cow = bm.append_token(s)
        slots.append(slot)
        if cow:
            pairs.append(cow)
    bm.check()
    assert len(pairs) == expect_pairs * prompts
    pairs = np.array(pairs, np.int64).reshape(-1, 2)
    slots = np.array(slots, np.int64)
    new_k = W.to_storage(rng.standard_normal((len(seqs), Hkv, D), dtype=np.float32), "bf16")
    new_v = W.to_storage(rng.standard_normal((len(seqs), Hkv, D), dtype=np.float32), "bf16")
    q = W.to_storage(rng.standard_normal((len(seqs), Hq, D), dtype=np.float32), "bf16")
    L = prompt_len + 1
    tables = np.full((len(seqs), -(-L // B)), -1, np.int32)
    for i, s in enumerate(seqs):
        tables[i] = bm.table(s)
    lens = np.full(len(seqs), L, np.int32)

    kd, vd = to_dev(k_host, "bf16"), to_dev(v_host, "bf16")
    gpu_lib.copy_blocks([kd], [vd], torch.from_numpy(pairs).cuda())
    gpu_lib.reshape_and_cache(to_dev(new_k, "bf16"), to_dev(new_v, "bf16"), kd, vd,
                              torch.from_numpy(slots).cuda())
    out = torch.full((len(seqs), Hq, D), float("nan"), device="cuda")
    gpu_lib.paged_attention_decode(out, to_dev(q, "bf16"), kd, vd, torch.from_numpy(tables).cuda(),
                                   torch.from_numpy(lens).cuda(), L, 1 / np.sqrt(D))
    torch.cuda.synchronize()

    oracle.copy_blocks([k_host], [v_host], pairs, "bf16")
    oracle.reshape_and_cache(new_k, new_v, k_host, v_host, slots, "bf16")
    assert to_host_bits(kd).tobytes() == k_host.tobytes()
    assert to_host_bits(vd).tobytes() == v_host.tobytes()
    ref = oracle.decode(q, k_host, v_host, "bf16", tables, lens, 1 / np.sqrt(D))
    assert max_abs(out, ref) <= TOL["bf16"]
    # the samples of a prompt share the prompt but not their new token
    assert not torch.equal(out[0], out[1])
