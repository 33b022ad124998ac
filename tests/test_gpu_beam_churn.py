"""Beam-search churn on the device, driven by the host block manager: at every
step some beams are killed (their blocks released), survivors are forked to
refill the beam (tables shared, refcounts raised), and every live beam
appends one token -- a write into a shared, partly filled last block first
copies it (copy_blocks), then reshape_and_cache writes the token.  After every
step the device pools equal, byte for byte, the host pools that the oracle's
copy and scatter produced from the same pairs and slots, and the beams'
decode matches the oracle.  The one-call variant runs each step's scatter
and decode as one pkv_decode_step call (after the copies).

CS349D lecture 3 sec. 4.2 (beam search: candidates fork from a parent, killed
candidates release their blocks, shared blocks are copied on first write) and
CMU 11-868 lecture 24 sec. 4.2 (fork and kill, refcounts) with its exercise
answer 5."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_71_amd as pkv
from gpu_util import TOL, max_abs, to_dev, to_host_bits
from paged_kv_cache_71_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("one_call", [False, True])
@pytest.mark.parametrize("B,prompt_len,width,steps", [(16, 37, 4, 30), (4, 9, 6, 30),
                                                      (16, 48, 3, 40)])
def test_beam_search_churn(gpu_lib, B, prompt_len, width, steps, one_call):
    print(f"[beam] B={B} prompt={prompt_len} width={width} steps={steps} one_call={one_call}",
          flush=True)
    rng = np.random.default_rng(B * 1000 + prompt_len)
    Hq, Hkv, D, dt = 32, 8, 128, "bf16"
    NB = width * (-(-(prompt_len + steps) // B) + 2) * 3
    bm = pkv.BlockManager(NB, B, free_order=rng.permutation(NB).astype(np.int32))
    k_host = np.full((NB, B, Hkv, D), W.NAN_BITS[dt], np.uint16)
    v_host = k_host.copy()
    kd, vd = to_dev(k_host, dt), to_dev(v_host, dt)

    def write(slots, pairs, beams=None):
        """One step's copies and scatter, on the device and on the host; with
        beams (one-call variant) the scatter rides in the step's decode."""
        slots = np.asarray(slots, np.int64)
        new_k = W.to_storage(rng.standard_normal((slots.size, Hkv, D), dtype=np.float32), dt)
        new_v = W.to_storage(rng.standard_normal((slots.size, Hkv, D), dtype=np.float32), dt)
        if pairs:
            p = np.asarray(pairs, np.int64).reshape(-1, 2)
            gpu_lib.copy_blocks([kd], [vd], torch.from_numpy(p).cuda())
            oracle.copy_blocks([k_host], [v_host], p, dt)
        oracle.reshape_and_cache(new_k, new_v, k_host, v_host, slots, dt)
        if beams is None:
            gpu_lib.reshape_and_cache(to_dev(new_k, dt), to_dev(new_v, dt), kd, vd,
                                      torch.from_numpy(slots).cuda())
        else:
            decode_and_compare(beams, step=(to_dev(new_k, dt), to_dev(new_v, dt),
                                            torch.from_numpy(slots).cuda()))
        torch.cuda.synchronize()
        assert to_host_bits(kd).tobytes() == k_host.tobytes()
        assert to_host_bits(vd).tobytes() == v_host.tobytes()

    def decode_and_compare(beams, step=None):
        lens = np.array([bm.seq_len(s) for s in beams], np.int32)
        max_nb = int(-(-lens.max() // B))
        tables = np.full((len(beams), max_nb), -1, np.int32)
        for i, s in enumerate(beams):
            t = bm.table(s)
            tables[i, :len(t)] = t
        q = W.to_storage(rng.standard_normal((len(beams), Hq, D), dtype=np.float32), dt)
        out = torch.full((len(beams), Hq, D), float("nan"), device="cuda")
        args = (torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), int(lens.max()),
                1 / np.sqrt(D))
        if step is None:
            gpu_lib.paged_attention_decode(out, to_dev(q, dt), kd, vd, *args)
        else:  # the step's new rows (token L - 1 of each beam) with the decode
            gpu_lib.decode_step(out, to_dev(q, dt), *step, kd, vd, *args)
        torch.cuda.synchronize()
        ref = oracle.decode(q, k_host, v_host, dt, tables, lens, 1 / np.sqrt(D))
        assert max_abs(out, ref) <= TOL[dt]

    parent = bm.add_seq(prompt_len)
    write(bm.slots(parent, 0, prompt_len), [])
    beams = [parent] + [bm.fork(parent) for _ in range(width - 1)]
    n_copies = n_killed = 0
    for step in range(steps):
        # kill up to half of the beams, then refill by forking random survivors
        kill = rng.choice(len(beams), int(rng.integers(0, width // 2 + 1)), replace=False)
        for i in sorted(kill, reverse=True):
            bm.free_seq(beams.pop(i))
        n_killed += len(kill)
        while len(beams) < width:
            beams.append(bm.fork(beams[int(rng.integers(len(beams)))]))
        bm.check()
        slots, pairs = [], []
        for s in beams:
            slot, cow = bm.append_token(s)
            slots.append(slot)
            if cow:
                pairs.append(cow)
        bm.check()
        n_copies += len(pairs)
        if one_call:
            write(slots, pairs, beams)
        else:
            write(slots, pairs)
            decode_and_compare(beams)
    # the churn really exercised copy-on-write and release
    assert n_copies > steps // 4 and n_killed > steps // 4
    held = set()
    for s in beams:
        held.update(bm.table(s))
    assert bm.num_free() == NB - len(held)
