"""Benchmark of the paged-attention hot path on one MI355X.

A step is one decode step of the Llama-3-8B-shaped layer batch (256 sequences,
32 query / 8 KV heads, head_dim 128, block 16, bf16 KV, log-normal context
lengths with median 1024 clipped to [16, 8192], blocks scattered over a 12 GB
pool): the 256 new tokens' K/V written to their slots and every sequence's
attention over its cache, in one pkv_decode_step call (the cache write rides
in the decode kernel's launch; the two calls made separately, reshape_and_cache
then paged_attention_decode, are timed as a row beside it).
The headline metric is the achieved KV-read bandwidth of that step:
algorithmic K+V bytes (every valid token of every sequence, once per KV head)
divided by the step time.

Also reported (``rows``): the other kernels of the path on their own
workloads -- OPT-13B-shaped fp16 decode, shared-prefix decode, the 192-pair
copy-on-write copy_blocks, and the chunked causal prefill (TFLOP/s).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--headline-only]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other rows and the CPU baseline (used under the profilers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill row (used under the profilers)")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the FP8 decode row (used under the profilers)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="context tokens of the bounded oracle sample (0: the whole batch)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE run and a "
                         "WRITE_SIZE run (both with --calibrate-copy) into the traffic record under profiles/")
    return ap.parse_args()


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is by sequence, KV head or context; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_71_amd as pkv
    from paged_kv_cache_71_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

    def up(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(TD[dtype])

    class Dev:
        def __init__(self, b):
            self.b = b
            shape = (b.NB, b.B, b.Hkv, b.D)
            self.k = torch.full(shape, float("nan"), dtype=TD[b.dtype], device=dev)
            self.v = torch.full(shape, float("nan"), dtype=TD[b.dtype], device=dev)
            idx = torch.from_numpy(b.block_ids).to(dev)
            self.k.index_copy_(0, idx, up(b.k_blocks, b.dtype))
            self.v.index_copy_(0, idx, up(b.v_blocks, b.dtype))
            self.q = up(b.q, b.dtype)
            self.tables = torch.from_numpy(b.block_tables).to(dev)
            self.lens = torch.from_numpy(b.context_lens).to(dev)
            self.cu = torch.from_numpy(b.cu_seqlens_q).to(dev) if b.cu_seqlens_q is not None else None
            self.slots = torch.from_numpy(b.new_slots).to(dev)
            self.new_k = up(b.new_k, b.dtype)
            self.new_v = up(b.new_v, b.dtype)
            self.out = torch.empty(tuple(self.q.shape), dtype=torch.float32, device=dev)
            if b.cu_seqlens_q is None:
                n = pkv.decode_workspace_size(b.S, b.Hq, b.Hkv, b.D, b.B, b.max_context_len)
            else:
                self.maxq = int(np.max(np.diff(b.cu_seqlens_q)))
                n = pkv.prefill_workspace_size(b.S, self.q.shape[0], self.maxq, b.Hq, b.Hkv, b.D, b.B,
                                               b.dtype, b.max_context_len)
            self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)

        def reshape(self):
            pkv.reshape_and_cache(self.new_k, self.new_v, self.k, self.v, self.slots)

        def step(self):
            b = self.b
            assert self.new_k.shape[0] == b.S, "decode_step: one new token per sequence"
            pkv.decode_step(self.out, self.q, self.new_k, self.new_v, self.slots, self.k, self.v,
                            self.tables, self.lens, b.max_context_len, b.scale, workspace=self.ws)

        def decode(self):
            b = self.b
            pkv.paged_attention_decode(self.out, self.q, self.k, self.v, self.tables, self.lens,
                                       b.max_context_len, b.scale, workspace=self.ws)

        def prefill(self):
            b = self.b
            pkv.paged_attention_prefill(self.out, self.q, self.cu, self.maxq, self.k, self.v,
                                        self.tables, self.lens, b.max_context_len, b.scale,
                                        workspace=self.ws)

        def free(self):
            del self.k, self.v

    def time_fn(fn, iters, warm=3, warm_ms=300.0):
        """Mean ms of fn() over iters launches, HIP events on the current stream,
        after at least `warm` untimed launches and `warm_ms` of back-to-back work
        (the clocks take tens of milliseconds of load to settle)."""
        t0, n = time.time(), 0
        while n < warm or (time.time() - t0) * 1e3 < warm_ms:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        torch.cuda.synchronize()
        for a, z in evs:
            a.record(s)
            fn()
            z.record(s)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(z) for a, z in evs])
        return float(t.mean()), float(np.median(t))

    def graph_time(fn, n_inner=32, reps=20):
        """Device ms per call of a launch-bound call: n_inner calls captured in
        one graph and replayed back to back, so no host work sits between the
        launches (the call-level rows above include the binding's host time)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_inner):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        z.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(z) / (reps * n_inner)
        del g
        return ms

    def mixed_row():
        """The Llama-3-8B decode batch plus one 512-token prefill chunk (after
        8192 cached tokens) in one batch: the mixed call against the decode and
        prefill calls made separately."""
        mb = W.llama3_8b_mixed_bf16(args.seed)
        md = Dev(mb)
        nd = mb.meta["num_decode"]
        cu = md.cu
        maxq = int(np.max(np.diff(mb.cu_seqlens_q)))
        Tq = md.q.shape[0]
        ws = torch.empty(max(pkv.mixed_workspace_size(mb.S, nd, Tq, maxq, mb.Hq, mb.Hkv, mb.D, mb.B,
                                                      mb.dtype, mb.max_context_len), 1),
                         dtype=torch.uint8, device=dev)
        pws = torch.empty(max(pkv.prefill_workspace_size(mb.S - nd, Tq - nd, maxq, mb.Hq, mb.Hkv, mb.D,
                                                         mb.B, mb.dtype, mb.max_context_len), 1),
                          dtype=torch.uint8, device=dev)
        dws = torch.empty(max(pkv.decode_workspace_size(nd, mb.Hq, mb.Hkv, mb.D, mb.B,
                                                        mb.max_context_len), 1),
                          dtype=torch.uint8, device=dev)
        qd, qp = md.q[:nd], md.q[nd:].contiguous()
        od, op = md.out[:nd], md.out[nd:]
        tdec, tpre = md.tables[:nd].contiguous(), md.tables[nd:].contiguous()
        ldec, lpre = md.lens[:nd].contiguous(), md.lens[nd:].contiguous()
        cup = (cu[nd:] - nd).contiguous()

        def mixed():
            pkv.paged_attention_mixed(md.out, md.q, cu, nd, maxq, md.k, md.v, md.tables, md.lens,
                                      mb.max_context_len, mb.scale, workspace=ws)

        def serial():
            pkv.paged_attention_decode(od, qd, md.k, md.v, tdec, ldec, mb.max_context_len,
                                       mb.scale, workspace=dws)
            pkv.paged_attention_prefill(op, qp, cup, maxq, md.k, md.v, tpre, lpre,
                                        mb.max_context_len, mb.scale, workspace=pws)

        ms_m, _ = time_fn(mixed, 20)
        ms_s, _ = time_fn(serial, 20)
        log(f"[bench] mixed: {ms_m * 1e3:.1f} us (separate calls {ms_s * 1e3:.1f} us)")
        md.free()
        del md
        torch.cuda.empty_cache()
        return {"ms": round(ms_m, 5), "separate_calls_ms": round(ms_s, 5),
                "speedup_vs_separate_calls": round(ms_s / ms_m, 3)}

    def prefill_row():
        """Chunked causal prefill of 8 sequences x 512 new tokens (bf16)."""
        pb = W.prefill_bf16(args.seed)
        pd = Dev(pb)
        ms, _ = time_fn(pd.prefill, 10)
        flops = 0
        for s in range(pb.S):
            Q = int(pb.cu_seqlens_q[s + 1] - pb.cu_seqlens_q[s])
            L = int(pb.context_lens[s])
            flops += 4 * pb.Hq * pb.D * sum(L - Q + i + 1 for i in range(Q))
        log(f"[bench] prefill: {ms:.3f} ms, {flops / ms / 1e9:.0f} TFLOP/s")
        pd.free()
        del pd
        torch.cuda.empty_cache()
        return {"ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 1),
                "frac_of_bf16_peak": round(flops / ms / 1e9 / BF16_DENSE_TFLOPS, 4)}

    def prefill_fp8_row(bf16_ms):
        """The same 8 x 512 chunks over FP8 (E4M3) pools with per-KV-head scales
        (q bf16); the codes are widened to bf16 on their way into LDS."""
        pb = W.prefill_bf16(args.seed)
        f8 = W.fp8_pools(pb, args.seed + 2)
        shape = (pb.NB, pb.B, pb.Hkv, pb.D)
        idx = torch.from_numpy(pb.block_ids).to(dev)
        k8 = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
        v8 = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
        k8.index_copy_(0, idx, torch.from_numpy(f8.k_blocks).to(dev))
        v8.index_copy_(0, idx, torch.from_numpy(f8.v_blocks).to(dev))
        ks8 = torch.from_numpy(f8.k_scale).to(dev)
        vs8 = torch.from_numpy(f8.v_scale).to(dev)
        del f8
        q = up(pb.q, "bf16")
        cu = torch.from_numpy(pb.cu_seqlens_q).to(dev)
        tables = torch.from_numpy(pb.block_tables).to(dev)
        lens = torch.from_numpy(pb.context_lens).to(dev)
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=dev)
        maxq = int(np.max(np.diff(pb.cu_seqlens_q)))
        ws = torch.empty(max(pkv.prefill_workspace_size(pb.S, q.shape[0], maxq, pb.Hq, pb.Hkv, pb.D,
                                                        pb.B, "fp8", pb.max_context_len), 1),
                         dtype=torch.uint8, device=dev)

        def run():
            pkv.paged_attention_prefill_fp8(out, q, cu, maxq, k8, v8, ks8, vs8, tables, lens,
                                            pb.max_context_len, pb.scale, workspace=ws)

        ms, _ = time_fn(run, 10)
        flops = 0
        for s in range(pb.S):
            Q = int(pb.cu_seqlens_q[s + 1] - pb.cu_seqlens_q[s])
            L = int(pb.context_lens[s])
            flops += 4 * pb.Hq * pb.D * sum(L - Q + i + 1 for i in range(Q))
        log(f"[bench] prefill fp8: {ms:.3f} ms, {flops / ms / 1e9:.0f} TFLOP/s")
        del k8, v8, q, out, ws
        torch.cuda.empty_cache()
        return {"ms": round(ms, 4), "TFLOP/s": round(flops / ms / 1e9, 1),
                "speedup_vs_bf16": round(bf16_ms / ms, 3)}

    if args.prefill_only:
        print(json.dumps({"prefill_bf16_8x512": prefill_row()}), flush=True)
        return

    def cascade_row(bb, dd, plain_ms):
        """The shared-prefix batch through the cascade path: each prompt's
        prefix blocks read once per 4-sample group, merged with the suffixes."""
        n = bb.meta["n"]
        cu = torch.arange(0, bb.S + 1, n, dtype=torch.int32, device=dev)
        plen = (bb.meta["prompt_len"] // bb.B) * bb.B
        plens = torch.full((bb.S // n,), plen, dtype=torch.int32, device=dev)
        ws = torch.empty(max(pkv.decode_cascade_workspace_size(
            bb.S, bb.Hq, bb.Hkv, bb.D, bb.B, bb.max_context_len, bb.S // n, n, plen, bb.dtype), 1),
            dtype=torch.uint8, device=dev)

        def run():
            pkv.paged_attention_decode_cascade(dd.out, dd.q, dd.k, dd.v, dd.tables, dd.lens,
                                               bb.max_context_len, bb.scale, cu, plens, n, plen,
                                               workspace=ws)

        ms, _ = time_fn(run, 20)
        log(f"[bench] decode_shared_prefix_bf16_cascade: {ms * 1e3:.1f} us")
        return {"ms": round(ms, 5), "logical_GB/s": round(bb.kv_read_bytes() / ms / 1e6, 1),
                "unique_GB/s": round(bb.unique_kv_bytes() / ms / 1e6, 1),
                "speedup_vs_plain": round(plain_ms / ms, 3)}

    def fp8_row(b, d, bf16_ms):
        """The Llama-3-8B batch over FP8 (E4M3) pools with per-KV-head scales:
        half the KV bytes of the bf16 step."""
        t0 = time.time()
        f8 = W.fp8_pools(b, args.seed + 1)
        shape = (b.NB, b.B, b.Hkv, b.D)
        idx = torch.from_numpy(b.block_ids).to(dev)
        k8 = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
        v8 = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
        k8.index_copy_(0, idx, torch.from_numpy(f8.k_blocks).to(dev))
        v8.index_copy_(0, idx, torch.from_numpy(f8.v_blocks).to(dev))
        ks8 = torch.from_numpy(f8.k_scale).to(dev)
        vs8 = torch.from_numpy(f8.v_scale).to(dev)
        del f8
        log(f"[bench] fp8 pools generated in {time.time() - t0:.1f}s")

        def dec8():
            pkv.paged_attention_decode_fp8(d.out, d.q, k8, v8, ks8, vs8, d.tables, d.lens,
                                           b.max_context_len, b.scale, workspace=d.ws)

        ms8, _ = time_fn(dec8, 20)
        b8 = b.kv_read_bytes() // 2
        log(f"[bench] decode_llama3_8b_fp8: {ms8 * 1e3:.1f} us, {b8 / ms8 / 1e6:.0f} GB/s of FP8 KV")
        row = {"ms": round(ms8, 5), "GB/s": round(b8 / ms8 / 1e6, 1),
               "frac_of_hbm_peak": round(b8 / ms8 / 1e6 / HBM_PEAK_GBS, 4)}
        if bf16_ms:
            row["speedup_vs_bf16"] = round(bf16_ms / ms8, 3)
        del k8, v8
        return row

    if args.fp8_only:
        b = W.llama3_8b_bf16(args.seed)
        d = Dev(b)
        d.free()
        print(json.dumps({"decode_llama3_8b_fp8": fp8_row(b, d, None)}), flush=True)
        return

    # ------------------------------------------------------------ headline
    t0 = time.time()
    b = W.llama3_8b_bf16(args.seed)
    log(f"[bench] llama3_8b_bf16 generated in {time.time() - t0:.1f}s: S={b.S} sum(L)="
        f"{int(b.context_lens.sum())} max={b.max_context_len} blocks={b.block_ids.shape[0]}")
    d = Dev(b)
    kv_bytes = b.kv_read_bytes()
    stream = torch.cuda.current_stream()

    step = d.step

    # W untimed warm-up steps, continued (still untimed) until 300 ms of steps
    # have run: the clocks take tens of milliseconds of load to settle
    t0, n_warm = time.time(), 0
    while n_warm < args.warmup or (time.time() - t0) * 1e3 < 300.0:
        step()
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # the timed region: exactly K steps, events at its two ends only (an event
    # recorded between launches costs the stream a few microseconds)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    # at least 100 more steps (K if larger) with an event after every step
    # (its launches: the decode kernels' duration for the roofline): the
    # distribution of step times
    n_ev = max(100, args.steps)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
    torch.cuda.synchronize()
    step_ev[0].record(stream)
    for i in range(n_ev):
        step()
        step_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(n_ev)])
    dec_ms = float(np.mean(step_ms))
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (dec_ms * 1e-3) / 1e9
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us, "
        f"{achieved:.0f} GB/s on the decode kernels")

    result = {
        "metric": "paged-attn decode achieved KV-read HBM GB/s (% of peak), Llama-3-8B GQA",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_gqa_decode_bf16: one decode step (the new tokens' cache "
                        "write + paged attention, pkv_decode_step), 256 sequences, 32 q / 8 kv "
                        "heads, head_dim 128, block 16, log-normal lengths median 1024 clipped "
                        "[16, 8192], 12 GB pool",
            "sequences": b.S,
            "context_tokens": int(b.context_lens.sum()),
            "kv_bytes_per_step": kv_bytes,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
            "warmup_steps_run": n_warm,
            "evented_steps": n_ev,
            "evented_step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5)
                                            for q in (10, 50, 90)],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "decode_step (decode_split_kernel with the cache write + "
                      "decode_merge_kernel launches)",
            "ms_per_launch": round(dec_ms, 5),
        },
    }

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.headline_only:
        rows = {}
        # decode with cold caches: before every launch a 2 GiB buffer is READ
        # (larger than L2 + the 256 MB Infinity Cache), which evicts the KV
        # without leaving dirty lines whose write-back would be charged to decode
        flush = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        fl = []
        for _ in range(100):
            flush.sum()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            d.decode()
            z.record(stream)
            fl.append((a, z))
        torch.cuda.synchronize()
        ft = np.array([a.elapsed_time(z) for a, z in fl])
        fms = float(np.median(ft))
        rows["decode_llama3_8b_flushed"] = {
            "ms_median": round(fms, 5), "GB/s": round(kv_bytes / fms / 1e6, 1),
            "ms_p10_p90": [round(float(np.percentile(ft, q)), 5) for q in (10, 90)],
            "launches": len(fl)}
        del flush
        def two_calls():
            d.reshape()
            d.decode()

        tms, _ = time_fn(two_calls, 20)
        rows["decode_step_as_two_calls"] = {"ms": round(tms, 5),
                                            "GB/s": round(kv_bytes / tms / 1e6, 1)}
        rms, _ = time_fn(d.reshape, 20)
        rb = 2 * 2 * b.new_k.size * 2   # read + write of K and V rows
        rgms = graph_time(d.reshape)
        rows["reshape_and_cache_256_tokens"] = {"ms": round(rms, 5), "GB/s": round(rb / rms / 1e6, 1),
                                                "graph_ms_per_call": round(rgms, 5),
                                                "graph_GB/s": round(rb / rgms / 1e6, 1)}

        rows["decode_llama3_8b_fp8"] = fp8_row(b, d, dec_ms)
        d.free()
        del d
        torch.cuda.empty_cache()

        # one GPU's share of the same batch at tensor parallelism 8: 4 query
        # heads over 1 KV head of every block (an eighth of the bytes)
        sb = W.llama3_8b_tp8_shard(args.seed)
        sd = Dev(sb)
        ms, _ = time_fn(sd.decode, 100)
        rows["decode_llama3_8b_tp8_shard"] = {"ms": round(ms, 5),
                                              "GB/s": round(sb.kv_read_bytes() / ms / 1e6, 1),
                                              "kv_bytes": sb.kv_read_bytes()}
        log(f"[bench] decode_llama3_8b_tp8_shard: {ms * 1e3:.1f} us")
        sd.free()
        del sd
        torch.cuda.empty_cache()

        for name, gen in (("decode_opt13b_f16", lambda: W.opt13b_f16(args.seed)),
                          ("decode_shared_prefix_bf16", lambda: W.shared_prefix_bf16(args.seed))):
            bb = gen()
            dd = Dev(bb)
            ms, _ = time_fn(dd.decode, 20)
            rows[name] = {"ms": round(ms, 5), "logical_GB/s": round(bb.kv_read_bytes() / ms / 1e6, 1),
                          "unique_GB/s": round(bb.unique_kv_bytes() / ms / 1e6, 1)}
            log(f"[bench] {name}: {ms * 1e3:.1f} us")
            if name == "decode_shared_prefix_bf16":
                rows[name + "_cascade"] = cascade_row(bb, dd, ms)
            dd.free()
            del dd
            torch.cuda.empty_cache()

        # copy-on-write copy of the shared-prefix sub-case: 64 prompts x 3 copies of a 16-token block
        B, Hkv, D = 16, 8, 128
        NBc = 4096
        kc = torch.randn((NBc, B, Hkv, D), device=dev).to(torch.bfloat16)
        vc = torch.randn((NBc, B, Hkv, D), device=dev).to(torch.bfloat16)
        perm = np.random.default_rng(0).permutation(NBc)
        pairs = torch.from_numpy(np.stack([np.repeat(perm[:64], 3), perm[64:64 + 192]], 1)
                                 .astype(np.int64)).to(dev)
        ms, _ = time_fn(lambda: pkv.copy_blocks([kc], [vc], pairs), 20)
        cb = 192 * 2 * 2 * B * Hkv * D * 2
        gms = graph_time(lambda: pkv.copy_blocks([kc], [vc], pairs))
        rows["copy_blocks_192_pairs"] = {"ms": round(ms, 5), "GB/s": round(cb / ms / 1e6, 1),
                                         "graph_ms_per_call": round(gms, 5),
                                         "graph_GB/s": round(cb / gms / 1e6, 1)}

        # swap-out of 1024 scattered blocks (K and V, 64 KiB per block) to a
        # pinned host pool: one swap_blocks launch against one copy per block
        host_k = torch.empty((1024, B, Hkv, D), dtype=torch.bfloat16).pin_memory()
        host_v = torch.empty_like(host_k).pin_memory()
        src = np.random.default_rng(1).permutation(NBc)[:1024]
        sp = torch.from_numpy(np.stack([src, np.arange(1024)], 1).astype(np.int64)).to(dev)
        ms_k, _ = time_fn(lambda: pkv.swap_blocks([kc, vc], [host_k, host_v], sp), 10)
        src_l = src.tolist()

        def per_block():
            for i, s_ in enumerate(src_l):
                host_k[i].copy_(kc[s_], non_blocking=True)
                host_v[i].copy_(vc[s_], non_blocking=True)

        ms_p, _ = time_fn(per_block, 3, warm=1)
        sb = 1024 * 2 * B * Hkv * D * 2
        rows["swap_out_1024_blocks"] = {"ms": round(ms_k, 4), "GB/s": round(sb / ms_k / 1e6, 1),
                                        "per_block_copies_ms": round(ms_p, 4),
                                        "speedup_vs_per_block": round(ms_p / ms_k, 2)}
        log(f"[bench] swap_out 1024 blocks: {ms_k * 1e3:.1f} us ({sb / ms_k / 1e6:.1f} GB/s), "
            f"per-block copies {ms_p * 1e3:.1f} us")
        del host_k, host_v
        del kc, vc
        torch.cuda.empty_cache()

        rows["prefill_bf16_8x512"] = prefill_row()
        rows["prefill_fp8_8x512"] = prefill_fp8_row(rows["prefill_bf16_8x512"]["ms"])
        rows["mixed_llama3_8b_256_decodes_512_chunk"] = mixed_row()
        result["rows"] = rows

    if not args.headline_only and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_sample_tokens)

    print(json.dumps(result), flush=True)


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "decode_llama3_8b_bf16_traffic.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_71_amd", "csrc", "decode.hip")
COPY_BYTES = 1 << 30


def _counter_means(path):
    """Per-kernel mean of one rocprofv3 counter (KiB per dispatch), and the
    value the largest __amd_rocclr_copyBuffer dispatch (the 1 GiB copy) read."""
    import csv
    per, copy = {}, 0.0
    for r in csv.DictReader(open(path)):
        name, val = r["Kernel_Name"], float(r["Counter_Value"])
        if "__amd_rocclr_copyBuffer" in name:
            copy = max(copy, val)
        for k in ("decode_split_kernel", "decode_merge_kernel", "reshape_and_cache_kernel"):
            if k in name:
                per.setdefault(k, []).append(val)
    if copy <= 0:
        raise SystemExit(f"{path}: no 1 GiB copy dispatch (run the counter pass with --calibrate-copy)")
    return {k: float(np.mean(v)) for k, v in per.items()}, copy


def record_traffic(fetch_csv, write_csv):
    """Scale FETCH_SIZE / WRITE_SIZE so that the 1 GiB copy reads and writes
    exactly 1 GiB, then store bytes per dispatch of the decode kernels together
    with the sha256 of the decode source they were measured on."""
    import hashlib
    from paged_kv_cache_71_amd import workloads as W
    fetch, fcopy = _counter_means(fetch_csv)
    write, wcopy = _counter_means(write_csv)
    fs, ws = COPY_BYTES / 1024 / fcopy, COPY_BYTES / 1024 / wcopy
    per = {}
    for k, short in (("decode_split_kernel", "split"), ("decode_merge_kernel", "merge"),
                     ("reshape_and_cache_kernel", "reshape")):
        if k in fetch and k in write:  # (no reshape launch when the step is one call)
            per[short] = {"read": round(fetch[k] * 1024 * fs), "write": round(write[k] * 1024 * ws)}
    step = sum(per[k]["read"] + per[k]["write"] for k in ("split", "merge"))
    rec = {
        "workload": "Llama-3-8B-shaped decode, bf16 KV, 256 sequences, 32 q / 8 kv heads, head_dim 128, block 16",
        "decode_hip_sha256": hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest(),
        "traffic_bytes_per_step": step,
        "algorithmic_kv_bytes_per_step": int(W.llama3_8b_bf16(0).kv_read_bytes()),
        "fetch_scale": round(fs, 5),
        "write_scale": round(ws, 5),
        "per_kernel_bytes": per,
    }
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def measured_traffic():
    """HBM bytes per decode step from the committed rocprofv3 counter runs, if
    they were taken on the decode source as it is now (else None)."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_JSON))
        digest = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("decode_hip_sha256") != digest:
        return None
    return rec.get("traffic_bytes_per_step")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, sample_tokens):
    """The fp64 oracle as it is, on a bounded sample of the same workload (the
    first sequences of the batch until ``sample_tokens`` context tokens; all of
    them by default), run on every core of this process's affinity mask: the
    sample's sequences are cut into parts of similar length, one oracle call per
    part (the oracle itself is unchanged; its result is that of one call)."""
    from oracle.parallel import decode_par, host_threads
    k, v, tables = b.compact_pool()
    n = b.S
    if sample_tokens:
        n = min(b.S, int(np.searchsorted(np.cumsum(b.context_lens), sample_tokens) + 1))
    sel = np.arange(n)
    threads = host_threads(cap=1 << 16)
    times, t0 = [], time.perf_counter()
    # about 10 s of wall time: whole passes until 10 s have gone by (3 to 30)
    while len(times) < 30 and (len(times) < 3 or time.perf_counter() - t0 < 10.0):
        t1 = time.perf_counter()
        decode_par(b.q, k, v, b.dtype, tables, b.context_lens, b.scale, seqs=sel, threads=threads)
        times.append(time.perf_counter() - t1)
    dt = float(np.median(times))
    tokens = int(b.context_lens[sel].sum())
    bytes_ = tokens * 2 * b.Hkv * b.D * 2
    log(f"[bench] cpu oracle: {n} sequences, {tokens} tokens, {threads} threads, "
        f"median {dt:.2f} s per pass of {len(times)}")
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} of {b.S} sequences ({tokens} context tokens, {bytes_ / 1e6:.0f} MB of "
                      f"KV), fp64 C oracle on {threads} threads (one per core of the affinity "
                      f"mask, {cpu_model()}), median of {len(times)} passes of {dt:.2f} s"}


if __name__ == "__main__":
    main()
