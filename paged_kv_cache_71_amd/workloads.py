"""Seeded synthetic inputs shaped like the pages' workloads.

This module only DRAWS inputs: sequence lengths, a shuffled free list, block
tables that hand out blocks in free-list order, and N(0, 1) query/key/value
values rounded to the storage dtype.  It holds none of the attention
arithmetic, so both the HIP path and the fp64 oracle can consume its output
without sharing any code with each other.

Workloads (stand-ins for the ShareGPT/Alpaca traces the pages measure on,
which are not available here):

* ``tiny_f32``      - 4 sequences, lengths {6, 17, 1, 33}, MHA 4 heads, head_dim 64,
                      block 4, 64-block pool, tables from a seeded shuffle.
* ``opt13b_f16``    - OPT-13B-shaped layer: 40 q / 40 kv heads, head_dim 128, block 16,
                      40 sequences with lengths uniform on [1, 2048].
* ``llama3_8b_bf16``- Llama-3-8B-shaped layer: 32 q / 8 kv heads (GQA 4), head_dim 128,
                      block 16, 256 sequences, log-normal lengths (median 1024,
                      sigma 1 in log space) clipped to [16, 8192].
* ``shared_prefix_bf16`` - 64 prompts of 2000 tokens, each forked into 4 samples whose
                      tables alias the prompt's blocks, plus private suffixes of
                      uniform [1, 512] tokens.
* ``prefill_bf16``  - 8 sequences, each a 512-token query chunk after a paged prior
                      context of uniform [4096, 32768] tokens.
* ``fp8_pools``     - FP8 (OCP E4M3) K/V codes for any of the batches above: random
                      codes drawn directly (no quantization is computed here) and
                      one random scale per KV head for K and for V.

Draw order for every workload: lengths -> free-list permutation -> q -> K/V.
Rows of a block past the sequence's fill, unreferenced pool blocks and table
entries past a sequence's last block are poisoned (NaN bit patterns, -1), so a
kernel that reads them shows it.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}

# Pool sized like a 12 GB (1e9-byte units) K+V budget for one layer.
POOL_BYTES = 12e9


def pool_blocks_for(B: int, Hkv: int, D: int, dtype: str, pool_bytes: float = POOL_BYTES) -> int:
    """Number of physical blocks (K and V) that fit in ``pool_bytes``."""
    return int(pool_bytes // (2 * B * Hkv * D * DTYPE_BYTES[dtype]))


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one token occupies across ``num_layers`` layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage dtype (round-to-nearest-even) and return
    the stored representation: float32 for f32, raw uint16 bits otherwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        bits = x.view(np.uint32)
        rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out = rounded.astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            out[nan] = 0x7FC0
        return out
    raise ValueError(dtype)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float32 (exact for all three dtypes)."""
    if dtype == "f32":
        return np.asarray(a, np.float32)
    if dtype == "f16":
        return np.asarray(a, np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


@dataclass
class PagedBatch:
    """One batch of paged attention inputs.

    Physical pool layout is ``[NB, B, Hkv, D]`` for K and for V.  Only the blocks
    in ``block_ids`` hold data (``k_blocks[i]`` is the content of physical block
    ``block_ids[i]``); every other block is poison.
    """
    name: str
    dtype: str
    S: int
    Hq: int
    Hkv: int
    D: int
    B: int
    NB: int
    scale: float
    context_lens: np.ndarray          # int32 [S] (prefill: prior + chunk)
    block_tables: np.ndarray          # int32 [S, max_nb], -1 past each sequence's last block
    block_ids: np.ndarray             # int64 [n] distinct physical blocks holding data
    k_blocks: np.ndarray              # storage [n, B, Hkv, D]
    v_blocks: np.ndarray              # storage [n, B, Hkv, D]
    q: np.ndarray                     # storage [S, Hq, D] (decode) or [Tq, Hq, D] (prefill)
    new_slots: np.ndarray             # int64 [T] slots of this step's new tokens
    new_k: np.ndarray                 # storage [T, Hkv, D]
    new_v: np.ndarray                 # storage [T, Hkv, D]
    cu_seqlens_q: np.ndarray | None = None   # int32 [S+1] (prefill only)
    meta: dict = field(default_factory=dict)

    @property
    def max_nb(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0

    @property
    def is_prefill(self) -> bool:
        return self.cu_seqlens_q is not None

    def kv_read_bytes(self) -> int:
        """Algorithmic K+V bytes one attention pass reads: every valid token of
        every sequence, once per KV head (aliased blocks counted per sequence)."""
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.Hkv * self.D * DTYPE_BYTES[self.dtype]

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct written rows (aliased blocks counted once)."""
        written = self.meta.get("written_rows")
        if written is None:
            return self.kv_read_bytes()
        return int(written) * 2 * self.Hkv * self.D * DTYPE_BYTES[self.dtype]

    def compact_pool(self, extra_poison_blocks: int = 1):
        """Pool holding only the data blocks (plus ``extra_poison_blocks`` poisoned
        ones) and tables remapped to it.  Attention results do not depend on
        which physical blocks hold the data, so this is an equivalent input of
        small size for host-side checks."""
        n = self.block_ids.shape[0]
        shape = (n + extra_poison_blocks, self.B, self.Hkv, self.D)
        k = np.empty(shape, STORAGE_NP[self.dtype])
        v = np.empty(shape, STORAGE_NP[self.dtype])
        k[:n], v[:n] = self.k_blocks, self.v_blocks
        k[n:], v[n:] = NAN_BITS[self.dtype], NAN_BITS[self.dtype]
        order = np.argsort(self.block_ids, kind="stable")
        ids_sorted = self.block_ids[order]
        tables = np.full_like(self.block_tables, -1)
        used = self.block_tables >= 0          # padding entries are -1
        tables[used] = order[np.searchsorted(ids_sorted, self.block_tables[used])]
        return k, v, tables

    def full_pool(self):
        """The whole poisoned pool ``[NB, B, Hkv, D]`` with data blocks scattered in
        (host memory; only for small pools)."""
        shape = (self.NB, self.B, self.Hkv, self.D)
        k = np.full(shape, NAN_BITS[self.dtype], STORAGE_NP[self.dtype])
        v = np.full(shape, NAN_BITS[self.dtype], STORAGE_NP[self.dtype])
        k[self.block_ids], v[self.block_ids] = self.k_blocks, self.v_blocks
        return k, v


def _normal(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 22) -> np.ndarray:
    """N(0, 1) values rounded to ``dtype``.  Large draws are split into chunks, each
    from its own generator seeded by one draw of ``rng``, filled in parallel;
    the result depends only on ``rng``'s state and the shape."""
    n = int(np.prod(shape))
    out = np.empty(n, STORAGE_NP[dtype])
    if n <= chunk:
        out[:] = to_storage(rng.standard_normal(n, dtype=np.float32), dtype)
        return out.reshape(shape)
    starts = list(range(0, n, chunk))
    seeds = rng.integers(0, 2**63 - 1, size=len(starts))

    def fill(i):
        lo = starts[i]
        m = min(chunk, n - lo)
        g = np.random.default_rng(int(seeds[i]))
        out[lo:lo + m] = to_storage(g.standard_normal(m, dtype=np.float32), dtype)

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(len(starts))))
    return out.reshape(shape)


def _hand_out(free_order: np.ndarray, counts) -> list[np.ndarray]:
    """Give each request ``counts[i]`` blocks, popping the front of the free list."""
    total = int(np.sum(counts))
    if total > free_order.shape[0]:
        raise MemoryError(f"pool too small: need {total} blocks, have {free_order.shape[0]}")
    out, pos = [], 0
    for c in counts:
        out.append(free_order[pos:pos + c].astype(np.int64))
        pos += c
    return out


def _tables(per_seq_blocks: list[np.ndarray], max_nb: int | None = None) -> np.ndarray:
    S = len(per_seq_blocks)
    width = max([len(b) for b in per_seq_blocks] + [1]) if max_nb is None else max_nb
    t = np.full((S, width), -1, np.int32)
    for s, b in enumerate(per_seq_blocks):
        t[s, :len(b)] = b
    return t


def _slots_of(table_row: np.ndarray, positions: np.ndarray, B: int) -> np.ndarray:
    return table_row[positions // B].astype(np.int64) * B + positions % B


def _build(name, rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows, chunk_lens=None, meta=None,
           free_order=None, seq_blocks=None, block_fill=None):
    """Common tail of every generator: values for the data blocks, poison, the
    new-token slots of this step."""
    S = len(lengths)
    lengths = np.asarray(lengths, np.int32)
    if seq_blocks is None:
        counts = [-(-int(L) // B) for L in lengths]
        seq_blocks = _hand_out(free_order, counts)
    tables = _tables(seq_blocks)
    # distinct data blocks, in order of first use, and how many rows each holds
    if block_fill is None:
        block_fill = {}
        for s in range(S):
            L = int(lengths[s])
            for j, b in enumerate(seq_blocks[s]):
                block_fill[int(b)] = max(block_fill.get(int(b), 0), min(B, L - j * B))
    block_ids = np.array(list(block_fill.keys()), np.int64)
    q = _normal(rng, (q_rows, Hq, D), dtype)
    n = block_ids.shape[0]
    k_blocks = _normal(rng, (n, B, Hkv, D), dtype)
    v_blocks = _normal(rng, (n, B, Hkv, D), dtype)
    fills = np.array([block_fill[int(b)] for b in block_ids], np.int64)
    stale = np.arange(B)[None, :] >= fills[:, None]          # rows never written
    k_blocks[stale] = NAN_BITS[dtype]
    v_blocks[stale] = NAN_BITS[dtype]
    # this step's new tokens: the last token of each sequence (decode) or the
    # whole chunk (prefill); their K/V are the values already at their slots
    where = {int(b): i for i, b in enumerate(block_ids)}
    slots, ks, vs = [], [], []
    for s in range(S):
        L = int(lengths[s])
        nnew = 1 if chunk_lens is None else int(chunk_lens[s])
        if L == 0:
            continue
        pos = np.arange(L - nnew, L)
        sl = _slots_of(tables[s], pos, B)
        slots.append(sl)
        idx = np.array([where[int(x)] for x in sl // B])
        ks.append(k_blocks[idx, sl % B])
        vs.append(v_blocks[idx, sl % B])
    new_slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    new_k = np.concatenate(ks) if ks else np.zeros((0, Hkv, D), STORAGE_NP[dtype])
    new_v = np.concatenate(vs) if vs else np.zeros((0, Hkv, D), STORAGE_NP[dtype])
    cu = None
    if chunk_lens is not None:
        cu = np.zeros(S + 1, np.int32)
        cu[1:] = np.cumsum(chunk_lens)
    meta = dict(meta or {})
    meta.setdefault("written_rows", int(fills.sum()))
    return PagedBatch(name=name, dtype=dtype, S=S, Hq=Hq, Hkv=Hkv, D=D, B=B, NB=NB,
                      scale=1.0 / math.sqrt(D), context_lens=lengths, block_tables=tables,
                      block_ids=block_ids, k_blocks=k_blocks, v_blocks=v_blocks, q=q,
                      new_slots=new_slots, new_k=new_k, new_v=new_v, cu_seqlens_q=cu, meta=meta)


def decode_batch(seed: int, lengths, Hq: int, Hkv: int, D: int, B: int, dtype: str,
                 NB: int | None = None, name: str = "decode") -> PagedBatch:
    """Decode batch with the given context lengths and a shuffled pool."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int32)
    if NB is None:
        NB = max(64, 2 * int(sum(-(-int(L) // B) for L in lengths)))
    free_order = rng.permutation(NB)
    return _build(name, rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows=len(lengths),
                  free_order=free_order)


def tiny_f32(seed: int = 0) -> PagedBatch:
    """4 sequences {6, 17, 1, 33}, MHA 4 heads, head_dim 64, block 4, pool of 64."""
    rng = np.random.default_rng(seed)
    lengths = np.array([6, 17, 1, 33], np.int32)
    free_order = rng.permutation(64)
    return _build("tiny_f32", rng, lengths, 4, 4, 64, 4, 64, "f32", q_rows=4,
                  free_order=free_order)


def opt13b_f16(seed: int = 0, S: int = 40, max_len: int = 2048, NB: int | None = None) -> PagedBatch:
    """OPT-13B-shaped decode layer (MHA 40 heads, head_dim 128, block 16, fp16)."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=S).astype(np.int32)
    NB = pool_blocks_for(16, 40, 128, "f16") if NB is None else NB
    free_order = rng.permutation(NB)
    return _build("opt13b_f16", rng, lengths, 40, 40, 128, 16, NB, "f16", q_rows=S,
                  free_order=free_order)


def lognormal_lengths(rng: np.random.Generator, S: int, median: float = 1024.0,
                      sigma: float = 1.0, lo: int = 16, hi: int = 8192) -> np.ndarray:
    """clip(round(exp(N(ln median, sigma))), lo, hi)."""
    x = np.exp(rng.normal(math.log(median), sigma, size=S))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def llama3_8b_bf16(seed: int = 0, S: int = 256, median: float = 1024.0, hi: int = 8192,
                   NB: int | None = None) -> PagedBatch:
    """Llama-3-8B-shaped decode layer (32 q / 8 kv heads, head_dim 128, block 16, bf16)."""
    rng = np.random.default_rng(seed)
    lengths = lognormal_lengths(rng, S, median=median, hi=hi)
    NB = pool_blocks_for(16, 8, 128, "bf16") if NB is None else NB
    free_order = rng.permutation(NB)
    return _build("llama3_8b_bf16", rng, lengths, 32, 8, 128, 16, NB, "bf16", q_rows=S,
                  free_order=free_order)


def llama3_8b_tp8_shard(seed: int = 0, S: int = 256, median: float = 1024.0,
                        hi: int = 8192) -> PagedBatch:
    """One GPU's share of the Llama-3-8B decode layer at tensor parallelism 8:
    4 query heads over 1 KV head, the same lengths, block count and block
    placement as ``llama3_8b_bf16(seed)`` (each GPU holds one KV head of every
    block)."""
    rng = np.random.default_rng(seed)
    lengths = lognormal_lengths(rng, S, median=median, hi=hi)
    NB = pool_blocks_for(16, 8, 128, "bf16")
    free_order = rng.permutation(NB)
    return _build("llama3_8b_tp8_shard", rng, lengths, 4, 1, 128, 16, NB, "bf16", q_rows=S,
                  free_order=free_order)


def shared_prefix_bf16(seed: int = 0, prompts: int = 64, n: int = 4, prompt_len: int = 2000,
                       max_suffix: int = 512, NB: int | None = None) -> PagedBatch:
    """Shared-prefix decode batch after forking: each prompt's ``n`` samples alias
    the prompt's blocks (refcount n) and own private suffix blocks.

    If ``prompt_len`` is not a multiple of the block size, the prompt's last block
    is partly filled; its copy-on-write has already happened in this state: the
    first n-1 samples hold private copies (same prompt rows, then their own
    tokens) and the last sample writes into the original block."""
    B, Hq, Hkv, D, dtype = 16, 32, 8, 128, "bf16"
    rng = np.random.default_rng(seed)
    suffix = rng.integers(1, max_suffix + 1, size=prompts * n).astype(np.int32)
    NB = pool_blocks_for(B, Hkv, D, dtype) if NB is None else NB
    free_order = rng.permutation(NB)
    lengths = (prompt_len + suffix).astype(np.int32)
    full_prefix = prompt_len // B
    partial = prompt_len % B
    pos, seq_blocks, copies = 0, [], []
    block_fill: dict[int, int] = {}

    def take(c):
        nonlocal pos
        if pos + c > NB:
            raise MemoryError("pool too small")
        r = free_order[pos:pos + c].astype(np.int64)
        pos += c
        return r

    for p in range(prompts):
        prefix = take(full_prefix + (1 if partial else 0))
        for b in prefix[:full_prefix]:
            block_fill[int(b)] = B
        for j in range(n):
            s = p * n + j
            L = int(lengths[s])
            blocks = list(prefix[:full_prefix])
            if partial:
                if j < n - 1:          # copy-on-write: private copy of the shared last block
                    cp = int(take(1)[0])
                    copies.append((int(prefix[full_prefix]), cp))
                    blocks.append(cp)
                else:                  # last writer keeps the original
                    blocks.append(int(prefix[full_prefix]))
                block_fill[int(blocks[-1])] = min(B, L - full_prefix * B)
            need = -(-L // B) - len(blocks)
            extra = take(need)
            for k, b in enumerate(extra):
                block_fill[int(b)] = min(B, L - (len(blocks) + k) * B)
            blocks.extend(int(b) for b in extra)
            seq_blocks.append(np.array(blocks, np.int64))
    batch = _build("shared_prefix_bf16", rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows=prompts * n,
                   seq_blocks=seq_blocks, block_fill=block_fill,
                   meta={"prompts": prompts, "n": n, "prompt_len": prompt_len,
                         "cow_pairs": np.array(copies, np.int64).reshape(-1, 2)})
    if partial:
        # the private copies start as copies of the shared block: same prompt rows
        where = {int(b): i for i, b in enumerate(batch.block_ids)}
        for src, dst in copies:
            batch.k_blocks[where[dst], :partial] = batch.k_blocks[where[src], :partial]
            batch.v_blocks[where[dst], :partial] = batch.v_blocks[where[src], :partial]
        # refresh the new-token values (a suffix token may live in a copy block)
        sl = batch.new_slots
        idx = np.array([where[int(x)] for x in sl // B])
        batch.new_k = batch.k_blocks[idx, sl % B]
        batch.new_v = batch.v_blocks[idx, sl % B]
    return batch


def grouped_batch(seed: int, group_sizes, prefix_blocks, suffix_lens, Hq: int, Hkv: int, D: int,
                  B: int, dtype: str, NB: int | None = None, name: str = "grouped") -> PagedBatch:
    """Decode batch whose sequences come in consecutive groups: group g has
    ``group_sizes[g]`` members that all alias its ``prefix_blocks[g]`` full
    blocks, then hold private blocks for their ``suffix_lens`` tokens (one
    entry per sequence, 0 allowed).  ``meta`` records ``cu_group_seqs`` and
    ``group_prefix_lens`` (tokens)."""
    rng = np.random.default_rng(seed)
    group_sizes = [int(x) for x in group_sizes]
    prefix_blocks = [int(x) for x in prefix_blocks]
    suffix_lens = np.asarray(suffix_lens, np.int64)
    S = sum(group_sizes)
    assert len(prefix_blocks) == len(group_sizes) and suffix_lens.shape == (S,)
    lengths = np.zeros(S, np.int32)
    s = 0
    for g, n in enumerate(group_sizes):
        lengths[s:s + n] = prefix_blocks[g] * B + suffix_lens[s:s + n]
        s += n
    need = sum(prefix_blocks) + int(sum(-(-int(x) // B) for x in suffix_lens))
    NB = max(64, 2 * need) if NB is None else NB
    free_order = rng.permutation(NB)
    pos, seq_blocks, block_fill = 0, [], {}

    def take(c):
        nonlocal pos
        r = free_order[pos:pos + c].astype(np.int64)
        pos += c
        return r

    s = 0
    for g, n in enumerate(group_sizes):
        prefix = take(prefix_blocks[g])
        for b in prefix:
            block_fill[int(b)] = B
        for _ in range(n):
            suf = int(suffix_lens[s])
            extra = take(-(-suf // B))
            for k, b in enumerate(extra):
                block_fill[int(b)] = min(B, suf - k * B)
            seq_blocks.append(np.concatenate([prefix, extra]).astype(np.int64))
            s += 1
    cu = np.zeros(len(group_sizes) + 1, np.int32)
    cu[1:] = np.cumsum(group_sizes)
    return _build(name, rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows=S, seq_blocks=seq_blocks,
                  block_fill=block_fill,
                  meta={"cu_group_seqs": cu,
                        "group_prefix_lens": np.array(prefix_blocks, np.int32) * B})


def mixed_batch(seed: int, decode_lens, prefill_prior, prefill_chunks, Hq: int, Hkv: int, D: int,
                B: int, dtype: str, NB: int | None = None, name: str = "mixed") -> PagedBatch:
    """A batch mixing decodes and prefill chunks, decodes first: sequence i <
    len(decode_lens) has one query row over decode_lens[i] cached tokens; the
    others a chunk of prefill_chunks[j] rows after prefill_prior[j] tokens.
    ``meta["num_decode"]`` is the number of decodes."""
    rng = np.random.default_rng(seed)
    dl = np.asarray(decode_lens, np.int32)
    prior = np.asarray(prefill_prior, np.int32)
    chunks = np.asarray(prefill_chunks, np.int32)
    lengths = np.concatenate([dl, prior + chunks]).astype(np.int32)
    chunk_lens = np.concatenate([np.ones(dl.shape[0], np.int32), chunks]).astype(np.int32)
    if NB is None:
        NB = max(64, 2 * int(sum(-(-int(L) // B) for L in lengths)))
    free_order = rng.permutation(NB)
    return _build(name, rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows=int(chunk_lens.sum()),
                  chunk_lens=chunk_lens, free_order=free_order, meta={"num_decode": int(dl.shape[0])})


def llama3_8b_mixed_bf16(seed: int = 0, chunk: int = 512, prior: int = 8192) -> PagedBatch:
    """The Llama-3-8B decode batch (256 sequences, log-normal lengths) plus one
    prefill chunk of ``chunk`` tokens after ``prior`` cached tokens, in one
    batch (decodes first), 12 GB pool."""
    rng = np.random.default_rng(seed)
    lengths = lognormal_lengths(rng, 256)
    return mixed_batch(seed + 1, lengths, [prior], [chunk], 32, 8, 128, 16, "bf16",
                       NB=pool_blocks_for(16, 8, 128, "bf16"), name="llama3_8b_mixed_bf16")


def prefill_bf16(seed: int = 0, S: int = 8, chunk: int = 512, prior_lo: int = 4096,
                 prior_hi: int = 32768, Hq: int = 32, Hkv: int = 8, D: int = 128, B: int = 16,
                 NB: int | None = None) -> PagedBatch:
    """Chunked causal prefill: each sequence has a paged prior context of uniform
    [prior_lo, prior_hi] tokens and a ``chunk``-token query chunk after it."""
    dtype = "bf16"
    rng = np.random.default_rng(seed)
    prior = rng.integers(prior_lo, prior_hi + 1, size=S).astype(np.int32)
    chunks = np.full(S, chunk, np.int32)
    lengths = (prior + chunks).astype(np.int32)
    NB = pool_blocks_for(B, Hkv, D, dtype) if NB is None else NB
    free_order = rng.permutation(NB)
    return _build("prefill_bf16", rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows=int(chunks.sum()),
                  chunk_lens=chunks, free_order=free_order)


def varlen_prefill(seed: int, prior, chunks, Hq: int, Hkv: int, D: int, B: int, dtype: str,
                   NB: int | None = None, name: str = "prefill") -> PagedBatch:
    """Prefill batch with explicit prior-context and chunk lengths per sequence."""
    rng = np.random.default_rng(seed)
    prior = np.asarray(prior, np.int32)
    chunks = np.asarray(chunks, np.int32)
    lengths = (prior + chunks).astype(np.int32)
    if NB is None:
        NB = max(64, 2 * int(sum(-(-int(L) // B) for L in lengths)))
    free_order = rng.permutation(NB)
    return _build(name, rng, lengths, Hq, Hkv, D, B, NB, dtype, q_rows=int(chunks.sum()),
                  chunk_lens=chunks, free_order=free_order)


def strided_chunk_rows(cu_seqlens_q, stride: int) -> np.ndarray:
    """Query rows of a varlen batch to compare: every ``stride``-th row of each
    chunk from its first, plus its last."""
    cu = np.asarray(cu_seqlens_q, np.int64)
    rows = [np.r_[np.arange(a, b, stride), b - 1] for a, b in zip(cu[:-1], cu[1:]) if b > a]
    return np.unique(np.concatenate(rows)) if rows else np.zeros(0, np.int64)


def split_chunks(n_tokens: int, budget: int) -> list[int]:
    """Cut a prompt into prefill chunks of at most ``budget`` tokens, in order."""
    out = []
    while n_tokens > 0:
        out.append(min(budget, n_tokens))
        n_tokens -= out[-1]
    return out


def cu_seqlens(counts) -> np.ndarray:
    """Prefix sums [0, c0, c0+c1, ...] of per-request token counts."""
    out = np.zeros(len(counts) + 1, np.int32)
    out[1:] = np.cumsum(counts)
    return out


# ---------------------------------------------------------------- FP8 (E4M3) pools
FP8_NAN = np.uint8(0x7F)


def _fp8_code_table() -> np.ndarray:
    """Code for each 16-bit random draw u: bit 15 is the sign; t = u & 0x7FFF
    picks the magnitude code -- t < 3328 (about 10%) cycles through all 127
    finite magnitudes (zeros, subnormals and 448 included), the rest spread
    over exponent fields 10..14 with all 8 mantissas (magnitudes 4..240, like
    quantized N(0, 1) / scale data).  No NaN code."""
    u = np.arange(65536, dtype=np.int64)
    t = u & 0x7FFF
    j = t - 3328
    mag = np.where(t < 3328, t % 127, ((10 + (j * 5) // (32768 - 3328)) << 3) | (j % 8))
    return (mag | ((u >> 8) & 0x80)).astype(np.uint8)


_FP8_TABLE = _fp8_code_table()


def fp8_codes(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """Random finite OCP E4M3 codes (table lookup of uniform 16-bit draws,
    chunked over threads like ``_normal``; depends only on ``rng`` and shape)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint8)
    starts = list(range(0, n, chunk)) or [0]
    seeds = rng.integers(0, 2**63 - 1, size=len(starts))

    def fill(i):
        lo = starts[i]
        m = min(chunk, n - lo)
        g = np.random.default_rng(int(seeds[i]))
        out[lo:lo + m] = _FP8_TABLE[g.integers(0, 65536, m, dtype=np.uint16)]

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(len(starts))))
    return out.reshape(shape)


@dataclass
class Fp8Pools:
    """E4M3 contents for a PagedBatch's data blocks (same indexing as
    ``k_blocks`` / ``v_blocks``; stale rows hold the NaN code), the new-token
    rows of this step, and fp32 scales [Hkv]."""
    k_blocks: np.ndarray   # uint8 [n, B, Hkv, D]
    v_blocks: np.ndarray
    new_k: np.ndarray      # uint8 [T, Hkv, D]: the codes already at this step's slots
    new_v: np.ndarray
    k_scale: np.ndarray    # float32 [Hkv]
    v_scale: np.ndarray

    def full_pool(self, batch: "PagedBatch"):
        shape = (batch.NB, batch.B, batch.Hkv, batch.D)
        k = np.full(shape, FP8_NAN, np.uint8)
        v = np.full(shape, FP8_NAN, np.uint8)
        k[batch.block_ids], v[batch.block_ids] = self.k_blocks, self.v_blocks
        return k, v


def fp8_pools(batch: "PagedBatch", seed: int) -> Fp8Pools:
    """FP8 codes for ``batch``'s data blocks: rows the batch marks stale (NaN in
    its 16-bit blocks) stay NaN codes; scales uniform on [0.004, 0.02]."""
    rng = np.random.default_rng(seed)
    shape = batch.k_blocks.shape
    kc = fp8_codes(rng, shape)
    vc = fp8_codes(rng, shape)
    stale = np.isnan(storage_to_f32(batch.k_blocks[:, :, 0, 0], batch.dtype))  # [n, B]
    kc[stale] = FP8_NAN
    vc[stale] = FP8_NAN
    ks = rng.uniform(0.004, 0.02, batch.Hkv).astype(np.float32)
    vs = rng.uniform(0.004, 0.02, batch.Hkv).astype(np.float32)
    where = {int(b): i for i, b in enumerate(batch.block_ids)}
    if batch.new_slots.size:
        idx = np.array([where[int(x)] for x in batch.new_slots // batch.B])
        off = batch.new_slots % batch.B
        nk, nv = kc[idx, off], vc[idx, off]
    else:
        nk = np.zeros((0, batch.Hkv, batch.D), np.uint8)
        nv = nk.copy()
    return Fp8Pools(k_blocks=kc, v_blocks=vc, new_k=nk, new_v=nv, k_scale=ks, v_scale=vs)
