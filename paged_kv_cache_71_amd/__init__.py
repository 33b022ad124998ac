"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libpkv.so`` behind the C ABI declared in
``include/pkv.h``; this package is its thin Python binding (argument
marshalling only) plus the seeded workload generators used by the tests and the
benchmark.  Loading is lazy: ``load_library()`` (or the first call) loads the
library and raises if it has not been built.
"""
from ._binding import (BlockManager, PkvError, PkvOOM, copy_blocks, declared_symbols,
                       decode_cascade_workspace_size, decode_step, decode_workspace_size,
                       load_library,
                       mixed_workspace_size, paged_attention_decode,
                       paged_attention_decode_cascade, paged_attention_decode_cascade_fp8,
                       paged_attention_decode_fp8, paged_attention_decode_noalloc, paged_attention_mixed, paged_attention_mixed_fp8,
                       paged_attention_prefill,
                       paged_attention_prefill_fp8, prefill_workspace_size,
                       reshape_and_cache, reshape_and_cache_fp8, swap_blocks)

__all__ = [
    "BlockManager", "PkvError", "PkvOOM", "copy_blocks", "declared_symbols",
    "decode_cascade_workspace_size", "decode_step", "decode_workspace_size", "load_library",
    "mixed_workspace_size", "paged_attention_decode", "paged_attention_decode_cascade",
    "paged_attention_decode_cascade_fp8", "paged_attention_decode_fp8",
    "paged_attention_decode_noalloc", "paged_attention_mixed",
    "paged_attention_mixed_fp8", "paged_attention_prefill",
    "paged_attention_prefill_fp8",
    "prefill_workspace_size", "reshape_and_cache", "reshape_and_cache_fp8", "swap_blocks",
]
