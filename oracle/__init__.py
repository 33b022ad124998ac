"""Reference oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.

The arithmetic lives in ``pkv_oracle.c`` (plain fp64 C); this module only
compiles it on demand and marshals numpy arrays through ctypes.  Each wrapper
names the passage of the pages that the underlying C function follows:

* gather + textbook attention: CS349D lecture 3 notes, sec. 3.2 (block-wise
  attention equals contiguous attention); S06 PagedAttention chapter,
  "implementation" section (pool layout, only written rows of the last block).
* GQA grouping: "LLM inference, part 3: single node", ch. 9 sec. 1.
* causal chunked prefill: same book, ch. 13 sec. 2; CS349D lecture 3 sec. 7.2.
* reshape_and_cache (slot writes): same book, ch. 13 sec. 1 (slot_mapping).
* copy_blocks (copy-on-write): CS349D lecture 3 sec. 3.2 and sec. 4.1.
* swap_blocks (swap-out / swap-in of a preempted sequence): CS349D lecture 3
  sec. 5.2.
* FP8 (OCP E4M3) KV cache -- quantizing reshape_and_cache and decode over
  dequantized values: "LLM inference, part 3: single node", ch. 10 (scale and
  clip on write, scale back on read).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv_oracle.so")
_SRC_PATH = os.path.join(_HERE, "pkv_oracle.c")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}

_lib = None


def build(force: bool = False) -> str:
    """Compile pkv_oracle.c into libpkv_oracle.so (gcc, via the Makefile)."""
    stale = (not os.path.exists(_LIB_PATH)) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH))
    if force or stale:
        subprocess.run(["make", "-s"] + (["-B"] if force else []) + ["-C", _HERE], check=True)
    return _LIB_PATH


def _load(path: str | None = None):
    global _lib
    if _lib is None or path is not None:
        if path is None:
            build()
        lib = ctypes.CDLL(path or _LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl, ci = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        lib.pkvo_load_elem.restype = dbl
        lib.pkvo_load_elem.argtypes = [P, ci, i64]
        lib.pkvo_gather.restype = ci
        lib.pkvo_gather.argtypes = [P, P, ci, P, i32, i64, i32, i32, i32, i32]
        lib.pkvo_attend.restype = ci
        lib.pkvo_attend.argtypes = [P, P, P, P, i32, i32, dbl]
        lib.pkvo_decode.restype = ci
        lib.pkvo_decode.argtypes = [P, P, P, P, ci, P, i32, P, i64, i32, i32, i32, i32, i32, dbl]
        lib.pkvo_prefill_rows.restype = ci
        lib.pkvo_prefill_rows.argtypes = [P, P, P, i32, P, P, ci, P, i32, P, i64, i32, i32, i32,
                                          i32, i32, dbl, P, i32]
        lib.pkvo_reshape_and_cache.restype = ci
        lib.pkvo_reshape_and_cache.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i64, ci]
        lib.pkvo_copy_blocks.restype = ci
        lib.pkvo_copy_blocks.argtypes = [P, P, i32, P, i32, i32, i32, i32, i64, ci]
        lib.pkvo_swap_blocks.restype = ci
        lib.pkvo_swap_blocks.argtypes = [P, P, i32, P, i32, i64, i64, i64]
        lib.pkvo_e4m3_to_f64.restype = dbl
        lib.pkvo_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.pkvo_e4m3_from_f32.restype = ctypes.c_uint8
        lib.pkvo_e4m3_from_f32.argtypes = [ctypes.c_float]
        lib.pkvo_reshape_and_cache_fp8.restype = ci
        lib.pkvo_reshape_and_cache_fp8.argtypes = [P, P, ci, P, P, P, i32, i32, i32, i32, i64, P, P]
        lib.pkvo_decode_fp8.restype = ci
        lib.pkvo_decode_fp8.argtypes = [P, P, ci, P, P, P, P, P, i32, P, i64, i32, i32, i32, i32,
                                        i32, dbl]
        lib.pkvo_prefill_fp8_rows.restype = ci
        lib.pkvo_prefill_fp8_rows.argtypes = [P, P, ci, P, i32, P, P, P, P, P, i32, P, i64, i32, i32,
                                              i32, i32, i32, dbl, P, i32]
        if path is not None:
            return lib
        _lib = lib
    return _lib


class use_library:
    """Context manager: route every wrapper through another build of the oracle
    (used by the pin-strength tests, which compile deliberately broken copies)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _load()
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what}: oracle returned {rc}")


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous, "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype=None) -> np.ndarray:
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of every stored element (elementwise pkvo_load_elem)."""
    lib = _load()
    bits = _c(bits)
    flat = bits.reshape(-1)
    out = np.empty(flat.size, np.float64)
    code = DTYPE_CODE[dtype]
    for i in range(flat.size):
        out[i] = lib.pkvo_load_elem(_ptr(flat), code, i)
    return out.reshape(bits.shape)


def gather(cache: np.ndarray, dtype: str, table: np.ndarray, L: int, kv_head: int) -> np.ndarray:
    """Contiguous [L, D] fp64 rows of one sequence / KV head, read through its table."""
    lib = _load()
    cache = _c(cache)
    NB, B, Hkv, D = cache.shape
    table = _c(table, np.int32)
    out = np.empty((max(L, 1), D), np.float64)
    _check(lib.pkvo_gather(_ptr(out), _ptr(cache), DTYPE_CODE[dtype], _ptr(table), L, NB, Hkv, D,
                           B, kv_head), "gather")
    return out[:L]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook softmax attention of one fp64 query row over contiguous fp64 K/V."""
    lib = _load()
    q, K, V = _c(q, np.float64), _c(K, np.float64), _c(V, np.float64)
    n, D = K.shape if K.size else (0, q.shape[0])
    out = np.empty(D, np.float64)
    Kp = K if K.size else np.zeros((1, D))
    Vp = V if V.size else np.zeros((1, D))
    _check(lib.pkvo_attend(_ptr(out), _ptr(q), _ptr(Kp), _ptr(Vp), n, D, scale), "attend")
    return out


def decode(q, k_cache, v_cache, dtype: str, block_tables, context_lens, scale: float,
           num_kv_heads: int | None = None) -> np.ndarray:
    """fp64 decode output [S, Hq, D]: each sequence's single query over its context."""
    lib = _load()
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    S, Hq, D = q.shape
    NB, B, Hkv, Dk = k_cache.shape
    assert Dk == D and v_cache.shape == k_cache.shape
    assert num_kv_heads in (None, Hkv)
    if block_tables.ndim == 1:
        block_tables = block_tables.reshape(S, -1)
    max_nb = block_tables.shape[1] if block_tables.size else 0
    bt = block_tables if block_tables.size else np.zeros((max(S, 1), 1), np.int32)
    out = np.zeros((S, Hq, D), np.float64)
    _check(lib.pkvo_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), DTYPE_CODE[dtype],
                           _ptr(bt), max_nb, _ptr(context_lens), NB, S, Hq, Hkv, D, B, scale),
           "decode")
    return out


def prefill(q, cu_seqlens_q, k_cache, v_cache, dtype: str, block_tables, context_lens,
            scale: float, rows=None) -> np.ndarray:
    """fp64 causal prefill output [Tq, Hq, D]; with ``rows`` only those query
    tokens are computed (the rest stay NaN)."""
    lib = _load()
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    cu = _c(cu_seqlens_q, np.int32)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    Tq, Hq, D = q.shape
    S = cu.shape[0] - 1
    NB, B, Hkv, _ = k_cache.shape
    max_nb = block_tables.shape[1]
    out = np.full((Tq, Hq, D), np.nan, np.float64)
    if rows is None:
        rp, nr = None, 0
    else:
        rows = _c(rows, np.int32)
        rp, nr = _ptr(rows), rows.shape[0]
    _check(lib.pkvo_prefill_rows(_ptr(out), _ptr(q), _ptr(cu), Tq, _ptr(k_cache), _ptr(v_cache),
                                 DTYPE_CODE[dtype], _ptr(block_tables), max_nb, _ptr(context_lens),
                                 NB, S, Hq, Hkv, D, B, scale, rp, nr), "prefill")
    return out


def prefill_fp8(q, q_dtype: str, cu_seqlens_q, k_cache, v_cache, k_scale, v_scale, block_tables,
                context_lens, scale: float, rows=None) -> np.ndarray:
    """fp64 causal prefill output [Tq, Hq, D] over FP8 pools read as code * scale;
    with ``rows`` only those query tokens are computed (the rest stay NaN)."""
    lib = _load()
    q, k_cache, v_cache = _c(q), _c(k_cache, np.uint8), _c(v_cache, np.uint8)
    k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
    cu = _c(cu_seqlens_q, np.int32)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    Tq, Hq, D = q.shape
    S = cu.shape[0] - 1
    NB, B, Hkv, Dk = k_cache.shape
    assert Dk == D and v_cache.shape == k_cache.shape
    assert k_scale.shape == (Hkv,) and v_scale.shape == (Hkv,)
    max_nb = block_tables.shape[1]
    out = np.full((Tq, Hq, D), np.nan, np.float64)
    if rows is None:
        rp, nr = None, 0
    else:
        rows = _c(rows, np.int32)
        rp, nr = _ptr(rows), rows.shape[0]
    _check(lib.pkvo_prefill_fp8_rows(_ptr(out), _ptr(q), DTYPE_CODE[q_dtype], _ptr(cu), Tq,
                                     _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                     _ptr(block_tables), max_nb, _ptr(context_lens), NB, S, Hq, Hkv,
                                     D, B, scale, rp, nr), "prefill_fp8")
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, dtype: str) -> None:
    """In place: write each token's K/V row into its slot (negative slot = skip)."""
    lib = _load()
    key, value = _c(key), _c(value)
    slot_mapping = _c(slot_mapping, np.int64)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    NB, B, Hkv, D = k_cache.shape
    T = key.shape[0]
    _check(lib.pkvo_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(slot_mapping), T, Hkv, D, B, NB, DTYPE_CODE[dtype]),
           "reshape_and_cache")


def copy_blocks(k_caches, v_caches, pairs, dtype: str) -> None:
    """In place: for every layer, block dst := block src (K and V) for each pair."""
    lib = _load()
    pairs = _c(pairs, np.int64).reshape(-1, 2)
    L = len(k_caches)
    for a in list(k_caches) + list(v_caches):
        assert a.flags.c_contiguous
    NB, B, Hkv, D = k_caches[0].shape
    kp = (ctypes.c_void_p * max(L, 1))(*[a.ctypes.data for a in k_caches])
    vp = (ctypes.c_void_p * max(L, 1))(*[a.ctypes.data for a in v_caches])
    _check(lib.pkvo_copy_blocks(ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
                                L, _ptr(pairs) if pairs.size else 0, pairs.shape[0], B, Hkv, D, NB,
                                DTYPE_CODE[dtype]), "copy_blocks")


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact fp64 value of every OCP E4M3 code (uint8 array)."""
    lib = _load()
    codes = _c(codes, np.uint8)
    flat = codes.reshape(-1)
    out = np.array([lib.pkvo_e4m3_to_f64(int(c)) for c in flat], np.float64)
    return out.reshape(codes.shape)


def e4m3_from_f32(x) -> np.ndarray:
    """OCP E4M3 code of every fp32 value: nearest finite value, ties to even."""
    lib = _load()
    x = _c(x, np.float32)
    flat = x.reshape(-1)
    out = np.array([lib.pkvo_e4m3_from_f32(float(v)) for v in flat], np.uint8)
    return out.reshape(x.shape)


def reshape_and_cache_fp8(key, value, in_dtype: str, k_cache, v_cache, slot_mapping, k_scale,
                          v_scale) -> None:
    """In place: quantize each token's K/V row (code = e4m3(fp32(x) / scale of
    its KV head)) into its slot of the uint8 pools (negative slot = skip)."""
    lib = _load()
    key, value = _c(key), _c(value)
    slot_mapping = _c(slot_mapping, np.int64)
    k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
    assert k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    NB, B, Hkv, D = k_cache.shape
    assert k_scale.shape == (Hkv,) and v_scale.shape == (Hkv,)
    T = key.shape[0]
    _check(lib.pkvo_reshape_and_cache_fp8(_ptr(key), _ptr(value), DTYPE_CODE[in_dtype],
                                          _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv,
                                          D, B, NB, _ptr(k_scale), _ptr(v_scale)),
           "reshape_and_cache_fp8")


def decode_fp8(q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
               scale: float) -> np.ndarray:
    """fp64 decode output [S, Hq, D] over an FP8 pool read as code * scale."""
    lib = _load()
    q, k_cache, v_cache = _c(q), _c(k_cache, np.uint8), _c(v_cache, np.uint8)
    k_scale, v_scale = _c(k_scale, np.float32), _c(v_scale, np.float32)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    S, Hq, D = q.shape
    NB, B, Hkv, Dk = k_cache.shape
    assert Dk == D and v_cache.shape == k_cache.shape
    assert k_scale.shape == (Hkv,) and v_scale.shape == (Hkv,)
    max_nb = block_tables.shape[1] if block_tables.size else 0
    bt = block_tables if block_tables.size else np.zeros((max(S, 1), 1), np.int32)
    out = np.zeros((S, Hq, D), np.float64)
    _check(lib.pkvo_decode_fp8(_ptr(out), _ptr(q), DTYPE_CODE[q_dtype], _ptr(k_cache),
                               _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(bt), max_nb,
                               _ptr(context_lens), NB, S, Hq, Hkv, D, B, scale), "decode_fp8")
    return out


def swap_blocks(src_pools, dst_pools, pairs) -> None:
    """In place: for every pool index p, dst_pools[p][dst] := src_pools[p][src]
    for each (src, dst) pair (whole blocks, any dtype)."""
    lib = _load()
    pairs = _c(pairs, np.int64).reshape(-1, 2)
    n = len(src_pools)
    assert len(dst_pools) == n
    for a in list(src_pools) + list(dst_pools):
        assert a.flags.c_contiguous
    if n == 0:
        return
    block_bytes = src_pools[0][0].nbytes
    sp = (ctypes.c_void_p * n)(*[a.ctypes.data for a in src_pools])
    dp = (ctypes.c_void_p * n)(*[a.ctypes.data for a in dst_pools])
    _check(lib.pkvo_swap_blocks(ctypes.cast(sp, ctypes.c_void_p), ctypes.cast(dp, ctypes.c_void_p),
                                n, _ptr(pairs) if pairs.size else 0, pairs.shape[0], block_bytes,
                                src_pools[0].shape[0], dst_pools[0].shape[0]), "swap_blocks")
