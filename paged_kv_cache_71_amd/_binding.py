"""ctypes binding of libpkv.so: argument marshalling only.

Every computation runs in the library's HIP kernels; torch is used for device
memory and the current stream.  The library must be built
(``python -m paged_kv_cache_71_amd.build``); if it is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pkv.h")

PKV_OK = 0
STATUS = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARG", 2: "PKV_ERR_UNSUPPORTED", 3: "PKV_ERR_WORKSPACE",
          4: "PKV_ERR_OOM", 5: "PKV_ERR_HIP"}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{where}: {self.name}: {detail}")


class PkvOOM(PkvError):
    pass


_lib = None


def load_library(path: str | None = None):
    """Load libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_71_amd.build`")
    # torch first: its bundled HIP runtime must be the one the library binds
    # to (loaded the other way round, the process ends up with two runtimes
    # and the library cannot see torch's device state)
    _torch()
    lib = ctypes.CDLL(path)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                           ctypes.c_size_t)
    I32P, I64P, SZP = (ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                       ctypes.POINTER(ctypes.c_size_t))
    st = ctypes.c_int
    sig = {
        "pkv_status_string": (ctypes.c_char_p, [st]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_version": (ctypes.c_char_p, []),
        "pkv_reshape_and_cache": (st, [P, P, P, P, P, i32, i32, i32, i32, i64, st, P]),
        "pkv_decode_workspace_size": (st, [i32, i32, i32, i32, i32, i32, SZP]),
        "pkv_paged_attention_decode": (st, [P, st, P, P, P, st, P, i32, P, i32, i32, i32, i32, i32,
                                            i32, f32, P, sz, P]),
        "pkv_paged_attention_decode_noalloc": (st, [P, st, P, P, P, st, P, i32, P, i32, i32, i32,
                                                    i32, i32, i32, f32, P]),
        "pkv_decode_step": (st, [P, st, P, P, P, P, P, P, i64, st, P, i32, P, i32, i32, i32, i32,
                                 i32, i32, f32, P, sz, P]),
        "pkv_prefill_workspace_size": (st, [i32, i32, i32, i32, i32, i32, i32, st, i32, SZP]),
        "pkv_paged_attention_prefill": (st, [P, st, P, P, i32, i32, P, P, st, P, i32, P, i32, i32,
                                             i32, i32, i32, i32, f32, P, sz, P]),
        "pkv_copy_blocks": (st, [P, P, i32, P, i32, i32, i32, i32, st, P]),
        "pkv_swap_blocks": (st, [P, P, i32, P, i32, i32, i32, i32, st, P]),
        "pkv_bm_set_cpu_blocks": (st, [P, i32]),
        "pkv_bm_num_free_cpu": (st, [P, I32P]),
        "pkv_bm_swap_out": (st, [P, i32, P, i32, I32P]),
        "pkv_bm_swap_in": (st, [P, i32, P, i32, I32P]),
        "pkv_reshape_and_cache_fp8": (st, [P, P, st, P, P, P, i32, i32, i32, i32, i64, P, P, P]),
        "pkv_mixed_workspace_size": (st, [i32, i32, i32, i32, i32, i32, i32, i32, st, i32, SZP]),
        "pkv_paged_attention_mixed": (st, [P, st, P, P, i32, i32, i32, P, P, st, P, i32, P, i32, i32,
                                           i32, i32, i32, i32, f32, P, sz, P]),
        "pkv_decode_cascade_workspace_size": (st, [i32, i32, i32, i32, i32, i32, i32, i32, i32, st,
                                                   SZP]),
        "pkv_paged_attention_decode_cascade": (st, [P, st, P, P, P, st, P, i32, P, i32, i32, i32,
                                                    i32, i32, i32, f32, P, P, i32, i32, i32, P, sz,
                                                    P]),
        "pkv_paged_attention_decode_cascade_fp8": (st, [P, st, P, st, P, P, P, P, P, i32, P, i32,
                                                        i32, i32, i32, i32, i32, f32, P, P, i32,
                                                        i32, i32, P, sz, P]),
        "pkv_paged_attention_mixed_fp8": (st, [P, st, P, st, P, i32, i32, i32, P, P, P, P, P, i32,
                                               P, i32, i32, i32, i32, i32, i32, f32, P, sz, P]),
        "pkv_paged_attention_decode_fp8": (st, [P, st, P, st, P, P, P, P, P, i32, P, i32, i32, i32,
                                                i32, i32, i32, f32, P, sz, P]),
        "pkv_paged_attention_prefill_fp8": (st, [P, st, P, st, P, i32, i32, P, P, P, P, P, i32, P,
                                                 i32, i32, i32, i32, i32, i32, f32, P, sz, P]),
        "pkv_bm_create": (st, [i32, i32, P, ctypes.POINTER(P)]),
        "pkv_bm_destroy": (None, [P]),
        "pkv_bm_add_seq": (st, [P, i32, I32P]),
        "pkv_bm_append_token": (st, [P, i32, I64P, I32P, I32P]),
        "pkv_bm_fork": (st, [P, i32, I32P]),
        "pkv_bm_free_seq": (st, [P, i32]),
        "pkv_bm_table": (st, [P, i32, P, i32, I32P]),
        "pkv_bm_seq_len": (st, [P, i32, I32P]),
        "pkv_bm_slots": (st, [P, i32, i32, i32, P]),
        "pkv_bm_refcount": (st, [P, i32, I32P]),
        "pkv_bm_num_free": (st, [P, I32P]),
        "pkv_bm_check": (st, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def declared_symbols(header: str = HEADER) -> list[str]:
    """Names of the functions include/pkv.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def _check(rc: int, where: str) -> None:
    if rc != PKV_OK:
        detail = _lib.pkv_last_error().decode()
        raise (PkvOOM if rc == 4 else PkvError)(rc, where, detail)


# ---------------------------------------------------------------- tensor helpers
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    """Library dtype of a tensor; uint8 and float8_e4m3fn tensors are FP8 (E4M3) pools."""
    torch = _torch()
    m = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.uint8: 3,
         torch.float8_e4m3fn: 3}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ---------------------------------------------------------------- kernels
def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write each new token's K/V row ([T, Hkv, D]) into its slot of the pools."""
    torch = _torch()
    lib = load_library()
    T, Hkv, D = key.shape
    NB, B, Hkv2, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("reshape_and_cache: shape mismatch")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("reshape_and_cache: dtype mismatch")
    if slot_mapping.shape != (T,):
        raise ValueError("reshape_and_cache: slot_mapping must be [T]")
    _check(lib.pkv_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(slot_mapping, "slot_mapping", torch.int64), T, Hkv, D, B, NB, dtype_code(key),
        _stream(stream)), "reshape_and_cache")


def decode_workspace_size(S: int, Hq: int, Hkv: int, D: int, B: int, max_context_len: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.pkv_decode_workspace_size(S, Hq, Hkv, D, B, max_context_len, ctypes.byref(out)),
           "decode_workspace_size")
    return out.value


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                           max_context_len: int, scale: float, workspace=None, stream=None):
    """Decode attention: out[s, h] = softmax(scale q[s,h] K_s^T) V_s over each
    sequence's paged context.  ``workspace`` (uint8 device tensor) is allocated
    here if not given."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_decode: shape mismatch")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("paged_attention_decode: q/k/v dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_decode: block_tables [S, max_nb] / context_lens [S]")
    need = decode_workspace_size(S, Hq, Hkv, D, B, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_decode(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), dtype_code(k_cache),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), ws_ptr, ws_bytes, _stream(stream)), "paged_attention_decode")
    return out


def decode_step(out, q, key, value, slot_mapping, k_cache, v_cache, block_tables, context_lens,
                max_context_len: int, scale: float, workspace=None, stream=None):
    """One decode step: the new tokens' K/V rows (``key``/``value`` [S, Hkv, D],
    token context_lens[s] - 1 of each sequence) are written to their slots and
    attended, as reshape_and_cache followed by paged_attention_decode.
    ``workspace`` (uint8 device tensor) is allocated here if not given."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("decode_step: shape mismatch")
    if key.shape != (S, Hkv, D) or value.shape != key.shape or slot_mapping.shape != (S,):
        raise ValueError("decode_step: key/value must be [S, Hkv, D], slot_mapping [S]")
    if not (q.dtype == key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("decode_step: q/key/value/pool dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("decode_step: block_tables [S, max_nb] / context_lens [S]")
    need = decode_workspace_size(S, Hq, Hkv, D, B, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_decode_step(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), _dev(key, "key"), _dev(value, "value"),
        _dev(slot_mapping, "slot_mapping", torch.int64), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), NB, dtype_code(k_cache),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), ws_ptr, ws_bytes, _stream(stream)), "decode_step")
    return out


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens,
                                   max_context_len: int, scale: float, stream=None):
    """Decode attention like paged_attention_decode, with the partial states in
    the library's static device scratch instead of a workspace: nothing is
    allocated.  Calls that overlap on one device race on that scratch."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_decode_noalloc: shape mismatch")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("paged_attention_decode_noalloc: q/k/v dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_decode_noalloc: block_tables [S, max_nb] / context_lens [S]")
    _check(lib.pkv_paged_attention_decode_noalloc(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), dtype_code(k_cache),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), _stream(stream)), "paged_attention_decode_noalloc")
    return out


def prefill_workspace_size(S: int, Tq: int, max_query_len: int, Hq: int, Hkv: int, D: int, B: int,
                           dtype: str, max_context_len: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.pkv_prefill_workspace_size(S, Tq, max_query_len, Hq, Hkv, D, B, DTYPE_CODE[dtype],
                                          max_context_len, ctypes.byref(out)), "prefill_workspace_size")
    return out.value


def paged_attention_prefill(out, q, cu_seqlens_q, max_query_len: int, k_cache, v_cache,
                            block_tables, context_lens, max_context_len: int, scale: float,
                            workspace=None, stream=None):
    """Causal attention of each sequence's query chunk over its paged context.
    ``workspace`` (uint8 device tensor) is allocated here if the call needs one
    and none is given."""
    torch = _torch()
    lib = load_library()
    Tq, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    S = cu_seqlens_q.shape[0] - 1
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_prefill: shape mismatch")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("paged_attention_prefill: q/k/v dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_prefill: block_tables [S, max_nb] / context_lens [S]")
    kv_code = dtype_code(k_cache)
    need = ctypes.c_size_t(0)
    _check(lib.pkv_prefill_workspace_size(S, Tq, int(max_query_len), Hq, Hkv, D, B, kv_code,
                                          int(max_context_len), ctypes.byref(need)), "prefill_workspace_size")
    if workspace is None and need.value:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_prefill(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), Tq, int(max_query_len),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), kv_code,
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), ws_ptr, ws_bytes, _stream(stream)), "paged_attention_prefill")
    return out


def mixed_workspace_size(S: int, num_decode: int, Tq: int, max_query_len: int, Hq: int, Hkv: int,
                         D: int, B: int, dtype: str, max_context_len: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.pkv_mixed_workspace_size(S, num_decode, Tq, max_query_len, Hq, Hkv, D, B,
                                        DTYPE_CODE[dtype], max_context_len, ctypes.byref(out)),
           "mixed_workspace_size")
    return out.value


def paged_attention_mixed(out, q, cu_seqlens_q, num_decode: int, max_query_len: int, k_cache,
                          v_cache, block_tables, context_lens, max_context_len: int, scale: float,
                          workspace=None, stream=None):
    """One call for a batch whose first ``num_decode`` sequences are decodes
    (one query row each) and the rest prefill chunks.  Same rows as
    paged_attention_decode / _prefill, bit for bit."""
    torch = _torch()
    lib = load_library()
    Tq, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    S = cu_seqlens_q.shape[0] - 1
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_mixed: shape mismatch")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("paged_attention_mixed: q/k/v dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_mixed: block_tables [S, max_nb] / context_lens [S]")
    need = ctypes.c_size_t(0)
    _check(lib.pkv_mixed_workspace_size(S, int(num_decode), Tq, int(max_query_len), Hq, Hkv, D, B,
                                        dtype_code(k_cache), int(max_context_len), ctypes.byref(need)),
           "mixed_workspace_size")
    need = need.value
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.pkv_paged_attention_mixed(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), Tq, int(num_decode), int(max_query_len),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), dtype_code(k_cache),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), _dev(workspace, "workspace"), workspace.numel(), _stream(stream)),
        "paged_attention_mixed")
    return out


def copy_blocks(k_caches, v_caches, block_pairs, stream=None) -> None:
    """For every layer: block dst := block src (K and V pools) for each (src, dst) pair."""
    torch = _torch()
    lib = load_library()
    if len(k_caches) != len(v_caches):
        raise ValueError("copy_blocks: need as many V pools as K pools")
    L = len(k_caches)
    N = block_pairs.shape[0] if block_pairs.dim() == 2 else 0
    if block_pairs.numel() and (block_pairs.dim() != 2 or block_pairs.shape[1] != 2):
        raise ValueError("copy_blocks: block_pairs must be [N, 2]")
    if L == 0:
        return
    NB, B, Hkv, D = k_caches[0].shape
    for t in list(k_caches) + list(v_caches):
        if t.shape != k_caches[0].shape or t.dtype != k_caches[0].dtype:
            raise ValueError("copy_blocks: every pool must have the same shape and dtype")
    kp = (ctypes.c_void_p * L)(*[_dev(t, "k_cache") for t in k_caches])
    vp = (ctypes.c_void_p * L)(*[_dev(t, "v_cache") for t in v_caches])
    pairs_ptr = _dev(block_pairs, "block_pairs", torch.int64) if N else None
    _check(lib.pkv_copy_blocks(ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p),
                               L, pairs_ptr, N, B, Hkv, D, dtype_code(k_caches[0]),
                               _stream(stream)), "copy_blocks")


def decode_cascade_workspace_size(S: int, Hq: int, Hkv: int, D: int, B: int, max_context_len: int,
                                  n_groups: int, max_group_size: int, max_prefix_len: int,
                                  dtype: str) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.pkv_decode_cascade_workspace_size(S, Hq, Hkv, D, B, max_context_len, n_groups,
                                                 max_group_size, max_prefix_len, DTYPE_CODE[dtype],
                                                 ctypes.byref(out)), "decode_cascade_workspace_size")
    return out.value


def paged_attention_decode_cascade(out, q, k_cache, v_cache, block_tables, context_lens,
                                   max_context_len: int, scale: float, cu_group_seqs,
                                   group_prefix_lens, max_group_size: int, max_prefix_len: int,
                                   workspace=None, stream=None):
    """Decode for consecutive groups of sequences sharing a prefix of blocks
    (``cu_group_seqs`` [n_groups + 1], ``group_prefix_lens`` [n_groups], device
    int32): each group's prefix is read once and merged with every member's
    suffix.  Same result as paged_attention_decode up to fp32 rounding."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_decode_cascade: shape mismatch")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("paged_attention_decode_cascade: q/k/v dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_decode_cascade: block_tables [S, max_nb] / context_lens [S]")
    n_groups = cu_group_seqs.shape[0] - 1
    if group_prefix_lens.shape != (n_groups,):
        raise ValueError("paged_attention_decode_cascade: group_prefix_lens must be [n_groups]")
    kdt = {0: "f32", 1: "f16", 2: "bf16"}[dtype_code(k_cache)]
    need = decode_cascade_workspace_size(S, Hq, Hkv, D, B, max_context_len, n_groups,
                                         max_group_size, max_prefix_len, kdt)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_decode_cascade(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), dtype_code(k_cache),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), _dev(cu_group_seqs, "cu_group_seqs", torch.int32),
        _dev(group_prefix_lens, "group_prefix_lens", torch.int32), n_groups, int(max_group_size),
        int(max_prefix_len), ws_ptr, ws_bytes, _stream(stream)), "paged_attention_decode_cascade")
    return out


def paged_attention_decode_cascade_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                       context_lens, max_context_len: int, scale: float,
                                       cu_group_seqs, group_prefix_lens, max_group_size: int,
                                       max_prefix_len: int, workspace=None, stream=None):
    """paged_attention_decode_cascade over FP8 pools read as code * scale of
    the KV head; q is f16 or bf16."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_decode_cascade_fp8: shape mismatch")
    if k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("paged_attention_decode_cascade_fp8: scales must be [Hkv]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_decode_cascade_fp8: block_tables [S, max_nb] / context_lens [S]")
    n_groups = cu_group_seqs.shape[0] - 1
    if group_prefix_lens.shape != (n_groups,):
        raise ValueError("paged_attention_decode_cascade_fp8: group_prefix_lens must be [n_groups]")
    qdt = {1: "f16", 2: "bf16"}.get(dtype_code(q))
    if qdt is None:
        raise TypeError("paged_attention_decode_cascade_fp8: q must be f16 or bf16")
    need = decode_cascade_workspace_size(S, Hq, Hkv, D, B, max_context_len, n_groups,
                                         max_group_size, max_prefix_len, qdt)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_decode_cascade_fp8(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), dtype_code(q),
        _fp8_pool(k_cache, "k_cache"), _fp8_pool(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), _dev(cu_group_seqs, "cu_group_seqs", torch.int32),
        _dev(group_prefix_lens, "group_prefix_lens", torch.int32), n_groups, int(max_group_size),
        int(max_prefix_len), ws_ptr, ws_bytes, _stream(stream)), "paged_attention_decode_cascade_fp8")
    return out


def paged_attention_mixed_fp8(out, q, cu_seqlens_q, num_decode: int, max_query_len: int, k_cache,
                              v_cache, k_scale, v_scale, block_tables, context_lens,
                              max_context_len: int, scale: float, workspace=None, stream=None):
    """paged_attention_mixed over FP8 pools read as code * scale of the KV
    head; q is f16 or bf16.  Same rows as paged_attention_decode_fp8 /
    paged_attention_prefill_fp8, bit for bit."""
    torch = _torch()
    lib = load_library()
    Tq, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    S = cu_seqlens_q.shape[0] - 1
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_mixed_fp8: shape mismatch")
    if k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("paged_attention_mixed_fp8: scales must be [Hkv]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_mixed_fp8: block_tables [S, max_nb] / context_lens [S]")
    need = mixed_workspace_size(S, int(num_decode), Tq, int(max_query_len), Hq, Hkv, D, B, "fp8",
                                int(max_context_len))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.pkv_paged_attention_mixed_fp8(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), dtype_code(q),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), Tq, int(num_decode), int(max_query_len),
        _fp8_pool(k_cache, "k_cache"), _fp8_pool(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), _dev(workspace, "workspace"), workspace.numel(), _stream(stream)),
        "paged_attention_mixed_fp8")
    return out


def _fp8_pool(t, name):
    if dtype_code(t) != 3:
        raise TypeError(f"{name} must be an FP8 pool (uint8 or float8_e4m3fn), got {t.dtype}")
    return _dev(t, name)


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale,
                          stream=None) -> None:
    """Quantize each new token's K/V row ([T, Hkv, D], f32/f16/bf16) into its
    slot of the FP8 pools: code = e4m3(x / scale of the row's KV head)."""
    torch = _torch()
    lib = load_library()
    T, Hkv, D = key.shape
    NB, B, Hkv2, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or value.shape != key.shape or v_cache.shape != k_cache.shape:
        raise ValueError("reshape_and_cache_fp8: shape mismatch")
    if key.dtype != value.dtype:
        raise TypeError("reshape_and_cache_fp8: key/value dtype mismatch")
    if slot_mapping.shape != (T,) or k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("reshape_and_cache_fp8: slot_mapping [T], scales [Hkv]")
    _check(lib.pkv_reshape_and_cache_fp8(
        _dev(key, "key"), _dev(value, "value"), dtype_code(key), _fp8_pool(k_cache, "k_cache"),
        _fp8_pool(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping", torch.int64), T, Hkv, D,
        B, NB, _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _stream(stream)), "reshape_and_cache_fp8")


def paged_attention_decode_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                               context_lens, max_context_len: int, scale: float, workspace=None,
                               stream=None):
    """Decode attention over FP8 pools read as code * scale of the KV head; q
    is f16 or bf16.  ``workspace`` as for paged_attention_decode."""
    torch = _torch()
    lib = load_library()
    S, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_decode_fp8: shape mismatch")
    if k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("paged_attention_decode_fp8: scales must be [Hkv]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_decode_fp8: block_tables [S, max_nb] / context_lens [S]")
    need = decode_workspace_size(S, Hq, Hkv, D, B, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_decode_fp8(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), dtype_code(q),
        _fp8_pool(k_cache, "k_cache"), _fp8_pool(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), ws_ptr, ws_bytes, _stream(stream)), "paged_attention_decode_fp8")
    return out


def paged_attention_prefill_fp8(out, q, cu_seqlens_q, max_query_len: int, k_cache, v_cache, k_scale,
                                v_scale, block_tables, context_lens, max_context_len: int,
                                scale: float, workspace=None, stream=None):
    """Causal chunk attention over FP8 pools read as code * scale of the KV
    head; q is f16 or bf16.  ``workspace`` as for paged_attention_prefill."""
    torch = _torch()
    lib = load_library()
    Tq, Hq, D = q.shape
    NB, B, Hkv, D2 = k_cache.shape
    S = cu_seqlens_q.shape[0] - 1
    if D2 != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("paged_attention_prefill_fp8: shape mismatch")
    if k_scale.shape != (Hkv,) or v_scale.shape != (Hkv,):
        raise ValueError("paged_attention_prefill_fp8: scales must be [Hkv]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("paged_attention_prefill_fp8: block_tables [S, max_nb] / context_lens [S]")
    need = prefill_workspace_size(S, Tq, int(max_query_len), Hq, Hkv, D, B, "fp8", int(max_context_len))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pkv_paged_attention_prefill_fp8(
        _dev(out, "out"), dtype_code(out), _dev(q, "q"), dtype_code(q),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), Tq, int(max_query_len),
        _fp8_pool(k_cache, "k_cache"), _fp8_pool(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), int(max_context_len), S, Hq, Hkv, D, B,
        float(scale), ws_ptr, ws_bytes, _stream(stream)), "paged_attention_prefill_fp8")
    return out


def swap_blocks(src_pools, dst_pools, block_pairs, stream=None) -> None:
    """For every pool index p: dst_pools[p][dst] := src_pools[p][src] for each
    (src, dst) pair.  Each pool is a device tensor or a pinned host tensor
    (``pin_memory``); block_pairs [N, 2] int64 on the device or pinned host."""
    torch = _torch()
    lib = load_library()
    if len(src_pools) != len(dst_pools):
        raise ValueError("swap_blocks: as many destination pools as source pools")
    n = len(src_pools)
    N = block_pairs.shape[0] if block_pairs.dim() == 2 else 0
    if block_pairs.numel() and (block_pairs.dim() != 2 or block_pairs.shape[1] != 2):
        raise ValueError("swap_blocks: block_pairs must be [N, 2]")
    if n == 0 or N == 0:
        return
    _, B, Hkv, D = src_pools[0].shape
    for t in list(src_pools) + list(dst_pools):
        if tuple(t.shape[1:]) != (B, Hkv, D) or t.dtype != src_pools[0].dtype:
            raise ValueError("swap_blocks: every pool must be [NB, B, Hkv, D] of one dtype")
        if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError("swap_blocks: pools must be contiguous device or pinned host tensors")
    if block_pairs.dtype != torch.int64 or not block_pairs.is_contiguous() or not (
            block_pairs.is_cuda or block_pairs.is_pinned()):
        raise ValueError("swap_blocks: block_pairs must be contiguous int64, device or pinned")
    sp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in src_pools])
    dp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst_pools])
    _check(lib.pkv_swap_blocks(ctypes.cast(sp, ctypes.c_void_p), ctypes.cast(dp, ctypes.c_void_p), n,
                               block_pairs.data_ptr(), N, B, Hkv, D, dtype_code(src_pools[0]),
                               _stream(stream)), "swap_blocks")


# ---------------------------------------------------------------- host block manager
class BlockManager:
    """Host block manager (free list, tables, refcounts, copy-on-write)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        lib = load_library()
        self._lib = lib
        self.block_size = block_size
        h = ctypes.c_void_p()
        arr = None
        if free_order is not None:
            arr = np.ascontiguousarray(free_order, np.int32)
            if arr.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        _check(lib.pkv_bm_create(num_blocks, block_size, arr.ctypes.data if arr is not None else None,
                                 ctypes.byref(h)), "bm_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    def add_seq(self, n_tokens: int) -> int:
        sid = ctypes.c_int32()
        _check(self._lib.pkv_bm_add_seq(self._h, n_tokens, ctypes.byref(sid)), "bm_add_seq")
        return sid.value

    def append_token(self, seq: int):
        """Returns (slot, cow) where cow is (src, dst) or None."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pkv_bm_append_token(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                             ctypes.byref(dst)), "bm_append_token")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def fork(self, seq: int) -> int:
        child = ctypes.c_int32()
        _check(self._lib.pkv_bm_fork(self._h, seq, ctypes.byref(child)), "bm_fork")
        return child.value

    def free_seq(self, seq: int) -> None:
        _check(self._lib.pkv_bm_free_seq(self._h, seq), "bm_free_seq")

    def seq_len(self, seq: int) -> int:
        n = ctypes.c_int32()
        _check(self._lib.pkv_bm_seq_len(self._h, seq, ctypes.byref(n)), "bm_seq_len")
        return n.value

    def table(self, seq: int) -> list[int]:
        n = ctypes.c_int32()
        cap = (self.seq_len(seq) + self.block_size - 1) // self.block_size
        buf = np.zeros(max(cap, 1), np.int32)
        _check(self._lib.pkv_bm_table(self._h, seq, buf.ctypes.data, buf.shape[0], ctypes.byref(n)),
               "bm_table")
        return buf[:n.value].tolist()

    def slots(self, seq: int, start: int, count: int) -> np.ndarray:
        out = np.zeros(max(count, 1), np.int64)
        _check(self._lib.pkv_bm_slots(self._h, seq, start, count, out.ctypes.data), "bm_slots")
        return out[:count]

    def refcount(self, block: int) -> int:
        n = ctypes.c_int32()
        _check(self._lib.pkv_bm_refcount(self._h, block, ctypes.byref(n)), "bm_refcount")
        return n.value

    def num_free(self) -> int:
        n = ctypes.c_int32()
        _check(self._lib.pkv_bm_num_free(self._h, ctypes.byref(n)), "bm_num_free")
        return n.value

    def check(self) -> None:
        _check(self._lib.pkv_bm_check(self._h), "bm_check")

    def set_cpu_blocks(self, n: int) -> None:
        _check(self._lib.pkv_bm_set_cpu_blocks(self._h, n), "bm_set_cpu_blocks")

    def num_free_cpu(self) -> int:
        n = ctypes.c_int32()
        _check(self._lib.pkv_bm_num_free_cpu(self._h, ctypes.byref(n)), "bm_num_free_cpu")
        return n.value

    def _swap(self, fn, seq: int, where: str) -> np.ndarray:
        cap = max(1, (self.seq_len(seq) + self.block_size - 1) // self.block_size)
        out = np.zeros((cap, 2), np.int64)
        n = ctypes.c_int32()
        _check(fn(self._h, seq, out.ctypes.data, cap, ctypes.byref(n)), where)
        return out[:n.value]

    def swap_out(self, seq: int) -> np.ndarray:
        """Pairs (GPU block, CPU block) to copy with swap_blocks; the GPU blocks are released."""
        return self._swap(self._lib.pkv_bm_swap_out, seq, "bm_swap_out")

    def swap_in(self, seq: int) -> np.ndarray:
        """Pairs (CPU block, GPU block) to copy with swap_blocks; the CPU blocks are released."""
        return self._swap(self._lib.pkv_bm_swap_in, seq, "bm_swap_in")
