"""ctypes binding of libpagedattn (argument marshalling only).

Every step of the computation runs in the HIP kernels of ``libpagedattn.so``;
this module only turns torch tensors into pointers, sizes and the current HIP
stream.  There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpagedattn.so")

PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2
PA_INT8 = 3

PA_OK = 0
STATUS_NAMES = {
    0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_DTYPE",
    -4: "PA_ERR_UNSUPPORTED", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_ALIAS", -7: "PA_ERR_LAUNCH",
    -8: "PA_ERR_OOM", -9: "PA_ERR_NO_SEQ", -10: "PA_ERR_SEQ_EXISTS", -11: "PA_ERR_INDEX",
    -12: "PA_ERR_SCRATCH",
}
PA_ERR_INDEX = -11

# exported symbol -> (restype, argtypes)
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
SIGNATURES = {
    "paged_attention_decode": (_I32, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP,
                                      _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                      _VP, ctypes.c_size_t, _VP]),
    "paged_attention_decode_prefix": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP,
                                             ctypes.c_float, ctypes.c_float, ctypes.c_float, _VP,
                                             _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                             _I32, _I32, _VP, ctypes.c_size_t, _VP]),
    "paged_attention_decode_plan": (_I32, [_VP, _VP, _I32, _VP, _I32, _I32, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _I32, _VP, _I32]),
    "paged_attention_prefix_workspace_size": (ctypes.c_size_t, [_I32] * 8),
    "pa_prefix_groups": (_I32, [_VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP]),
    "paged_attention_decode_noalloc": (_I32, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP,
                                              _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _VP]),
    "paged_attention_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "paged_attention_multi_query": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP,
                                           _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _VP, ctypes.c_size_t, _VP]),
    "paged_attention_multi_query_fp8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float,
                                               ctypes.c_float, ctypes.c_float, _VP, _I32, _I32,
                                               _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                               _I32, _VP, ctypes.c_size_t, _VP]),
    "paged_attention_multi_query_int8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float,
                                                ctypes.c_float, ctypes.c_float, _VP, _I32, _I32,
                                                _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                _I32, _VP, ctypes.c_size_t, _VP]),
    "paged_attention_multi_query_partitions": (_I32, [_I32] * 6),
    "paged_attention_multi_query_workspace_size": (ctypes.c_size_t, [_I32] * 8),
    "paged_attention_multi_query_prefix": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP,
                                                  _VP, ctypes.c_float, ctypes.c_float,
                                                  ctypes.c_float, _VP] + [_I32] * 12 +
                                           [_VP, ctypes.c_size_t, _VP]),
    "paged_attention_multi_query_plan": (_I32, [_VP, _VP, _I32, _VP] + [_I32] * 10 +
                                         [_VP, _I32]),
    "paged_attention_multi_query_prefix_workspace_size": (ctypes.c_size_t, [_I32] * 10),
    "paged_attention_decode_fp8": (_I32, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_float, _VP, _I32, _I32, _I32,
                                          _I32, _I32, _I32, _I32, _I32, _I32, _VP,
                                          ctypes.c_size_t, _VP]),
    "kv_cache_write_fp8": (_I32, [_VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                                  ctypes.c_float, ctypes.c_float, _VP]),
    "paged_attention_decode_int8": (_I32, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_float, _VP, _I32, _I32, _I32,
                                           _I32, _I32, _I32, _I32, _I32, _I32, _VP,
                                           ctypes.c_size_t, _VP]),
    "kv_cache_write_int8": (_I32, [_VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _I32,
                                   ctypes.c_float, ctypes.c_float, _VP]),
    "paged_attention_workspace_size": (ctypes.c_size_t, [_I32] * 6),
    "paged_attention_num_partitions": (_I32, [_I32] * 4),
    "paged_attention_partition_tokens": (_I32, [_I32] * 4),
    "kv_cache_write": (_I32, [_VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP]),
    "copy_blocks": (_I32, [_VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32, _I32, _VP, _VP]),
    "kv_cache_append": (_I32, [_VP, _I32, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I32,
                               _I32, _I32, ctypes.c_float, ctypes.c_float, _VP, _VP]),
    "pagedattn_status_string": (ctypes.c_char_p, [_I32]),
    "pagedattn_set_index_check": (None, [_I32]),
    "pagedattn_index_check": (_I32, []),
    # block manager (include/pagedattn_blocks.h)
    "pa_bm_create": (_VP, [_I32, _I32]),
    "pa_bm_destroy": (None, [_VP]),
    "pa_bm_num_free_blocks": (_I32, [_VP]),
    "pa_bm_can_allocate": (_I32, [_VP, _I32]),
    "pa_bm_add_sequence": (_I32, [_VP, ctypes.c_int64, _I32, _VP]),
    "pa_bm_fork": (_I32, [_VP, ctypes.c_int64, ctypes.c_int64]),
    "pa_bm_append_slot": (_I32, [_VP, ctypes.c_int64, _VP, _VP, _VP]),
    "pa_bm_free_sequence": (_I32, [_VP, ctypes.c_int64]),
    "pa_bm_context_len": (_I32, [_VP, ctypes.c_int64]),
    "pa_bm_block_table": (_I32, [_VP, ctypes.c_int64, _VP, _I32]),
    "pa_bm_prepare_decode": (_I32, [_VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "pa_bm_stats": (_I32, [_VP, _VP]),
    # engine (include/pagedattn_engine.h)
    "pa_engine_create": (_I32, [_VP, _VP, _VP, _VP]),
    "pa_engine_destroy": (None, [_VP]),
    "pa_engine_submit": (_I32, [_VP, ctypes.c_int64, _I32, _I32, _I32]),
    "pa_engine_step": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP]),
    "pa_engine_num_waiting": (_I32, [_VP]),
    "pa_engine_num_running": (_I32, [_VP]),
    "pa_engine_blocks": (_VP, [_VP]),
    "pagedattn_version": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().pagedattn_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({msg})")


def lib() -> ctypes.CDLL:
    """Load libpagedattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_386_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.uint8:
        return PA_FP8_E4M3  # pools of E4M3 codes
    if t.dtype == torch.int8:
        return PA_INT8  # pools of INT8 codes
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PagedAttnError(fn, status)


def set_index_check(enable: bool) -> None:
    """Turn the library's index checking (a debug mode) on or off: while on,
    calls check the indices their kernels would read and raise
    PagedAttnError(PA_ERR_INDEX) instead of launching when one is out of
    range."""
    lib().pagedattn_set_index_check(1 if enable else 0)


def index_check() -> bool:
    return bool(lib().pagedattn_index_check())


def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition_size: int = 0) -> int:
    return int(lib().paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                     head_dim, max_context_len, partition_size))


def num_partitions(num_seqs: int, num_kv_heads: int, max_context_len: int,
                   partition_size: int = 0) -> int:
    return int(lib().paged_attention_num_partitions(num_seqs, num_kv_heads, max_context_len,
                                                     partition_size))


def partition_tokens(num_seqs: int, num_kv_heads: int, max_context_len: int,
                     partition_size: int = 0) -> int:
    return int(lib().paged_attention_partition_tokens(num_seqs, num_kv_heads, max_context_len,
                                                      partition_size))


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
                           *, max_context_len: int, partition_size: int = 0, workspace=None,
                           stream=None) -> None:
    """Decode attention through the block tables (see include/pagedattn.h).

    q: [S, Hq, D]; k_cache/v_cache: [NB, Hkv, B, D] (float32 or bfloat16);
    block_tables: int32 [S, MB]; context_lens: int32 [S]; out: float32 [S, Hq, D].
    ``workspace`` (a uint8 device tensor) is allocated here when needed and not
    given; callers timing the kernel pass one in."""
    import torch
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    need = workspace_size(S, Hq, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    for t in (q, k_cache, v_cache, block_tables, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    st = lib().paged_attention_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(out), S, Hq, Hkv, D, B, NB, MB, int(max_context_len),
        _dtype_code(q), int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))
    _check("paged_attention_decode", st)


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens,
                                   scale: float, out, *, max_context_len: int,
                                   partition_size: int = 0, stream=None) -> None:
    """paged_attention_decode with the workspace in the library's static
    device scratch (include/pagedattn.h): nothing is allocated, here or in
    the library.  Raises PagedAttnError(PA_ERR_SCRATCH) when the call needs
    more than ``noalloc_scratch_bytes()``."""
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    for t in (q, k_cache, v_cache, block_tables, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    st = lib().paged_attention_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(out), S, Hq, Hkv, D, B, NB, MB, int(max_context_len),
        _dtype_code(q), int(partition_size), _stream(stream))
    _check("paged_attention_decode_noalloc", st)


def prefix_groups(block_tables, context_lens, block_size: int, num_q_heads: int,
                  num_kv_heads: int, min_shared_tokens: int = 16):
    """The shared-prefix groups of a batch from host block tables
    (pa_prefix_groups in include/pagedattn_blocks.h): numpy int32
    ``groups [n, 2]`` and ``shared_lens [S]``.  At most 64 / G members per
    group, as the decode kernel takes them."""
    import numpy as np
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = int(lens.shape[0])
    MB = int(tables.shape[1]) if tables.ndim == 2 and S else 1
    groups = np.zeros((max(S, 1), 2), np.int32)
    shared = np.zeros(max(S, 1), np.int32)
    G = num_q_heads // num_kv_heads
    n = lib().pa_prefix_groups(tables.ctypes.data, lens.ctypes.data, S, MB, int(block_size),
                               max(1, 64 // G), int(min_shared_tokens), groups.ctypes.data,
                               shared.ctypes.data)
    if n < 0:
        raise PagedAttnError("pa_prefix_groups", n)
    return groups[:n].copy(), shared[:S].copy()


def prefix_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          max_context_len: int, partition_size: int, num_groups: int,
                          kv_dtype: int) -> int:
    return int(lib().paged_attention_prefix_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size,
        num_groups, kv_dtype))


def decode_plan(context_lens, groups, shared_lens, *, num_q_heads: int, num_kv_heads: int,
                head_dim: int, block_size: int, max_blocks_per_seq: int, max_context_len: int,
                kv_dtype: int, partition_size: int = 0):
    """The dispatch list of paged_attention_decode_prefix planned on the host
    (paged_attention_decode_plan): numpy int32.  ``context_lens``,
    ``groups`` ([n, 2] or None) and ``shared_lens`` are host arrays."""
    import numpy as np
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = int(lens.shape[0])
    ng = 0 if groups is None else int(len(groups))
    g = np.ascontiguousarray(groups if ng else np.zeros((1, 2)), dtype=np.int32)
    sh = np.ascontiguousarray(shared_lens if ng else np.zeros(max(S, 1)), dtype=np.int32)
    P = num_partitions(S, num_kv_heads, max_context_len, partition_size)
    if P < 0:
        raise PagedAttnError("paged_attention_num_partitions", P)
    cap = max(S * P + 4 * ng, 1)
    out = np.zeros(cap, np.int32)
    n = lib().paged_attention_decode_plan(
        lens.ctypes.data, g.ctypes.data if ng else 0, ng, sh.ctypes.data if ng else 0, S,
        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        int(max_context_len), int(kv_dtype), int(partition_size), out.ctypes.data, cap)
    if n < 0:
        raise PagedAttnError("paged_attention_decode_plan", n)
    return out[:n].copy()


def paged_attention_decode_prefix(q, k_cache, v_cache, block_tables, context_lens, groups,
                                  shared_lens, scale: float, out, *, max_context_len: int,
                                  k_scale: float = 1.0, v_scale: float = 1.0,
                                  partition_size: int = 0, workspace=None, dispatch=None,
                                  stream=None) -> None:
    """Decode with shared prefixes read once per group (see
    include/pagedattn.h).  ``groups``: device int32 [n, 2] (first sequence,
    members); ``shared_lens``: device int32 [S].  The pool may be float32,
    bfloat16, or 8-bit codes (uint8 = FP8 E4M3, int8 = INT8, with bfloat16 q
    and the two scales).  ``dispatch``: an optional device int32 list from
    ``decode_plan`` (else the device sorts the work)."""
    import torch
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    kv = _dtype_code(k_cache)
    ng = int(groups.shape[0]) if groups is not None else 0
    need = prefix_workspace_size(S, Hq, Hkv, D, max_context_len, partition_size, ng, kv)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    for t in (q, k_cache, v_cache, block_tables, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if ng and not (groups.is_contiguous() and shared_lens.is_contiguous()):
        raise ValueError("groups and shared_lens must be contiguous")
    st = lib().paged_attention_decode_prefix(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(groups) if ng else 0, ng, _ptr(shared_lens) if ng else 0, _ptr(dispatch),
        float(scale),
        float(k_scale), float(v_scale), _ptr(out), S, Hq, Hkv, D, B, NB, MB,
        int(max_context_len), kv, int(partition_size), _ptr(workspace), ws_bytes,
        _stream(stream))
    _check("paged_attention_decode_prefix", st)


def noalloc_scratch_bytes() -> int:
    """Bytes of the static device scratch paged_attention_decode_noalloc uses."""
    return int(lib().paged_attention_noalloc_scratch_bytes())


def multi_query_partitions(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                           max_query_len: int, max_context_len: int,
                           partition_size: int = 0) -> int:
    return int(lib().paged_attention_multi_query_partitions(
        num_seqs, num_q_heads, num_kv_heads, max_query_len, max_context_len, partition_size))


def multi_query_workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int,
                               num_kv_heads: int, head_dim: int, max_query_len: int,
                               max_context_len: int, partition_size: int = 0) -> int:
    return int(lib().paged_attention_multi_query_workspace_size(
        num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len,
        max_context_len, partition_size))


def paged_attention_multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start,
                                scale: float, out, *, max_query_len: int, max_context_len: int,
                                partition_size: int = 0, workspace=None, stream=None) -> None:
    """Causal attention of several query tokens per sequence (see
    include/pagedattn.h).  q: [T, Hq, D] bfloat16; query_start: int32 [S+1];
    out: float32 [T, Hq, D].  ``workspace`` (a uint8 device tensor) is
    allocated here when needed and not given."""
    import torch
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    S = context_lens.shape[0]
    if query_start.shape[0] != S + 1:
        raise ValueError("query_start must have num_seqs + 1 entries")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    for t in (q, k_cache, v_cache, block_tables, context_lens, query_start, out):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    need = multi_query_workspace_size(S, T, Hq, Hkv, D, max_query_len, max_context_len,
                                      partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().paged_attention_multi_query(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start), float(scale), _ptr(out), S, T, Hq, Hkv, D, B, NB, MB,
        int(max_query_len), int(max_context_len), _dtype_code(q), int(partition_size),
        _ptr(workspace), ws_bytes, _stream(stream))
    _check("paged_attention_multi_query", st)


def paged_attention_multi_query_fp8(q, k_cache, v_cache, block_tables, context_lens,
                                    query_start, scale: float, k_scale: float, v_scale: float,
                                    out, *, max_query_len: int, max_context_len: int,
                                    partition_size: int = 0, workspace=None,
                                    stream=None) -> None:
    """paged_attention_multi_query over an FP8 pool (uint8 tensors of E4M3
    codes [NB, Hkv, B, D]); q: bfloat16 [T, Hq, D]; at most 64 (token, head)
    rows per KV head."""
    import torch
    _multi_query_q8("paged_attention_multi_query_fp8", torch.uint8, q, k_cache, v_cache,
                    block_tables, context_lens, query_start, scale, k_scale, v_scale, out,
                    max_query_len, max_context_len, partition_size, workspace, stream)


def paged_attention_multi_query_int8(q, k_cache, v_cache, block_tables, context_lens,
                                     query_start, scale: float, k_scale: float, v_scale: float,
                                     out, *, max_query_len: int, max_context_len: int,
                                     partition_size: int = 0, workspace=None,
                                     stream=None) -> None:
    """paged_attention_multi_query over an INT8 pool (int8 tensors
    [NB, Hkv, B, D]); q: bfloat16 [T, Hq, D]; at most 64 (token, head) rows
    per KV head."""
    import torch
    _multi_query_q8("paged_attention_multi_query_int8", torch.int8, q, k_cache, v_cache,
                    block_tables, context_lens, query_start, scale, k_scale, v_scale, out,
                    max_query_len, max_context_len, partition_size, workspace, stream)


def multi_query_prefix_workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int,
                                      num_kv_heads: int, head_dim: int, max_query_len: int,
                                      max_context_len: int, partition_size: int,
                                      num_groups: int, kv_dtype: int) -> int:
    return int(lib().paged_attention_multi_query_prefix_workspace_size(
        num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len,
        max_context_len, partition_size, num_groups, kv_dtype))


def paged_attention_multi_query_prefix(q, k_cache, v_cache, block_tables, context_lens,
                                       query_start, groups, shared_lens, scale: float, out, *,
                                       max_query_len: int, max_context_len: int,
                                       k_scale: float = 1.0, v_scale: float = 1.0,
                                       partition_size: int = 0, workspace=None, dispatch=None,
                                       stream=None) -> None:
    """paged_attention_multi_query for a batch whose sequences share prefix
    blocks (include/pagedattn.h): ``groups`` int32 [n, 2] (first sequence,
    members) and ``shared_lens`` int32 [S] on the device, as pa_prefix_groups
    gives them (None and 0 groups: the plain call).  The pool's dtype picks
    bf16, FP8 or INT8; q is bfloat16.  ``dispatch``: a device int32 list from
    multi_query_plan, or None to sort on the device."""
    import torch
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    S = context_lens.shape[0]
    if query_start.shape[0] != S + 1:
        raise ValueError("query_start must have num_seqs + 1 entries")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    ng = int(groups.shape[0]) if groups is not None and groups.dim() == 2 else 0
    for t in (q, k_cache, v_cache, block_tables, context_lens, query_start, out, groups,
              shared_lens, dispatch):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    kv = _dtype_code(k_cache)
    need = multi_query_prefix_workspace_size(S, T, Hq, Hkv, D, max_query_len, max_context_len,
                                             partition_size, ng, kv)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().paged_attention_multi_query_prefix(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start), _ptr(groups) if ng else None, ng,
        _ptr(shared_lens) if ng else None, _ptr(dispatch) if dispatch is not None else None,
        float(scale), float(k_scale), float(v_scale),
        _ptr(out), S, T, Hq, Hkv, D, B, NB, MB, int(max_query_len), int(max_context_len), kv,
        int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))
    _check("paged_attention_multi_query_prefix", st)


def multi_query_plan(context_lens, groups, shared_lens, *, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, block_size: int, max_blocks_per_seq: int,
                     max_query_len: int, max_context_len: int, kv_dtype: int,
                     partition_size: int = 0):
    """The dispatch list of paged_attention_multi_query_prefix planned on the
    host (paged_attention_multi_query_plan): numpy int32.  ``context_lens``,
    ``groups`` ([n, 2] or None) and ``shared_lens`` are host arrays."""
    import numpy as np
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = int(lens.shape[0])
    ng = 0 if groups is None else int(len(groups))
    g = np.ascontiguousarray(groups if ng else np.zeros((1, 2)), dtype=np.int32)
    sh = np.ascontiguousarray(shared_lens if ng else np.zeros(max(S, 1)), dtype=np.int32)
    P = multi_query_partitions(S, num_q_heads, num_kv_heads, max_query_len, max_context_len,
                               partition_size)
    if P < 0:
        raise PagedAttnError("paged_attention_multi_query_partitions", P)
    G = num_q_heads // num_kv_heads
    per = max_query_len * G
    cap = max(S * P + ng * per, 1)  # at least the prefix items a group can have
    out = np.zeros(cap, np.int32)
    n = lib().paged_attention_multi_query_plan(
        lens.ctypes.data, g.ctypes.data if ng else 0, ng, sh.ctypes.data if ng else 0, S,
        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        int(max_query_len), int(max_context_len), int(kv_dtype), int(partition_size),
        out.ctypes.data, cap)
    if n < 0:
        raise PagedAttnError("paged_attention_multi_query_plan", n)
    return out[:n].copy()


def _multi_query_q8(fn, pool_dtype, q, k_cache, v_cache, block_tables, context_lens,
                    query_start, scale, k_scale, v_scale, out, max_query_len, max_context_len,
                    partition_size, workspace, stream) -> None:
    import torch
    T, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    if k_cache.dtype != pool_dtype or v_cache.dtype != pool_dtype:
        raise TypeError(f"{fn} takes pools of {pool_dtype}")
    S = context_lens.shape[0]
    if query_start.shape[0] != S + 1:
        raise ValueError("query_start must have num_seqs + 1 entries")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    for t in (q, k_cache, v_cache, block_tables, context_lens, query_start, out):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    need = multi_query_workspace_size(S, T, Hq, Hkv, D, max_query_len, max_context_len,
                                      partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(lib(), fn)(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start), float(scale), float(k_scale), float(v_scale), _ptr(out), S, T, Hq,
        Hkv, D, B, NB, MB, int(max_query_len), int(max_context_len), int(partition_size),
        _ptr(workspace), ws_bytes, _stream(stream))
    _check(fn, st)


def _decode_q8(fn: str, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
               v_scale, out, max_context_len, partition_size, workspace, stream, dtype) -> None:
    import torch
    S, Hq, D = q.shape
    NB, Hkv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q/k_cache/v_cache shapes disagree")
    if k_cache.dtype != dtype or v_cache.dtype != dtype:
        raise TypeError(f"{fn} takes pools of {dtype}")
    MB = block_tables.shape[1] if block_tables.dim() == 2 else 0
    need = workspace_size(S, Hq, Hkv, D, max_context_len, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    for t in (q, k_cache, v_cache, block_tables, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    st = getattr(lib(), fn)(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), float(k_scale), float(v_scale), _ptr(out), S, Hq, Hkv, D, B, NB, MB,
        int(max_context_len), int(partition_size), _ptr(workspace), ws_bytes, _stream(stream))
    _check(fn, st)


def paged_attention_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                               k_scale: float, v_scale: float, out, *, max_context_len: int,
                               partition_size: int = 0, workspace=None, stream=None) -> None:
    """Decode over an FP8 pool (uint8 tensors of E4M3 codes [NB, Hkv, B, D]);
    q: bfloat16 [S, Hq, D]; out: float32 [S, Hq, D]."""
    import torch
    _decode_q8("paged_attention_decode_fp8", q, k_cache, v_cache, block_tables, context_lens,
               scale, k_scale, v_scale, out, max_context_len, partition_size, workspace, stream,
               torch.uint8)


def paged_attention_decode_int8(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                                k_scale: float, v_scale: float, out, *, max_context_len: int,
                                partition_size: int = 0, workspace=None, stream=None) -> None:
    """Decode over an INT8 pool (int8 tensors [NB, Hkv, B, D])."""
    import torch
    _decode_q8("paged_attention_decode_int8", q, k_cache, v_cache, block_tables, context_lens,
               scale, k_scale, v_scale, out, max_context_len, partition_size, workspace, stream,
               torch.int8)


def _write_q8(fn, k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream) -> None:
    T = k.shape[0]
    NB, Hkv, B, D = k_cache.shape
    for t in (k, v, slot_mapping, k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    st = getattr(lib(), fn)(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
                            _ptr(v_cache), NB, B, Hkv, D, _dtype_code(k), float(k_scale),
                            float(v_scale), _stream(stream))
    _check(fn, st)


def kv_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale: float, v_scale: float, *,
                       stream=None) -> None:
    """Quantise k[i], v[i] ([T, Hkv, D], float32 or bfloat16) into the FP8
    pool (uint8 [NB, Hkv, B, D]) at slot slot_mapping[i]."""
    _write_q8("kv_cache_write_fp8", k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale,
              stream)


def kv_cache_write_int8(k, v, slot_mapping, k_cache, v_cache, k_scale: float, v_scale: float, *,
                        stream=None) -> None:
    """Quantise k[i], v[i] into the INT8 pool (int8 [NB, Hkv, B, D])."""
    _write_q8("kv_cache_write_int8", k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale,
              stream)


def kv_cache_write(k, v, slot_mapping, k_cache, v_cache, *, stream=None) -> None:
    """Store k[i], v[i] ([T, Hkv, D]) at slot slot_mapping[i] of the pool."""
    T = k.shape[0]
    NB, Hkv, B, D = k_cache.shape
    for t in (k, v, slot_mapping, k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    st = lib().kv_cache_write(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
                              _ptr(v_cache), NB, B, Hkv, D, _dtype_code(k_cache), _stream(stream))
    _check("kv_cache_write", st)


def copy_blocks(src_dst_pairs, k_cache, v_cache, *, host_pairs=None, stream=None) -> None:
    """Copy block src onto block dst of both caches for each (src, dst) row of
    ``src_dst_pairs`` (int32 [P, 2] on the device).  ``host_pairs`` (a
    contiguous int32 CPU tensor or numpy array with the same pairs) turns on the
    host-side overlap check."""
    NB, Hkv, B, D = k_cache.shape
    P = src_dst_pairs.shape[0] if src_dst_pairs.dim() == 2 else 0
    hp = None
    keep = None
    if host_pairs is not None:
        import numpy as np
        keep = np.ascontiguousarray(np.asarray(host_pairs), dtype=np.int32)
        hp = keep.ctypes.data_as(ctypes.c_void_p)
    st = lib().copy_blocks(_ptr(src_dst_pairs), P, _ptr(k_cache), _ptr(v_cache), NB, B, Hkv, D,
                           _dtype_code(k_cache), hp, _stream(stream))
    del keep
    _check("copy_blocks", st)


def kv_cache_append(src_dst_pairs, k, v, slot_mapping, k_cache, v_cache, *, k_scale: float = 1.0,
                    v_scale: float = 1.0, host_pairs=None, stream=None) -> None:
    """copy_blocks(src_dst_pairs) followed by the write of k[i], v[i] at slot
    slot_mapping[i], in one launch.  With k and v of the pool's dtype the rows
    are stored as they are (kv_cache_write); with float32 or bfloat16 rows and
    an 8-bit pool they are quantised with k_scale and v_scale
    (kv_cache_write_fp8 / _int8).  ``host_pairs`` turns on the host-side
    overlap check of copy_blocks."""
    NB, Hkv, B, D = k_cache.shape
    P = src_dst_pairs.shape[0] if src_dst_pairs is not None and src_dst_pairs.dim() == 2 else 0
    T = k.shape[0] if k is not None else 0
    for t in (k, v, slot_mapping, k_cache, v_cache, src_dst_pairs):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    hp = None
    keep = None
    if host_pairs is not None:
        import numpy as np
        keep = np.ascontiguousarray(np.asarray(host_pairs), dtype=np.int32)
        hp = keep.ctypes.data_as(ctypes.c_void_p)
    kv = _dtype_code(k_cache)
    src = _dtype_code(k) if k is not None else kv
    st = lib().kv_cache_append(_ptr(src_dst_pairs) if P else None, P,
                               _ptr(k) if T else None, _ptr(v) if T else None,
                               _ptr(slot_mapping) if T else None, T, _ptr(k_cache),
                               _ptr(v_cache), NB, B, Hkv, D, src, kv, float(k_scale),
                               float(v_scale), hp, _stream(stream))
    del keep
    _check("kv_cache_append", st)


# ---------------------------------------------------------------- block manager

class BlockStats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("shared_blocks", ctypes.c_int32), ("num_sequences", ctypes.c_int32),
                ("tokens_logical", ctypes.c_int64), ("tokens_stored", ctypes.c_int64),
                ("slots_allocated", ctypes.c_int64), ("utilisation", ctypes.c_double)]


class BlockManager:
    """The host block manager of libpagedattn (include/pagedattn_blocks.h):
    pool, block tables, reference-counted forks with copy-on-write, and the
    index arrays of a decode step.  Argument marshalling only."""

    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.num_blocks = num_blocks
        self._h = lib().pa_bm_create(num_blocks, block_size)
        if not self._h:
            raise ValueError(f"bad block manager sizes ({num_blocks}, {block_size})")

    def close(self) -> None:
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free_blocks(self) -> int:
        return int(lib().pa_bm_num_free_blocks(self._h))

    def can_allocate(self, num_tokens: int) -> bool:
        return bool(lib().pa_bm_can_allocate(self._h, num_tokens))

    def add_sequence(self, seq_id: int, num_tokens: int):
        """Admit a sequence holding num_tokens tokens; returns their slots (int32)."""
        import numpy as np
        slots = np.zeros(max(num_tokens, 1), np.int32)
        _check("pa_bm_add_sequence", lib().pa_bm_add_sequence(
            self._h, seq_id, num_tokens, slots.ctypes.data_as(ctypes.c_void_p)))
        return slots[:num_tokens]

    def fork(self, parent: int, child: int) -> None:
        _check("pa_bm_fork", lib().pa_bm_fork(self._h, parent, child))

    def append_slot(self, seq_id: int):
        """Returns (slot, copy_src, copy_dst); the copy pair is (-1, -1) when none."""
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_append_slot", lib().pa_bm_append_slot(
            self._h, seq_id, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, src.value, dst.value

    def free_sequence(self, seq_id: int) -> None:
        _check("pa_bm_free_sequence", lib().pa_bm_free_sequence(self._h, seq_id))

    def context_len(self, seq_id: int) -> int:
        n = int(lib().pa_bm_context_len(self._h, seq_id))
        if n < 0:
            raise PagedAttnError("pa_bm_context_len", n)
        return n

    def block_table(self, seq_id: int):
        import numpy as np
        n = int(lib().pa_bm_block_table(self._h, seq_id, None, 0))
        if n < 0:
            raise PagedAttnError("pa_bm_block_table", n)
        t = np.zeros(max(n, 1), np.int32)
        lib().pa_bm_block_table(self._h, seq_id, t.ctypes.data_as(ctypes.c_void_p), n)
        return t[:n]

    def prepare_decode(self, seq_ids, max_blocks: int, pad_block: int = 0):
        """One decode step: returns (slot_mapping [n], copy_pairs [P, 2],
        block_tables [n, max_blocks], context_lens [n]) as int32 numpy arrays."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, np.int64))
        n = len(ids)
        slots = np.zeros(max(n, 1), np.int32)
        pairs = np.zeros((max(n, 1), 2), np.int32)
        tables = np.zeros((max(n, 1), max(max_blocks, 1)), np.int32)
        lens = np.zeros(max(n, 1), np.int32)
        npairs = ctypes.c_int32(0)
        vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
        _check("pa_bm_prepare_decode", lib().pa_bm_prepare_decode(
            self._h, vp(ids), n, max_blocks, pad_block, vp(slots), vp(pairs),
            ctypes.byref(npairs), vp(tables), vp(lens)))
        return slots[:n], pairs[:npairs.value].copy(), tables[:n, :max_blocks], lens[:n]

    def stats(self) -> BlockStats:
        st = BlockStats()
        _check("pa_bm_stats", lib().pa_bm_stats(self._h, ctypes.byref(st)))
        return st


# ---------------------------------------------------------------- engine

class EngineConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_blocks", "block_size", "num_q_heads", "num_kv_heads", "head_dim", "dtype",
        "max_batch", "max_context_len", "max_prompt_rows", "partition_size", "device")] + [
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("host_plan", ctypes.c_int32)]


class _StepInfo(ctypes.Structure):
    _P64 = ctypes.POINTER(ctypes.c_int64)
    _P32 = ctypes.POINTER(ctypes.c_int32)
    _fields_ = [
        ("batch", ctypes.c_int32), ("admitted", ctypes.c_int32),
        ("prompt_rows", ctypes.c_int32), ("preempted", ctypes.c_int32),
        ("finished", ctypes.c_int32), ("num_copies", ctypes.c_int32),
        ("max_context_len", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
        ("context_tokens", ctypes.c_int64),
        ("batch_seq_ids", _P64), ("context_lens", _P32), ("slot_mapping", _P32),
        ("block_tables", _P32), ("copy_pairs", _P32), ("admitted_seq_ids", _P64),
        ("admitted_rows", _P32), ("prompt_slots", _P32), ("preempted_seq_ids", _P64),
        ("finished_seq_ids", _P64), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_groups", ctypes.c_int32), ("prefix_groups", _P32), ("shared_lens", _P32),
        ("dispatch_len", ctypes.c_int32), ("dispatch", _P32),
        ("unique_tokens", ctypes.c_int64),
        ("host_us", ctypes.c_float), ("wait_us", ctypes.c_float),
    ]


class StepInfo:
    """What one engine step did, copied out of the engine's host arrays (the
    counts only when ``arrays`` is false)."""

    def __init__(self, raw: _StepInfo, arrays: bool = True):
        for k in ("batch", "admitted", "prompt_rows", "preempted", "finished", "num_copies",
                  "max_context_len", "free_blocks", "context_tokens", "num_groups",
                  "dispatch_len", "unique_tokens"):
            setattr(self, k, int(getattr(raw, k)))
        self.host_us = float(raw.host_us)
        self.wait_us = float(raw.wait_us)
        if not arrays:
            return
        import numpy as np

        def arr(p, n, dt, shape=None):
            if n == 0:
                return np.zeros(shape or (0,), dt)
            a = np.ctypeslib.as_array(p, shape=(n,)).copy()
            return a.reshape(shape) if shape else a

        n = raw.batch
        mb = raw.max_blocks_per_seq
        self.batch_seq_ids = arr(raw.batch_seq_ids, n, np.int64)
        self.context_lens = arr(raw.context_lens, n, np.int32)
        self.slot_mapping = arr(raw.slot_mapping, n, np.int32)
        self.block_tables = arr(raw.block_tables, n * mb, np.int32, (n, mb))
        self.copy_pairs = arr(raw.copy_pairs, 2 * raw.num_copies, np.int32,
                              (raw.num_copies, 2))
        self.admitted_seq_ids = arr(raw.admitted_seq_ids, raw.admitted, np.int64)
        self.admitted_rows = arr(raw.admitted_rows, raw.admitted, np.int32)
        self.prompt_slots = arr(raw.prompt_slots, raw.prompt_rows, np.int32)
        self.preempted_seq_ids = arr(raw.preempted_seq_ids, raw.preempted, np.int64)
        self.finished_seq_ids = arr(raw.finished_seq_ids, raw.finished, np.int64)
        self.prefix_groups = arr(raw.prefix_groups, 2 * raw.num_groups, np.int32,
                                 (raw.num_groups, 2))
        self.shared_lens = arr(raw.shared_lens, n, np.int32)
        self.dispatch = arr(raw.dispatch, raw.dispatch_len, np.int32)


class Engine:
    """The continuously batched decode engine of libpagedattn
    (include/pagedattn_engine.h).  Argument marshalling only.

    ``k_cache``/``v_cache`` (torch tensors [NB, Hkv, B, D]) give the pool;
    with ``k_cache=None`` the engine only plans (no GPU use), and then the
    pool sizes come from the keyword arguments."""

    def __init__(self, k_cache=None, v_cache=None, *, num_q_heads: int, max_batch: int,
                 max_context_len: int, max_prompt_rows: int = 0, partition_size: int = 0,
                 num_blocks: int = 0, block_size: int = 0, num_kv_heads: int = 0,
                 head_dim: int = 0, dtype: int = PA_BF16, k_scale: float = 1.0,
                 v_scale: float = 1.0, host_plan: bool = True):
        device = k_cache is not None
        if device:
            num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
            dtype = _dtype_code(k_cache)
            if tuple(v_cache.shape) != tuple(k_cache.shape) or not k_cache.is_contiguous() \
                    or not v_cache.is_contiguous():
                raise ValueError("k_cache/v_cache must be contiguous and of one shape")
        self.cfg = EngineConfig(num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                                dtype, max_batch, max_context_len,
                                max_prompt_rows or max_context_len, partition_size,
                                1 if device else 0, float(k_scale), float(v_scale),
                                1 if host_plan else 0)
        self._pool = (k_cache, v_cache)
        h = ctypes.c_void_p()
        _check("pa_engine_create", lib().pa_engine_create(
            ctypes.byref(self.cfg), _ptr(k_cache), _ptr(v_cache), ctypes.byref(h)))
        self._h = h.value

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().pa_engine_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, request_id: int, prompt_len: int, max_new_tokens: int,
               num_samples: int = 1) -> None:
        _check("pa_engine_submit", lib().pa_engine_submit(
            self._h, request_id, prompt_len, max_new_tokens, num_samples))

    def step(self, q=None, k_new=None, v_new=None, prompt_k=None, prompt_v=None,
             scale: float = 1.0, out=None, *, stream=None, arrays: bool = True) -> StepInfo:
        raw = _StepInfo()
        st = _stream(stream) if self.cfg.device else 0
        _check("pa_engine_step", lib().pa_engine_step(
            self._h, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(prompt_k), _ptr(prompt_v),
            float(scale), _ptr(out), st, ctypes.byref(raw)))
        return StepInfo(raw, arrays)

    def num_waiting(self) -> int:
        return int(lib().pa_engine_num_waiting(self._h))

    def num_running(self) -> int:
        return int(lib().pa_engine_num_running(self._h))

    def block_stats(self) -> BlockStats:
        st = BlockStats()
        _check("pa_bm_stats", lib().pa_bm_stats(lib().pa_engine_blocks(self._h),
                                                 ctypes.byref(st)))
        return st

    def context_len(self, seq_id: int) -> int:
        n = int(lib().pa_bm_context_len(lib().pa_engine_blocks(self._h), seq_id))
        if n < 0:
            raise PagedAttnError("pa_bm_context_len", n)
        return n
