"""Plain CPU oracle for the INT8 KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; it shares no code with the HIP library.

The pages name INT8 quantisation beside FP8 as a kernel-layer feature (the
devpress.csdn.net/amd vLLM walkthrough, architecture figure: "FP8/INT8 量化")
and give no scheme, so this oracle fixes the plainest symmetric one:

* a stored code c is a signed byte in [-127, 127] (-128 is never written)
  meaning c * scale, with one fp32 scale per cache (k_scale, v_scale);
* writing: y = x / scale in fp32 (IEEE division), rounded to the nearest
  integer with ties to even, clamped to [-127, 127]; NaN is stored as 0;
* attention reads c * scale in place of the K/V value and is otherwise the
  decode of ``oracle.py``.

Pinned in ``tests/test_oracle_int8.py`` against torch's round-half-even and
clamp, against the bf16 decode oracle on pools whose dequantised values are
exact in bf16, and against closed forms.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .oracle import dense_attention, to_f64

INT8_MAX = 127


def quantize(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """int8 codes of x (stored as ``dtype``) divided by ``scale`` in fp32."""
    y = to_f64(x, dtype).astype(np.float32) / np.float32(scale)
    y = np.where(np.isnan(y), np.float32(0), y)
    r = np.rint(y.astype(np.float64))  # round half to even
    return np.clip(r, -INT8_MAX, INT8_MAX).astype(np.int8)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    return np.asarray(codes).astype(np.int8).astype(np.float64) * np.float64(np.float32(scale))


def kv_cache_write_int8(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                        k_cache: np.ndarray, v_cache: np.ndarray, block_size: int, dtype: str,
                        k_scale: float, v_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the int8 caches with token i's K/V rows (all KV heads),
    quantised, at slot ``slot_mapping[i]``; negative slots are skipped."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    kq = quantize(k, dtype, k_scale)
    vq = quantize(v, dtype, v_scale)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        kc[slot // block_size, :, slot % block_size] = kq[i]
        vc[slot // block_size, :, slot % block_size] = vq[i]
    return kc, vc


def paged_attention_decode_int8(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                                block_tables: np.ndarray, context_lens: np.ndarray,
                                scale: float, block_size: int, q_dtype: str, k_scale: float,
                                v_scale: float, rows=None) -> np.ndarray:
    """Decode over an INT8 pool (dequantised K/V); ``rows`` restricts the
    work to (seq, head) pairs and returns ``[len(rows), D]``."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    qf = to_f64(q, q_dtype)
    sc = np.float64(np.float32(scale))

    def gather(s: int, kv_head: Optional[int] = None):
        L = int(context_lens[s])
        pos = np.arange(L)
        phys = np.asarray(block_tables[s])[pos // block_size]
        off = pos % block_size
        if kv_head is None:
            k, v = k_cache[phys, :, off], v_cache[phys, :, off]
        else:
            k, v = k_cache[phys, kv_head, off], v_cache[phys, kv_head, off]
        return dequantize(k, k_scale), dequantize(v, v_scale)

    if rows is not None:
        res = [dense_attention(qf[s, h], *gather(s, h // G), sc)[0] for s, h in rows]
        return np.array(res, np.float64).reshape(-1, D)
    out = np.zeros((S, Hq, D), np.float64)
    for s in range(S):
        K, V = gather(s)
        for g in range(Hkv):
            out[s, g * G:(g + 1) * G] = dense_attention(qf[s, g * G:(g + 1) * G], K[:, g],
                                                        V[:, g], sc)
    return out


def gather_sequence_int8(k_cache: np.ndarray, v_cache: np.ndarray, table_row: np.ndarray,
                         context_len: int, block_size: int, k_scale: float,
                         v_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Dequantised K and V of one sequence in logical order (float64,
    ``[L, Hkv, D]``)."""
    L = int(context_len)
    pos = np.arange(L)
    phys = np.asarray(table_row)[pos // block_size]
    off = pos % block_size
    return dequantize(k_cache[phys, :, off], k_scale), dequantize(v_cache[phys, :, off], v_scale)


def paged_attention_multi_query_int8(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                                     block_tables: np.ndarray, context_lens: np.ndarray,
                                     query_start: np.ndarray, scale: float, block_size: int,
                                     q_dtype: str, k_scale: float, v_scale: float) -> np.ndarray:
    """Causal multi-query attention (the definition of
    ``oracle.paged_attention_multi_query``: sequence s's n rows are its last n
    positions, row i attends [0, L - n + i]) over an INT8 pool read as
    code * scale.  Returns float64 ``[T, Hq, D]``."""
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    qf = to_f64(q, q_dtype)
    sc = np.float64(np.float32(scale))
    out = np.zeros((T, Hq, D), np.float64)
    starts = np.asarray(query_start).tolist()
    for s in range(len(starts) - 1):
        n = starts[s + 1] - starts[s]
        if n == 0:
            continue
        L = int(context_lens[s])
        if n > L:
            raise ValueError("a chunk is longer than its sequence's context")
        K, V = gather_sequence_int8(k_cache, v_cache, block_tables[s], L, block_size, k_scale,
                                    v_scale)
        for i in range(n):
            p = L - n + i
            row = starts[s] + i
            for g in range(Hkv):
                out[row, g * G:(g + 1) * G] = dense_attention(
                    qf[row, g * G:(g + 1) * G], K[:p + 1, g], V[:p + 1, g], sc)
    return out
