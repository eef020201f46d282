"""Plain CPU oracle for the FP8 (E4M3) KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; it shares no code with the HIP library.

The pages name FP8/INT8 quantisation only as a kernel-layer feature (the
devpress.csdn.net/amd vLLM walkthrough, architecture figure: "FP8/INT8 量化" in
the CUDA kernel layer) and say that FP8 trades a little precision for memory
and bandwidth (the chenxutan.com page, section 5.3).  They give no format or
scale scheme, so this oracle fixes the plainest one:

* element format: E4M3 of the OCP 8-bit floating point specification -- sign
  bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; the all-ones exponent with mantissa 7 is NaN; there
  are no infinities; the largest finite value is 448;
* one fp32 scale per cache (k_scale for K, v_scale for V): a stored code c
  means e4m3(c) * scale;
* writing: y = x / scale computed in fp32 (IEEE division), clamped to
  [-448, 448], then rounded to the nearest E4M3 value, ties to the even
  mantissa; NaN stays NaN (code 0x7F with the sign);
* attention reads e4m3(c) * scale in place of the K/V value and is otherwise
  the decode of ``oracle.py``.

Pinned in ``tests/test_oracle_fp8.py`` against torch's float8_e4m3fn
conversions (every code, and many fp32 values including every tie), against
the bf16 decode oracle on pools whose dequantised values are exact in bf16,
and against closed forms; the multi-query function against the bf16
multi-query oracle on such pools and against the FP8 decode for one token per
sequence.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .oracle import dense_attention, to_f64

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


# the 127 non-negative finite values, ascending with their code
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """E4M3 code of each value (float32 input): saturate to +-448, then the
    nearest representable magnitude, ties to the code with even mantissa."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    out = np.zeros(y.shape, np.uint8)
    nan = np.isnan(y)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], code)
    neg = np.signbit(y)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, 0x7F | (np.signbit(y).astype(np.int64) << 7), code)
    out[...] = code.astype(np.uint8)
    return out


def quantize(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Codes of x (stored as ``dtype``: float32 or bfloat16 bits) divided by
    ``scale`` in fp32."""
    xf = to_f64(x, dtype).astype(np.float32)
    y = xf / np.float32(scale)  # IEEE fp32 division
    return e4m3_encode(y)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    return e4m3_decode(codes) * np.float64(np.float32(scale))


def kv_cache_write_fp8(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                       k_cache: np.ndarray, v_cache: np.ndarray, block_size: int, dtype: str,
                       k_scale: float, v_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the uint8 caches with token i's K/V rows (all KV heads),
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


def gather_sequence_fp8(k_cache: np.ndarray, v_cache: np.ndarray, table_row: np.ndarray,
                        context_len: int, block_size: int, k_scale: float, v_scale: float,
                        kv_head: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Dequantised K and V of one sequence in logical order (float64)."""
    L = int(context_len)
    pos = np.arange(L)
    phys = np.asarray(table_row)[pos // block_size]
    off = pos % block_size
    if kv_head is None:
        k, v = k_cache[phys, :, off], v_cache[phys, :, off]
    else:
        k, v = k_cache[phys, kv_head, off], v_cache[phys, kv_head, off]
    return dequantize(k, k_scale), dequantize(v, v_scale)


def paged_attention_decode_fp8(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                               block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                               block_size: int, q_dtype: str, k_scale: float, v_scale: float,
                               rows=None) -> np.ndarray:
    """Decode over an FP8 pool: out[s, h] = attention of q[s, h] over the
    dequantised K/V of sequence s.  ``rows`` (optional (seq, head) pairs)
    restricts the work; the result is then ``[len(rows), D]``."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    qf = to_f64(q, q_dtype)
    sc = np.float64(np.float32(scale))
    if rows is not None:
        res = []
        for s, h in rows:
            K, V = gather_sequence_fp8(k_cache, v_cache, block_tables[s], int(context_lens[s]),
                                       block_size, k_scale, v_scale, kv_head=h // G)
            res.append(dense_attention(qf[s, h], K, V, sc)[0])
        return np.array(res, np.float64).reshape(-1, D)
    out = np.zeros((S, Hq, D), np.float64)
    for s in range(S):
        K, V = gather_sequence_fp8(k_cache, v_cache, block_tables[s], int(context_lens[s]),
                                   block_size, k_scale, v_scale)
        for g in range(Hkv):
            out[s, g * G:(g + 1) * G] = dense_attention(qf[s, g * G:(g + 1) * G], K[:, g],
                                                        V[:, g], sc)
    return out


def paged_attention_multi_query_fp8(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                                    block_tables: np.ndarray, context_lens: np.ndarray,
                                    query_start: np.ndarray, scale: float, block_size: int,
                                    q_dtype: str, k_scale: float, v_scale: float) -> np.ndarray:
    """Causal multi-query attention over an FP8 pool: the definition of
    ``oracle.paged_attention_multi_query`` (sequence s's n rows are its last n
    positions; row i attends positions [0, L - n + i]) with K/V read as the
    dequantised codes e4m3(c) * scale.  Returns float64 ``[T, Hq, D]``."""
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
        K, V = gather_sequence_fp8(k_cache, v_cache, block_tables[s], L, block_size, k_scale,
                                   v_scale)
        for i in range(n):
            p = L - n + i
            row = starts[s] + i
            for g in range(Hkv):
                out[row, g * G:(g + 1) * G] = dense_attention(
                    qf[row, g * G:(g + 1) * G], K[:p + 1, g], V[:p + 1, g], sc)
    return out
