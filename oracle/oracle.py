"""Plain CPU oracle for PagedAttention decode -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP library:
no kernels, headers, helpers or constants.  Everything is computed in float64
from the exact input values (bfloat16 inputs are widened bit-exactly).

What is computed, and where the pages say so:

* KV cache per token and head, appended each step and attended by the new
  query: "vLLM 深度拆解：当大模型推理学会「分页注意力」..." (page at
  chenxutan.com), section 1.1.
* Paging: a sequence's KV lives in fixed-size blocks reached through a block
  table that maps logical block numbers to scattered physical block numbers:
  same page, section 2.1; the devpress.csdn.net/amd vLLM walkthrough, sections
  "关键设计一：分页管理" and "核心代码拆解：PagedAttention 的 CUDA Kernel 是怎么读取 KV
  Cache 的" (translate the logical block through the table, read K, take the
  scaled dot with q, then softmax and the weighted sum of V "as in standard
  attention").
* Token write-back after generation and appending into the current block:
  chenxutan.com page, sections 3.1 and 3.3.
* Copying a shared block before a forked sequence appends to it: the
  devpress.csdn.net/amd walkthrough, section "关键设计二：Copy-on-Write".

Readings taken where the pages are silent (each also listed in the design
notes):

* cache layout ``[num_blocks, num_kv_heads, block_size, head_dim]``: the
  order of the key/value caches of the kernel in the devpress.csdn.net/amd
  walkthrough's "核心代码拆解" section (blocks, heads, block_size, head_size);
* query head h reads KV head ``h // (num_q_heads // num_kv_heads)``;
* a sequence attends exactly its positions ``[0, context_len)``; a context of
  length 0 produces zeros;
* softmax is base e with the maximum subtracted; no mask, bias or cap;
* slot of position t = ``table[t // B] * B + t % B``; a negative slot is
  skipped by the write;
* the split-K merge (not on the pages) is the log-sum-exp combination of
  per-partition maxima, sums and normalised outputs.
* multi-query attention (a chunk of prompt tokens, or tokens to verify, per
  sequence: the chenxutan.com page, sections 2.3 (prefill computes the KV of
  all input tokens at once), 4.3 and 5.1 (chunked prefill slices a long
  prompt into pieces run beside decode) and 5.4 (speculative decoding: the
  main model checks several guessed tokens in one pass)): the chunk's tokens
  are the sequence's last ``n`` cached positions, and chunk token i, at
  position ``p = L - n + i``, attends positions ``[0, p]`` (causal, as in
  standard attention); nothing else changes.

Parity is pinned (``tests/test_oracle_pins.py``) against: the library SDPA on
the densely gathered tokens, pure-Python brute force, block-id permutation
invariance, the 1-token and identical-key closed forms, block-size invariance,
and the pages' worked block-table examples.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly: a bfloat16 is the
    high half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(f"unknown dtype {dtype}")


def slot_of(table_row: Sequence[int], pos: int, block_size: int) -> int:
    """Physical slot of logical position ``pos``: the block table gives the
    physical block of logical block ``pos // B``; the token sits at offset
    ``pos % B`` inside it."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def gather_sequence(k_cache: np.ndarray, v_cache: np.ndarray, table_row: np.ndarray,
                    context_len: int, block_size: int, dtype: str,
                    kv_head: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of one sequence in logical order, as float64.

    The pool is ``[num_blocks, num_kv_heads, block_size, head_dim]``.
    Returns ``[L, Hkv, D]`` arrays, or ``[L, D]`` for one KV head.  Positions
    at or beyond ``context_len`` are never touched, nor are table entries past
    ``ceil(context_len / B)``."""
    L = int(context_len)
    pos = np.arange(L)
    phys = np.asarray(table_row)[pos // block_size]
    off = pos % block_size
    if kv_head is None:
        k = k_cache[phys, :, off]  # advanced indices first: [L, Hkv, D]
        v = v_cache[phys, :, off]
    else:
        k = k_cache[phys, kv_head, off]
        v = v_cache[phys, kv_head, off]
    return to_f64(k, dtype), to_f64(v, dtype)


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Single-query attention over contiguous K, V (float64).

    ``q``: [G, D] (the query heads sharing one KV head); ``K``, ``V``: [L, D].
    x = scale * K q; w = exp(x - max x); out = (w^T V) / sum(w).  L = 0 gives
    zeros."""
    q = np.atleast_2d(q)
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]), np.float64)
    x = np.float64(scale) * (K @ q.T)  # [L, G]
    m = x.max(axis=0, keepdims=True)
    w = np.exp(x - m)
    return (w.T @ V) / w.sum(axis=0)[:, None]


def _group(num_q_heads: int, num_kv_heads: int) -> int:
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return num_q_heads // num_kv_heads


def paged_attention_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                           block_size: int, dtype: str) -> np.ndarray:
    """out[s, h] = attention of q[s, h] over the K/V of sequence s's first
    ``context_lens[s]`` positions, gathered through ``block_tables[s]``.
    Returns float64 ``[S, Hq, D]``."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    qf = to_f64(q, dtype)
    out = np.zeros((S, Hq, D), np.float64)
    for s in range(S):
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], int(context_lens[s]),
                               block_size, dtype)
        for g in range(Hkv):
            out[s, g * G:(g + 1) * G] = dense_attention(qf[s, g * G:(g + 1) * G], K[:, g], V[:, g],
                                                        np.float64(np.float32(scale)))
    return out


def paged_attention_decode_rows(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                                block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                                block_size: int, dtype: str,
                                rows: Iterable[Tuple[int, int]]) -> np.ndarray:
    """The same as ``paged_attention_decode`` for selected (seq, q_head) pairs
    only; returns ``[len(rows), D]``."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    qf = to_f64(q, dtype)
    res = []
    for s, h in rows:
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], int(context_lens[s]),
                               block_size, dtype, kv_head=h // G)
        res.append(dense_attention(qf[s, h], K, V, np.float64(np.float32(scale)))[0])
    return np.array(res, np.float64).reshape(-1, D)


def paged_attention_decode_partitioned(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                                       block_tables: np.ndarray, context_lens: np.ndarray,
                                       scale: float, block_size: int, dtype: str,
                                       partition_size: int) -> np.ndarray:
    """Split-K form: each partition of ``partition_size`` positions yields its
    own maximum m_p, sum l_p = sum exp(x - m_p) and normalised output o_p; the
    partitions are then merged in ascending order with weights
    ``l_p * exp(m_p - max_p m_p)``.  Equal to ``paged_attention_decode`` up to
    rounding."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    qf = to_f64(q, dtype)
    sc = np.float64(np.float32(scale))
    out = np.zeros((S, Hq, D), np.float64)
    for s in range(S):
        L = int(context_lens[s])
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], L, block_size, dtype)
        for h in range(Hq):
            g = h // G
            parts: List[Tuple[float, float, np.ndarray]] = []
            for start in range(0, L, partition_size):
                Kp = K[start:start + partition_size, g]
                Vp = V[start:start + partition_size, g]
                x = sc * (Kp @ qf[s, h])
                m = x.max()
                w = np.exp(x - m)
                lsum = w.sum()
                parts.append((m, lsum, (w @ Vp) / lsum))
            if not parts:
                continue
            M = max(p[0] for p in parts)
            num = np.zeros(D, np.float64)
            den = 0.0
            for m, lsum, o in parts:
                wgt = lsum * np.exp(m - M)
                num += wgt * o
                den += wgt
            out[s, h] = num / den
    return out


def kv_cache_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, k_cache: np.ndarray,
                   v_cache: np.ndarray, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the caches with token i's K/V rows (all KV heads)
    stored at slot ``slot_mapping[i]``: block ``slot // B``, offset
    ``slot % B``.  Negative slots are skipped.  The copy is bit-exact."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        kc[slot // block_size, :, slot % block_size] = k[i]
        vc[slot // block_size, :, slot % block_size] = v[i]
    return kc, vc


def copy_blocks(pairs: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the caches after copying whole block ``src`` onto block
    ``dst`` for each (src, dst) pair, in list order."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc


def paged_attention_multi_query(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                                block_tables: np.ndarray, context_lens: np.ndarray,
                                query_start: np.ndarray, scale: float, block_size: int,
                                dtype: str) -> np.ndarray:
    """Several query tokens per sequence over the paged pool, causal.

    ``q`` is ``[T, Hq, D]``: sequence s owns rows ``query_start[s] ..
    query_start[s+1] - 1`` (n_s of them), which are its last n_s cached
    positions.  Row ``query_start[s] + i`` sits at position
    ``p = context_lens[s] - n_s + i`` and attends positions ``[0, p]``
    through the block table, each query head h reading KV head h // G.
    Returns float64 ``[T, Hq, D]``."""
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    qf = to_f64(q, dtype)
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
        K, V = gather_sequence(k_cache, v_cache, block_tables[s], L, block_size, dtype)
        for i in range(n):
            p = L - n + i
            row = starts[s] + i
            for g in range(Hkv):
                out[row, g * G:(g + 1) * G] = dense_attention(
                    qf[row, g * G:(g + 1) * G], K[:p + 1, g], V[:p + 1, g], sc)
    return out
