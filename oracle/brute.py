"""Pure-Python brute force for tiny paged-decode inputs -- TEST INFRASTRUCTURE.

No numpy arithmetic: values are read element by element, widened to Python
floats (float64) and combined with ``math.exp`` in plain loops, following the
walk through the block table described on the devpress.csdn.net/amd vLLM
walkthrough ("核心代码拆解" section): for each sequence and head, visit the
logical blocks in order, translate each to its physical block, take the
scaled dot of q with every K row up to the context length, then softmax and
the weighted sum of V.  Used only to pin the numpy oracle on small cases.
"""
from __future__ import annotations

import math
import struct
from typing import List


def _value(x, dtype: str) -> float:
    if dtype == "f32":
        return float(x)
    # bfloat16 bits: the high 16 bits of an IEEE binary32
    return struct.unpack("<f", struct.pack("<I", (int(x) & 0xFFFF) << 16))[0]


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, block_size: int,
           dtype: str) -> List[List[List[float]]]:
    S = len(q)
    Hq = len(q[0])
    D = len(q[0][0])
    Hkv = len(k_cache[0])  # pool [blocks][kv_heads][block_size][head_dim]
    G = Hq // Hkv
    sc = float(scale)
    out = []
    for s in range(S):
        L = int(context_lens[s])
        rows = []
        for h in range(Hq):
            g = h // G
            scores = []
            kv_pos = []
            nblocks = (L + block_size - 1) // block_size
            for j in range(nblocks):
                phys = int(block_tables[s][j])
                for o in range(block_size):
                    if j * block_size + o >= L:
                        break
                    dot = 0.0
                    for d in range(D):
                        dot += _value(q[s][h][d], dtype) * _value(k_cache[phys][g][o][d], dtype)
                    scores.append(sc * dot)
                    kv_pos.append((phys, o))
            if not scores:
                rows.append([0.0] * D)
                continue
            m = max(scores)
            w = [math.exp(x - m) for x in scores]
            tot = sum(w)
            acc = [0.0] * D
            for wi, (phys, o) in zip(w, kv_pos):
                for d in range(D):
                    acc[d] += wi * _value(v_cache[phys][g][o][d], dtype)
            rows.append([a / tot for a in acc])
        out.append(rows)
    return out


def multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                block_size: int, dtype: str) -> List[List[List[float]]]:
    """Causal multi-query attention in plain loops: for sequence s, its query
    rows query_start[s] .. query_start[s+1]-1 are its last positions; row i
    of the chunk (position p = L - n + i) scores every cached position t <= p
    found by walking the block table, then takes softmax and the weighted sum
    of V."""
    T = len(q)
    Hq = len(q[0])
    D = len(q[0][0])
    Hkv = len(k_cache[0])
    G = Hq // Hkv
    sc = float(scale)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for s in range(len(query_start) - 1):
        first, last = int(query_start[s]), int(query_start[s + 1])
        n = last - first
        L = int(context_lens[s])
        for i in range(n):
            p = L - n + i
            for h in range(Hq):
                g = h // G
                scores, where = [], []
                for t in range(p + 1):
                    phys = int(block_tables[s][t // block_size])
                    o = t % block_size
                    dot = 0.0
                    for d in range(D):
                        dot += _value(q[first + i][h][d], dtype) * \
                            _value(k_cache[phys][g][o][d], dtype)
                    scores.append(sc * dot)
                    where.append((phys, o))
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                tot = sum(w)
                acc = [0.0] * D
                for wi, (phys, o) in zip(w, where):
                    for d in range(D):
                        acc[d] += wi * _value(v_cache[phys][g][o][d], dtype)
                out[first + i][h] = [a / tot for a in acc]
    return out
