"""Checks that pin the oracle to things other than itself.

Each function returns a number (an error, or a count of mismatches) so the
same checks can be run against deliberately broken copies of the oracle in
``test_oracle_mutations.py``.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import brute
from oracle import oracle as O


def dense_sdpa_error(case, decode=None) -> float:
    """Max |oracle - SDPA| where SDPA runs in float64 on the generator's
    logical (never paged) K/V of each sequence.  Needs ``keep_logical``."""
    decode = decode or O.paged_attention_decode
    kc, vc = case.k_cache, case.v_cache
    if case.has_step:
        kc, vc = O.copy_blocks(case.copy_pairs, kc, vc)
        kc, vc = O.kv_cache_write(case.k_new, case.v_new, case.slot_mapping, kc, vc, case.block_size)
    got = decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                 case.block_size, case.dtype)
    G = case.num_q_heads // case.num_kv_heads
    err = 0.0
    for s in range(case.num_seqs):
        K = torch.from_numpy(O.to_f64(case.logical_k[s], case.dtype))  # [L, Hkv, D]
        V = torch.from_numpy(O.to_f64(case.logical_v[s], case.dtype))
        q = torch.from_numpy(O.to_f64(case.q[s], case.dtype))  # [Hq, D]
        if K.shape[0] == 0:
            ref = torch.zeros_like(q)
        else:
            Kh = K.permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()  # [Hq, L, D]
            Vh = V.permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[:, None, :], Kh, Vh, scale=float(np.float32(case.scale)))[:, 0, :]
        err = max(err, float(np.abs(got[s] - ref.numpy()).max()))
    return err


def brute_error(case, decode=None) -> float:
    """Max |oracle - pure-Python brute force| on the pool as given (no step)."""
    decode = decode or O.paged_attention_decode
    got = decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                 case.scale, case.block_size, case.dtype)
    ref = np.array(brute.decode(case.q.tolist(), case.k_cache.tolist(), case.v_cache.tolist(),
                                case.block_tables.tolist(), case.context_lens.tolist(),
                                float(case.scale), case.block_size, case.dtype))
    return float(np.abs(got - ref).max())


def one_token_mismatches(case, decode=None) -> int:
    """Sequences with one position must return that position's V exactly."""
    decode = decode or O.paged_attention_decode
    got = decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                 case.scale, case.block_size, case.dtype)
    G = case.num_q_heads // case.num_kv_heads
    bad = 0
    for s in range(case.num_seqs):
        if case.context_lens[s] != 1:
            continue
        p = case.block_tables[s, 0]
        for h in range(case.num_q_heads):
            v = O.to_f64(case.v_cache[p, h // G, 0], case.dtype)
            bad += int(not np.array_equal(got[s, h], v))
    return bad


def identical_keys_error(case, decode=None) -> float:
    """With every K row of a sequence equal, the weights are uniform and the
    output is the mean of V over the context."""
    decode = decode or O.paged_attention_decode
    kc = case.k_cache.copy()
    B = case.block_size
    for s in range(case.num_seqs):
        L = int(case.context_lens[s])
        if L == 0:
            continue
        p0 = case.block_tables[s, 0]
        row = kc[p0, :, 0].copy()
        for t in range(L):
            kc[case.block_tables[s, t // B], :, t % B] = row
    got = decode(case.q, kc, case.v_cache, case.block_tables, case.context_lens, case.scale,
                 B, case.dtype)
    G = case.num_q_heads // case.num_kv_heads
    err = 0.0
    for s in range(case.num_seqs):
        L = int(case.context_lens[s])
        if L == 0:
            continue
        V = np.stack([O.to_f64(case.v_cache[case.block_tables[s, t // B], :, t % B], case.dtype)
                      for t in range(L)])  # [L, Hkv, D]
        mean = V.mean(axis=0)
        for h in range(case.num_q_heads):
            err = max(err, float(np.abs(got[s, h] - mean[h // G]).max()))
    return err


def permutation_mismatches(case, decode=None, seed: int = 11) -> int:
    """Relabelling physical blocks (and the tables with them) must not change
    the output at all."""
    from workloads.generate import permute_pool
    decode = decode or O.paged_attention_decode
    a = decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
               case.scale, case.block_size, case.dtype)
    k2, v2, t2, _, _, _ = permute_pool(case, seed)
    b = decode(case.q, k2, v2, t2, case.context_lens, case.scale, case.block_size, case.dtype)
    return int((a.view(np.uint64) != b.view(np.uint64)).sum())
