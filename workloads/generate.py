"""Seeded synthetic decode workloads shaped like the PagedAttention pages.

Every workload is a *decode step* over a paged KV pool:

* a pool of physical blocks, ``k_cache``/``v_cache`` of shape
  ``[num_blocks, num_kv_heads, block_size, head_dim]`` (head_dim contiguous),
  stored as float32 or as raw bfloat16 bit patterns (``uint16``);
* per-sequence block tables (logical block -> physical block id) and context
  lengths;
* optionally, the two cache edits a serving step makes before attention: the
  copy-on-write block copies (``copy_pairs``) and the write of each sequence's
  newest token (``slot_mapping`` with ``k_new``/``v_new``).

Sources for the structure (page titles as published):

* "vLLM 深度拆解：当大模型推理学会「分页注意力」..." section 2.1: fixed-size
  blocks (16 tokens), a block table mapping logical to scattered physical
  blocks, prefix blocks shared between requests; section 3.3: ``append_slot``
  writes into the current block until it is full.
* The devpress.csdn.net/amd vLLM walkthrough, "关键设计二：Copy-on-Write":
  forked children share the parent's blocks and copy the shared last block on
  their first append.
* "vLLM为何成为大模型推理的事实标准？" (PagedAttention section): 512-token
  pages are also used.

Two random streams are used so that the values of the logical tokens do not
depend on the pool's structure: ``default_rng(seed)`` draws lengths and the
pool permutation; ``default_rng([seed, 1])`` draws q, the per-sequence K/V (in
sequence order) and finally the newly generated tokens.  Values are N(0, 1)
float32, rounded to bfloat16 (round-to-nearest-even) for bf16 workloads.

Parity workloads (``poison=True``) fill every slot that decode must never read
with NaN and point unused block-table entries at a NaN-filled poison block.
Performance workloads (``poison=False``) fill those slots with zeros.

This module places logical tokens into the pool (the inverse of the
block-table lookup) because that is what defines the input; it holds none of
the attention arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BF16_QNAN = 0x7FC0
F32_QNAN_BITS = 0x7FC00000

CONFIG_NAMES = {
    0: "tiny-f32 (4 seqs, lens 1/17/33/100, 2q/2kv, d64, B16)",
    1: "llama7b-layer-bf16 (64 seqs, lens U[512,4096], 32q/32kv, d128, B16)",
    2: "gqa8b-prefix-bf16 (256 seqs, lognormal lens median 1024 cap 8192, 32q/8kv, d128, B16, 16-seq groups share a 1024-token prefix)",
    3: "longctx-splitk-bf16 (8 seqs x 32768, 64q/8kv, d128, B512 or B16, 512-token partitions)",
    4: "cb-step-bf16 (512 seqs, lens U[16,2048], 32q/8kv, d128, B16, 16 fork groups of 4, copy+write+decode)",
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16, nearest-even; return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return x if dtype == "f32" else bf16_bits_from_f32(x)


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) values in the storage form of ``dtype`` (float32, or the
    bfloat16 bit patterns of the rounded values), for callers that build
    their own sequences token by token."""
    return _draw(rng, shape, dtype)


def _storage(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


@dataclass
class Case:
    """One decode step's inputs.  All arrays are host numpy arrays."""

    name: str
    dtype: str  # "f32" or "bf16" (bf16 arrays hold uint16 bit patterns)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray  # int32 [S]; counts every token attended, incl. the new one
    block_tables: np.ndarray  # int32 [S, MB]; table used by decode (after copy-on-write)
    k_cache: np.ndarray  # [NB, Hkv, B, D] pool before the step's edits
    v_cache: np.ndarray
    q: np.ndarray  # [S, Hq, D]
    scale: np.float32
    poison_block: int  # physical id of the NaN block (or zero block when poison=False); -1 if none
    block_tables_pre: Optional[np.ndarray] = None  # table before copy-on-write (step workloads)
    copy_pairs: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), np.int32))
    slot_mapping: np.ndarray = field(default_factory=lambda: np.zeros((0,), np.int32))
    k_new: Optional[np.ndarray] = None  # [T, Hkv, D]
    v_new: Optional[np.ndarray] = None
    logical_k: Optional[List[np.ndarray]] = None  # per sequence [L, Hkv, D] after the step
    logical_v: Optional[List[np.ndarray]] = None
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def has_step(self) -> bool:
        return self.k_new is not None


class _Pool:
    def __init__(self, nb: int, B: int, hkv: int, d: int, dtype: str, poison: bool):
        st = _storage(dtype)
        shape = (nb, hkv, B, d)
        if poison:
            fill = F32_QNAN_BITS if dtype == "f32" else BF16_QNAN
            if dtype == "f32":
                self.k = np.full(shape, fill, np.uint32).view(np.float32)
                self.v = np.full(shape, fill, np.uint32).view(np.float32)
            else:
                self.k = np.full(shape, fill, st)
                self.v = np.full(shape, fill, st)
        else:
            self.k = np.zeros(shape, st)
            self.v = np.zeros(shape, st)
        self.B = B

    def put(self, blocks: np.ndarray, start: int, k: np.ndarray, v: np.ndarray) -> None:
        """Place a run of a sequence's logical tokens [start, start+len) given
        the physical id of each of its logical blocks."""
        if len(k) == 0:
            return
        t = np.arange(start, start + len(k))
        phys = blocks[t // self.B]
        off = t % self.B
        self.k[phys, :, off] = k  # k is [len, Hkv, D]
        self.v[phys, :, off] = v


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _scale_for(head_dim: int) -> np.float32:
    return np.float32(1.0 / np.sqrt(np.float64(head_dim)))


def make_private_case(name: str, lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      block_size: int, dtype: str, seed: int, *, pool_blocks: Optional[int] = None,
                      max_blocks_per_seq: Optional[int] = None, poison: bool = True,
                      keep_logical: bool = False, scale: Optional[float] = None,
                      rng: Optional[np.random.Generator] = None) -> Case:
    """Every sequence owns its blocks; physical ids are a seeded permutation of
    the pool handed out in sequence order.  Decode only (no cache edits)."""
    lens = np.asarray(lens, np.int64)
    S, B = len(lens), block_size
    rng = rng if rng is not None else np.random.default_rng(seed)
    vrng = np.random.default_rng([seed, 1])
    nblk = np.array([_cdiv(int(L), B) for L in lens], np.int64)
    used = int(nblk.sum())
    NB = pool_blocks if pool_blocks is not None else used + 1
    if NB < used:
        raise ValueError("pool too small")
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, int(nblk.max(initial=0)))
    perm = rng.permutation(NB).astype(np.int32)
    poison_id = int(perm[used]) if NB > used else -1
    tables = np.full((S, MB), max(poison_id, 0), np.int32)
    off = 0
    for s in range(S):
        tables[s, : nblk[s]] = perm[off: off + nblk[s]]
        off += nblk[s]
    pool = _Pool(NB, B, num_kv_heads, head_dim, dtype, poison)
    q = _draw(vrng, (S, num_q_heads, head_dim), dtype)
    lk, lv = [], []
    for s in range(S):
        k = _draw(vrng, (int(lens[s]), num_kv_heads, head_dim), dtype)
        v = _draw(vrng, (int(lens[s]), num_kv_heads, head_dim), dtype)
        pool.put(tables[s], 0, k, v)
        if keep_logical:
            lk.append(k)
            lv.append(v)
    return Case(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, block_size=B, context_lens=lens.astype(np.int32),
                block_tables=tables, k_cache=pool.k, v_cache=pool.v, q=q,
                scale=np.float32(scale) if scale is not None else _scale_for(head_dim),
                poison_block=poison_id,
                logical_k=lk if keep_logical else None, logical_v=lv if keep_logical else None)


def make_prefix_case(name: str, lens, group_size: int, prefix_len: int, num_q_heads: int,
                     num_kv_heads: int, head_dim: int, block_size: int, dtype: str, seed: int, *,
                     max_blocks_per_seq: Optional[int] = None, poison: bool = True,
                     keep_logical: bool = False, rng: Optional[np.random.Generator] = None) -> Case:
    """Groups of ``group_size`` consecutive sequences share the physical blocks of
    a common ``prefix_len``-token prefix, and each sequence appends one new token.

    ``lens`` are the context lengths after the append; sequence s holds history
    positions [0, n) with n = L-1 and writes its new token at position n.  Its
    logical block j < n // B maps to the group's prefix block j when j lies in
    the prefix, else to a private block.  The block holding position n is
    always private: when it lies inside the prefix and already holds history
    tokens (n % B != 0) it starts as the shared prefix block and the step copies
    it to a private block first (copy-on-write); otherwise it is a fresh block.
    """
    lens = np.asarray(lens, np.int64)
    S, B = len(lens), block_size
    if prefix_len % B:
        raise ValueError("prefix_len must be a multiple of block_size")
    if S % group_size:
        raise ValueError("num_seqs must be a multiple of group_size")
    if lens.min(initial=1) < 1:
        raise ValueError("a step workload needs L >= 1")
    rng = rng if rng is not None else np.random.default_rng(seed)
    vrng = np.random.default_rng([seed, 1])
    n_groups = S // group_size
    pblocks = prefix_len // B
    n = lens - 1
    jn = n // B
    # count physical blocks: prefix blocks per group, then private blocks per sequence
    priv_count = np.zeros(S, np.int64)
    for s in range(S):
        total = _cdiv(int(lens[s]), B)
        shared = min(int(jn[s]), pblocks)  # logical blocks before the new token's block that are prefix
        priv_count[s] = total - shared
    used = n_groups * pblocks + int(priv_count.sum())
    NB = used + 1
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else int(max(_cdiv(int(L), B) for L in lens))
    perm = rng.permutation(NB).astype(np.int32)
    poison_id = int(perm[used])
    prefix_ids = perm[: n_groups * pblocks].reshape(n_groups, pblocks)
    tables = np.full((S, MB), poison_id, np.int32)
    pre = np.full((S, MB), poison_id, np.int32)
    pairs = []
    cur = n_groups * pblocks
    for s in range(S):
        g = s // group_size
        total = _cdiv(int(lens[s]), B)
        shared = min(int(jn[s]), pblocks)
        tables[s, :shared] = prefix_ids[g, :shared]
        tables[s, shared:total] = perm[cur: cur + priv_count[s]]
        cur += priv_count[s]
        pre[s] = tables[s]
        if jn[s] < pblocks and n[s] % B != 0:
            pre[s, jn[s]] = prefix_ids[g, jn[s]]
            pairs.append((prefix_ids[g, jn[s]], tables[s, jn[s]]))
    pool = _Pool(NB, B, num_kv_heads, head_dim, dtype, poison)
    q = _draw(vrng, (S, num_q_heads, head_dim), dtype)
    pk, pv = [], []
    for g in range(n_groups):
        k = _draw(vrng, (prefix_len, num_kv_heads, head_dim), dtype)
        v = _draw(vrng, (prefix_len, num_kv_heads, head_dim), dtype)
        pool.put(prefix_ids[g], 0, k, v)
        pk.append(k)
        pv.append(v)
    hist_k, hist_v = [], []
    for s in range(S):
        extra = max(0, int(n[s]) - prefix_len)
        k = _draw(vrng, (extra, num_kv_heads, head_dim), dtype)
        v = _draw(vrng, (extra, num_kv_heads, head_dim), dtype)
        pool.put(tables[s], prefix_len, k, v)
        if keep_logical:
            hist_k.append(k)
            hist_v.append(v)
    k_new = _draw(vrng, (S, num_kv_heads, head_dim), dtype)
    v_new = _draw(vrng, (S, num_kv_heads, head_dim), dtype)
    slots = np.array([tables[s, jn[s]] * B + n[s] % B for s in range(S)], np.int32)
    lk = lv = None
    if keep_logical:
        lk, lv = [], []
        for s in range(S):
            g = s // group_size
            h = min(int(n[s]), prefix_len)
            lk.append(np.concatenate([pk[g][:h], hist_k[s], k_new[s: s + 1]]))
            lv.append(np.concatenate([pv[g][:h], hist_v[s], v_new[s: s + 1]]))
    return Case(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, block_size=B, context_lens=lens.astype(np.int32),
                block_tables=tables, k_cache=pool.k, v_cache=pool.v, q=q,
                scale=_scale_for(head_dim), poison_block=poison_id, block_tables_pre=pre,
                copy_pairs=np.array(pairs, np.int32).reshape(-1, 2), slot_mapping=slots,
                k_new=k_new, v_new=v_new, logical_k=lk, logical_v=lv)


def make_fork_case(name: str, lens, n_groups: int, fork_n: int, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, block_size: int, dtype: str, seed: int, *,
                   max_blocks_per_seq: Optional[int] = None, poison: bool = True,
                   keep_logical: bool = False, rng: Optional[np.random.Generator] = None) -> Case:
    """A continuous-batching step: every sequence appends one token; the first
    ``n_groups * fork_n`` sequences form fork groups of ``fork_n`` siblings.

    Siblings were forked from one parent, so before the step they share every
    block, including the partly filled last one (the group's length is nudged
    so that the new token never starts a fresh block).  On append, the first
    ``fork_n - 1`` siblings copy the shared last block into a spare block of
    their own; the last sibling is then the only holder and writes in place.
    Other sequences own all their blocks.
    """
    lens = np.asarray(lens, np.int64).copy()
    S, B = len(lens), block_size
    nf = n_groups * fork_n
    if nf > S:
        raise ValueError("more forked sequences than sequences")
    if lens.min(initial=1) < 1:
        raise ValueError("a step workload needs L >= 1")
    for g in range(n_groups):
        L = int(lens[g * fork_n])
        if (L - 1) % B == 0:
            L += 1
        lens[g * fork_n:(g + 1) * fork_n] = L
    rng = rng if rng is not None else np.random.default_rng(seed)
    vrng = np.random.default_rng([seed, 1])
    n = lens - 1
    jn = n // B
    counts = []
    for s in range(S):
        if s < nf:
            if s % fork_n == 0:
                counts.append(int(jn[s]) + 1 + (fork_n - 1))
        else:
            counts.append(_cdiv(int(lens[s]), B))
    used = int(sum(counts))
    NB = used + 1
    MB = max_blocks_per_seq if max_blocks_per_seq is not None else int(max(_cdiv(int(L), B) for L in lens))
    perm = rng.permutation(NB).astype(np.int32)
    poison_id = int(perm[used])
    tables = np.full((S, MB), poison_id, np.int32)
    pre = np.full((S, MB), poison_id, np.int32)
    pairs = []
    cur = 0
    for s in range(S):
        if s < nf:
            if s % fork_n == 0:
                nb = int(jn[s]) + 1
                shared = perm[cur: cur + nb]
                spares = perm[cur + nb: cur + nb + fork_n - 1]
                cur += nb + fork_n - 1
                for i in range(fork_n):
                    pre[s + i, :nb] = shared
                    tables[s + i, :nb] = shared
                    if i < fork_n - 1:
                        tables[s + i, nb - 1] = spares[i]
                        pairs.append((shared[nb - 1], spares[i]))
        else:
            nb = _cdiv(int(lens[s]), B)
            tables[s, :nb] = perm[cur: cur + nb]
            pre[s, :nb] = tables[s, :nb]
            cur += nb
    pool = _Pool(NB, B, num_kv_heads, head_dim, dtype, poison)
    q = _draw(vrng, (S, num_q_heads, head_dim), dtype)
    hist_k: List[np.ndarray] = [None] * S  # type: ignore
    hist_v: List[np.ndarray] = [None] * S  # type: ignore
    for s in range(S):
        if s < nf and s % fork_n:
            hist_k[s], hist_v[s] = hist_k[s - s % fork_n], hist_v[s - s % fork_n]
            continue
        k = _draw(vrng, (int(n[s]), num_kv_heads, head_dim), dtype)
        v = _draw(vrng, (int(n[s]), num_kv_heads, head_dim), dtype)
        pool.put(pre[s], 0, k, v)
        hist_k[s], hist_v[s] = k, v
    k_new = _draw(vrng, (S, num_kv_heads, head_dim), dtype)
    v_new = _draw(vrng, (S, num_kv_heads, head_dim), dtype)
    slots = np.array([tables[s, jn[s]] * B + n[s] % B for s in range(S)], np.int32)
    lk = lv = None
    if keep_logical:
        lk = [np.concatenate([hist_k[s], k_new[s: s + 1]]) for s in range(S)]
        lv = [np.concatenate([hist_v[s], v_new[s: s + 1]]) for s in range(S)]
    return Case(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, block_size=B, context_lens=lens.astype(np.int32),
                block_tables=tables, k_cache=pool.k, v_cache=pool.v, q=q,
                scale=_scale_for(head_dim), poison_block=poison_id, block_tables_pre=pre,
                copy_pairs=np.array(pairs, np.int32).reshape(-1, 2), slot_mapping=slots,
                k_new=k_new, v_new=v_new, logical_k=lk, logical_v=lv)


def make_aliased_case(name: str, lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      block_size: int, dtype: str, seed: int, n_alias: int, *,
                      poison: bool = True) -> Case:
    """A decode-only case whose block tables share blocks in arbitrary
    patterns, not just prefixes: starting from private blocks, ``n_alias``
    seeded times a sequence's logical block j is pointed at the physical block
    another sequence holds at the same logical position (both blocks full in
    both sequences, so no poisoned slot is ever attended).  Blocks of the
    second sequence that lose their last reference stay in the pool unread.
    The attended values follow from the tables alone."""
    c = make_private_case(name, lens, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
                          seed, poison=poison)
    rng = np.random.default_rng([seed, 2])
    B = block_size
    L = c.context_lens.astype(np.int64)
    S = len(L)
    tables = c.block_tables.copy()
    for _ in range(n_alias):
        a, b = (int(x) for x in rng.integers(0, S, size=2))
        full = int(min(L[a], L[b]) // B)
        if a == b or full == 0:
            continue
        lo = int(rng.integers(0, full))
        hi = int(rng.integers(lo + 1, full + 1))
        tables[b, lo:hi] = tables[a, lo:hi]
    c.block_tables = tables
    return c


def config_lengths(config: int, rng: np.random.Generator) -> np.ndarray:
    """Context lengths of the five named workloads (drawn first from the
    structure stream)."""
    if config == 0:
        return np.array([1, 17, 33, 100], np.int64)
    if config == 1:
        return rng.integers(512, 4097, size=64)
    if config == 2:
        x = rng.lognormal(mean=np.log(1024.0), sigma=1.0, size=256)
        return np.clip(np.rint(x), 1, 8192).astype(np.int64)
    if config == 3:
        return np.full(8, 32768, np.int64)
    if config == 4:
        return rng.integers(16, 2049, size=512)
    raise ValueError(f"unknown config {config}")


def make_case(config: int, *, seed: Optional[int] = None, poison: bool = True,
              block_size: Optional[int] = None, keep_logical: bool = False) -> Case:
    """Build one of the five named workloads.  ``seed`` defaults to the config
    index.  ``block_size`` only applies to config 3 (512 or 16)."""
    seed = config if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = config_lengths(config, rng)
    if config == 0:
        c = make_private_case("cfg0", lens, 2, 2, 64, 16, "f32", seed, pool_blocks=64,
                              poison=poison, keep_logical=keep_logical, scale=0.125, rng=rng)
    elif config == 1:
        c = make_private_case("cfg1", lens, 32, 32, 128, 16, "bf16", seed,
                              max_blocks_per_seq=256, poison=poison, keep_logical=keep_logical, rng=rng)
    elif config == 2:
        c = make_prefix_case("cfg2", lens, 16, 1024, 32, 8, 128, 16, "bf16", seed,
                             max_blocks_per_seq=512, poison=poison, keep_logical=keep_logical, rng=rng)
    elif config == 3:
        B = 512 if block_size is None else block_size
        c = make_private_case(f"cfg3-B{B}", lens, 64, 8, 128, B, "bf16", seed,
                              max_blocks_per_seq=32768 // B, poison=poison,
                              keep_logical=keep_logical, rng=rng)
    elif config == 4:
        c = make_fork_case("cfg4", lens, 16, 4, 32, 8, 128, 16, "bf16", seed,
                           max_blocks_per_seq=128, poison=poison, keep_logical=keep_logical, rng=rng)
    else:
        raise ValueError(f"unknown config {config}")
    c.description = CONFIG_NAMES[config]
    return c


def permute_pool(case: Case, seed: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, Optional[np.ndarray], np.ndarray, np.ndarray]:
    """Relabel physical blocks by a seeded permutation pi: block p moves to pi[p].
    Returns (k_cache', v_cache', block_tables', block_tables_pre', copy_pairs', slot_mapping')."""
    rng = np.random.default_rng([seed, 7])
    NB = case.num_blocks
    pi = rng.permutation(NB).astype(np.int32)
    k2 = np.empty_like(case.k_cache)
    v2 = np.empty_like(case.v_cache)
    k2[pi] = case.k_cache
    v2[pi] = case.v_cache
    t2 = pi[case.block_tables]
    tp2 = pi[case.block_tables_pre] if case.block_tables_pre is not None else None
    pairs2 = pi[case.copy_pairs] if case.copy_pairs.size else case.copy_pairs.copy()
    B = case.block_size
    sm = case.slot_mapping
    sm2 = np.where(sm >= 0, pi[np.maximum(sm, 0) // B] * B + np.maximum(sm, 0) % B, sm).astype(np.int32)
    return k2, v2, t2, tp2, pairs2, sm2


# ---------------------------------------------------------------- multi-query

def settle_step(case: Case) -> Case:
    """The same workload with its step already taken: the copy pairs applied
    (whole blocks, in list order) and each new token placed at its slot, so
    that the pool holds every position [0, L) of every sequence."""
    if not case.has_step:
        return case
    k, v = case.k_cache.copy(), case.v_cache.copy()
    for src, dst in case.copy_pairs.reshape(-1, 2).tolist():
        k[dst] = k[src]
        v[dst] = v[src]
    B = case.block_size
    for i, slot in enumerate(case.slot_mapping.tolist()):
        if slot >= 0:
            k[slot // B, :, slot % B] = case.k_new[i]
            v[slot // B, :, slot % B] = case.v_new[i]
    return Case(name=case.name, dtype=case.dtype, num_q_heads=case.num_q_heads,
                num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, block_size=B,
                context_lens=case.context_lens, block_tables=case.block_tables, k_cache=k,
                v_cache=v, q=case.q, scale=case.scale, poison_block=case.poison_block,
                logical_k=case.logical_k, logical_v=case.logical_v,
                description=case.description)


def subset_sequences(case: Case, keep) -> Case:
    """The workload restricted to the sequences ``keep`` (same pool)."""
    keep = np.asarray(keep)
    return Case(name=case.name, dtype=case.dtype, num_q_heads=case.num_q_heads,
                num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                block_size=case.block_size, context_lens=case.context_lens[keep],
                block_tables=case.block_tables[keep], k_cache=case.k_cache,
                v_cache=case.v_cache, q=case.q[keep], scale=case.scale,
                poison_block=case.poison_block,
                logical_k=[case.logical_k[i] for i in keep] if case.logical_k else None,
                logical_v=[case.logical_v[i] for i in keep] if case.logical_v else None,
                description=case.description)


@dataclass
class MultiQueryCase:
    """Several query tokens per sequence (a prompt chunk, or tokens to verify)
    over the pool of ``base``: sequence s owns query rows ``query_start[s] ..
    query_start[s+1] - 1``, which are its last cached positions.  ``base.q``
    is not used."""

    name: str
    base: Case
    q: np.ndarray             # [T, Hq, D]
    query_start: np.ndarray   # int32 [S + 1]
    description: str = ""

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start)

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return int(ql.max()) if ql.size else 0


def make_multi_query_case(base: Case, q_lens, seed: int, name: str = "",
                          description: str = "") -> MultiQueryCase:
    """Chunks of ``q_lens[s]`` query tokens (each at most the sequence's
    context length) drawn N(0, 1) from ``default_rng([seed, 2])``."""
    q_lens = np.asarray(q_lens, np.int64)
    if q_lens.shape != base.context_lens.shape or (q_lens < 0).any() or \
            (q_lens > base.context_lens).any():
        raise ValueError("each chunk must fit in its sequence's context")
    qs = np.zeros(len(q_lens) + 1, np.int32)
    qs[1:] = np.cumsum(q_lens)
    vrng = np.random.default_rng([seed, 2])
    q = _draw(vrng, (int(qs[-1]), base.num_q_heads, base.head_dim), base.dtype)
    return MultiQueryCase(name=name or base.name, base=base, q=q, query_start=qs,
                          description=description)


MULTI_QUERY_NAMES = {
    "chunked-prefill": ("chunked-prefill-bf16 (16 seqs, contexts U[1024,8192], a 512-token "
                        "prompt chunk each, 32q/8kv, d128, B16)"),
    "spec-verify": ("spec-verify-bf16 (256 seqs, lognormal contexts median 1024 cap 8192, "
                    "5 tokens to verify each, 32q/8kv, d128, B16, 16-seq groups share a "
                    "1024-token prefix)"),
}


def make_multi_query_workload(name: str, *, seed: int = 7, poison: bool = True,
                              scale_down: int = 1) -> MultiQueryCase:
    """The two multi-query workloads at full size (``scale_down`` > 1 keeps
    every ``scale_down``-th sequence, for quick checks)."""
    rng = np.random.default_rng(seed)
    if name == "chunked-prefill":
        lens = rng.integers(1024, 8192 + 1, size=16)[::scale_down]
        base = make_private_case(name, lens, 32, 8, 128, 16, "bf16", seed, poison=poison,
                                 rng=rng)
        q_lens = np.full(len(lens), 512)
    elif name == "spec-verify":
        lens = np.minimum(np.round(np.exp(rng.normal(np.log(1024.0), 1.0, size=256))), 8192)
        lens = np.maximum(lens, 5).astype(np.int64)
        keep = np.arange(0, 256, scale_down)
        base = settle_step(make_prefix_case(name, lens, 16, 1024, 32, 8, 128, 16, "bf16", seed,
                                            poison=poison, rng=rng))
        base = subset_sequences(base, keep)
        q_lens = np.full(len(keep), 5)
    else:
        raise ValueError(name)
    return make_multi_query_case(base, q_lens, seed, name, MULTI_QUERY_NAMES[name])


# ---------------------------------------------------------------- FP8 pools

E4M3_QNAN = 0x7F


@dataclass
class Fp8Case:
    """A workload whose pool holds FP8 (E4M3) codes: ``base`` gives the
    structure (tables, lengths, copy pairs, slots), the bfloat16 queries and
    the bfloat16 new tokens (to be quantised by the write); ``k8``/``v8``
    replace its pool, with one fp32 scale per cache."""

    base: Case
    k8: np.ndarray  # uint8 [NB, Hkv, B, D]
    v8: np.ndarray
    k_scale: np.float32
    v_scale: np.float32

    @property
    def name(self) -> str:
        return self.base.name


def draw_e4m3_codes(rng: np.random.Generator, shape, max_exponent_field: int = 9) -> np.ndarray:
    """Random E4M3 codes: random sign and mantissa, exponent field uniform in
    [0, max_exponent_field] (so never the NaN code; magnitudes below
    2^(max_exponent_field - 6))."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    e = rng.integers(0, max_exponent_field + 1, size=shape, dtype=np.uint8) << 3
    m = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign | e | m).astype(np.uint8)


def make_fp8_case(base: Case, seed: int, k_scale: float = 0.25, v_scale: float = 0.5) -> Fp8Case:
    """The same workload over an FP8 pool: every slot gets a random code from
    ``default_rng([seed, 3])``, except the slots that hold the NaN poison in
    ``base`` (never read), which get the E4M3 NaN code."""
    if base.dtype != "bf16":
        raise ValueError("FP8 workloads take bfloat16 queries and new tokens")
    rng = np.random.default_rng([seed, 3])
    k8 = draw_e4m3_codes(rng, base.k_cache.shape)
    v8 = draw_e4m3_codes(rng, base.v_cache.shape)
    k8[base.k_cache == BF16_QNAN] = E4M3_QNAN
    v8[base.v_cache == BF16_QNAN] = E4M3_QNAN
    return Fp8Case(base=base, k8=k8, v8=v8, k_scale=np.float32(k_scale),
                   v_scale=np.float32(v_scale))


# ---------------------------------------------------------------- INT8 pools

@dataclass
class Int8Case:
    """A workload over an INT8 pool (signed codes in [-127, 127], one fp32
    scale per cache); ``base`` as for Fp8Case."""

    base: Case
    k8: np.ndarray  # int8 [NB, Hkv, B, D]
    v8: np.ndarray
    k_scale: np.float32
    v_scale: np.float32

    @property
    def name(self) -> str:
        return self.base.name


def make_int8_case(base: Case, seed: int, k_scale: float = 0.02,
                   v_scale: float = 0.03) -> Int8Case:
    """The same workload over an INT8 pool: every slot gets a code uniform in
    [-127, 127] from ``default_rng([seed, 4])``; slots that ``base`` poisons
    (never read) get -128, a code no write produces."""
    if base.dtype != "bf16":
        raise ValueError("INT8 workloads take bfloat16 queries and new tokens")
    rng = np.random.default_rng([seed, 4])
    k8 = rng.integers(-127, 128, size=base.k_cache.shape, dtype=np.int8)
    v8 = rng.integers(-127, 128, size=base.v_cache.shape, dtype=np.int8)
    k8[base.k_cache == BF16_QNAN] = -128
    v8[base.v_cache == BF16_QNAN] = -128
    return Int8Case(base=base, k8=k8, v8=v8, k_scale=np.float32(k_scale),
                    v_scale=np.float32(v_scale))
