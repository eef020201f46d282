"""The host-planned dispatch list of multi-query calls
(paged_attention_multi_query_plan), no GPU needed: every item of the launch
exactly once, longest first by the tokens each item attends, restated here
from the call's item numbering (item c < S * P is sequence c % S, partition
P - 1 - c / S; a prefix item of group i is sized by the group's longest
shared length), equal sizes in item order, items with no work last."""
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_cache_386_amd", "libpagedattn.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpagedattn.so not built")


def _expected(lens, groups, shared, S, P, ps, cap, ipg):
    L = np.minimum(np.maximum(np.asarray(lens, np.int64), 0), cap)
    ng = 0 if groups is None else len(groups)
    sh = (np.minimum(np.maximum(np.asarray(shared, np.int64), 0), L) & ~15) if ng else 0 * L
    sizes = []
    for c in range(S * P):
        s, p = c % S, (P - 1) - c // S
        nparts = min(-(-int(L[s]) // ps), P)
        if p >= max(nparts, 1) or (sh[s] > 0 and p < sh[s] // ps):
            sizes.append(-1)
        else:
            sizes.append(max(0, min(int(L[s]), p * ps + ps) - max(p * ps, int(sh[s]))))
    for i in range(ng):
        f, m = int(groups[i][0]), int(groups[i][1])
        longest = int(sh[f:f + min(m, 16)].max()) if m > 0 else 0
        sizes += [longest if longest > 0 else -1] * ipg
    sizes = np.array(sizes, np.int64)
    # longest first, equal sizes in item order
    return np.array(sorted(range(len(sizes)), key=lambda c: (-sizes[c], c)), np.int32)


@pytest.mark.parametrize("S,G,Hkv,maxq,ps,prefix", [
    (48, 4, 8, 2, 0, True),      # prefix items (8 rows per KV head)
    (48, 4, 8, 2, 512, True),    # and split partitions
    (48, 4, 8, 5, 0, True),      # 20 rows: the plain call, groups ignored
    (16, 4, 8, 512, 0, False),   # chunked prefill (row tiles)
    (40, 2, 8, 64, 128, False),
])
def test_plan_is_the_longest_first_permutation(S, G, Hkv, maxq, ps, prefix):
    import paged_kv_cache_386_amd as pa
    rng = np.random.default_rng(S + maxq + ps)
    B, MB = 16, 256
    lens = rng.integers(maxq, 3000, size=S)
    lens[:5] = [0, 1, maxq, 1024, 4096]
    groups = shared = None
    if prefix:
        groups = np.array([[0, 16], [16, 16], [32, 3], [40, 1]], np.int32)
        shared = np.zeros(S, np.int32)
        for f, m in groups.tolist():
            shared[f:f + m] = rng.integers(0, 1100, size=m)
        shared[17] = 5000  # past its context: clamped
    max_ctx = int(lens.max())
    kw = dict(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=128, block_size=B,
              max_blocks_per_seq=MB, max_query_len=maxq, max_context_len=max_ctx,
              kv_dtype=pa.PA_BF16, partition_size=ps)
    got = pa.multi_query_plan(lens, groups, shared, **kw)
    P = pa.multi_query_partitions(S, G * Hkv, Hkv, maxq, max_ctx, ps)
    pfx = prefix and maxq * G <= 8
    ipg = maxq * G if pfx else 0
    n = S * P + (ipg * len(groups) if pfx else 0)
    assert len(got) == n and np.array_equal(np.sort(got), np.arange(n))
    pst = MB * B if P <= 1 else (pa.partition_tokens(S, Hkv, max_ctx, ps) + 63) // 64 * 64 \
        if ps == 0 else ps
    want = _expected(lens, groups if pfx else None, shared, S, P, pst, MB * B, ipg)
    assert np.array_equal(got, want)


def test_plan_errors():
    import paged_kv_cache_386_amd as pa
    lib = pa.lib()
    lens = np.array([10, 20], np.int32)
    out = np.zeros(4, np.int32)
    args = [lens.ctypes.data, None, 0, None, 2, 8, 2, 128, 16, 4, 1, 64, pa.PA_BF16, 0]
    assert lib.paged_attention_multi_query_plan(*args, out.ctypes.data, 4) == 2
    assert lib.paged_attention_multi_query_plan(*args, out.ctypes.data, 1) == -2  # capacity
    assert lib.paged_attention_multi_query_plan(*args, None, 4) == -1
    bad = list(args)
    bad[12] = 99
    assert lib.paged_attention_multi_query_plan(*bad, out.ctypes.data, 4) == -3
    bad = list(args)
    bad[2] = 1  # a group on the prefix path without its arrays
    assert lib.paged_attention_multi_query_plan(*bad, out.ctypes.data, 4) == -1
    bad = list(args)
    bad[8] = 24  # block size not a power of two
    assert lib.paged_attention_multi_query_plan(*bad, out.ctypes.data, 4) == -2
