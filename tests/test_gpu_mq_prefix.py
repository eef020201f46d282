"""Multi-query attention with shared prefixes read once per group
(paged_attention_multi_query_prefix) through the C ABI against the oracle
(needs an MI355X).

The groups only change which reads are shared, so the oracle is plain causal
multi-query attention on the same tables.  The prefix items serve calls with
at most 8 (token, head) rows per sequence and KV head; above that the call
is the plain one, as it is over 8-bit pools.  Covered: the
speculative-verification structure at full size with 2 tokens per sequence
(prefix items over bf16; the plain call over FP8 and INT8) and with 5 (the
plain call); every output element; prefix workloads at G = 1,
2, 4 and 8 on both sides of the threshold, several partition and block
sizes; hand-made groups whose shared lengths reach past some query tokens'
positions (a whole context shared), a member sharing nothing, chunks of no
tokens; an empty group list; index checking of bad groups."""
import numpy as np
import pytest
import torch

from oracle import fp8, int8
from oracle import oracle as O
from workloads import (make_fp8_case, make_int8_case, make_multi_query_case,
                       make_multi_query_workload, make_prefix_case, make_private_case)
from workloads.generate import settle_step

from gpu_helpers import REGRESS, TOL, max_err, say, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()
    yield
    torch.cuda.synchronize()


def host_groups(base, min_shared=16):
    """Groups of at most 16 members (the multi-query prefix limit) from the
    host tables."""
    import paged_kv_cache_386_amd as pa
    G = base.num_q_heads // base.num_kv_heads
    # pa.prefix_groups allows 64 / G members; the multi-query items take 16
    g, sh = pa.prefix_groups(base.block_tables, base.context_lens, base.block_size,
                             base.num_q_heads, base.num_kv_heads, min_shared)
    if G < 4:
        out = []
        for f, m in g.tolist():
            for s in range(f, f + m, 16):
                out.append([s, min(16, f + m - s)])
        g = np.array(out, np.int32).reshape(-1, 2)
    return g, sh


def _check(c, groups, shared):
    b = c.base
    NB, B = b.num_blocks, b.block_size
    qs = c.query_start
    assert qs[0] == 0 and (np.diff(qs) >= 0).all()
    for s, L in enumerate(b.context_lens.tolist()):
        nb = -(-L // B)
        assert ((b.block_tables[s, :nb] >= 0) & (b.block_tables[s, :nb] < NB)).all()
        assert qs[s + 1] - qs[s] <= L
    G = b.num_q_heads // b.num_kv_heads
    assert int(np.diff(qs).max()) * G <= 64
    for f, m in np.asarray(groups).reshape(-1, 2).tolist():
        assert 1 <= m <= 16 and f + m <= b.num_seqs
        # members name the same blocks below the shorter shared length
        for i in range(f, f + m):
            for j in range(f, f + m):
                k = min(shared[i], shared[j]) // B
                assert np.array_equal(b.block_tables[i, :k], b.block_tables[j, :k])


def run_mq_prefix(c, groups, shared, ps=0, pool=None, scales=(1.0, 1.0)):
    import paged_kv_cache_386_amd as pa
    _check(c, groups, shared)
    b = c.base
    if pool is None:
        kc, vc = to_torch(b.k_cache, b.dtype), to_torch(b.v_cache, b.dtype)
    else:
        kc, vc = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in pool)
    out = torch.full((c.num_tokens, b.num_q_heads, b.head_dim), 7.0, dtype=torch.float32,
                     device="cuda")
    g = torch.from_numpy(np.ascontiguousarray(groups, np.int32).reshape(-1, 2)).cuda()
    sh = torch.from_numpy(np.ascontiguousarray(shared, np.int32)).cuda()
    pa.paged_attention_multi_query_prefix(
        to_torch(c.q, "bf16"), kc, vc, torch.from_numpy(np.ascontiguousarray(b.block_tables)).cuda(),
        torch.from_numpy(b.context_lens).cuda(), torch.from_numpy(c.query_start).cuda(), g, sh,
        float(b.scale), out, max_query_len=c.max_query_len,
        max_context_len=int(b.context_lens.max()), k_scale=scales[0], v_scale=scales[1],
        partition_size=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(c):
    b = c.base
    return O.paged_attention_multi_query(c.q, b.k_cache, b.v_cache, b.block_tables,
                                         b.context_lens, c.query_start, b.scale, b.block_size,
                                         b.dtype)


def compare(c, groups, shared, name, ps=0):
    say(f"{name}: S={c.base.num_seqs} T={c.num_tokens} G={c.base.num_q_heads // c.base.num_kv_heads}"
        f" B={c.base.block_size} groups={len(groups)} ps={ps}")
    got = run_mq_prefix(c, groups, shared, ps)
    err = max_err(got, oracle(c))
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"{name}: max abs err {err}"
    return got


@pytest.mark.parametrize("G,Hkv,maxq", [(4, 8, 2), (4, 2, 2), (8, 4, 1), (8, 1, 1),
                                         (2, 4, 4), (1, 8, 8), (4, 8, 1),
                                         (4, 8, 5), (1, 8, 16), (4, 8, 8), (8, 4, 4),
                                         (2, 4, 13), (1, 8, 12), (4, 8, 9)])
@pytest.mark.parametrize("ps", [0, -1, 64, 512])
def test_prefix_workloads(G, Hkv, maxq, ps):
    """Prefix groups of 16 sequences (lengths below, at and past the 1024-token
    prefix; the step settled: copies and new tokens in place), 1 to maxq
    query tokens per sequence."""
    rng = np.random.default_rng(G * 100 + maxq)
    lens = rng.integers(maxq + 1, 3000, size=48)
    lens[:4] = [1024, 1030, 700, 1025]
    base = settle_step(make_prefix_case(f"mqp-{G}-{maxq}", lens, 16, 1024, G * Hkv, Hkv, 128, 16,
                                        "bf16", G + maxq))
    q_lens = [min(int(L), maxq - (i % 3 == 1 and maxq > 1)) for i, L in
              enumerate(base.context_lens)]
    c = make_multi_query_case(base, q_lens, G + maxq)
    g, sh = host_groups(base)
    assert len(g) > 0
    compare(c, g, sh, f"mq prefix G={G} maxq={maxq}", ps)


@pytest.mark.parametrize("B", [4, 16, 64])
def test_block_sizes(B):
    lens = [1100, 1100, 1040, 900, 2000, 1024, 1200, 1500]
    base = settle_step(make_prefix_case(f"mqp-B{B}", lens, 4, 1024, 32, 8, 128, B, "bf16", B))
    c = make_multi_query_case(base, [2, 1, 2, 1, 2, 2, 1, 2], B)
    g, sh = host_groups(base)
    compare(c, g, sh, f"mq prefix B={B}", 0)
    compare(c, g, sh, f"mq prefix B={B}", 64)


def _shared_block_case(lens, G, Hkv, B, seed, shared_blocks):
    c = make_private_case(f"mqp-edge-{seed}", lens, G * Hkv, Hkv, 128, B, "bf16", seed)
    tb = c.block_tables.copy()
    for s, k in enumerate(shared_blocks):
        tb[s, :k] = tb[0, :k]
    c.block_tables = tb
    return c


@pytest.mark.parametrize("G,Hkv", [(4, 2), (8, 1), (2, 2)])
@pytest.mark.parametrize("ps", [0, -1, 64, 512])
def test_hand_made_groups(G, Hkv, ps):
    """Shared lengths reaching past query positions (sequence 0 shares its
    whole 700-token context, sequence 3 its 512), a member sharing nothing, a
    chunk of no tokens, lengths off the 16-token grid."""
    B = 16
    lens = [700, 700, 33, 512, 640, 100, 257, 900, 64, 700]
    blocks = [44, 44, 3, 32, 40, 7, 17, 43, 4, 44]
    base = _shared_block_case(lens, G, Hkv, B, 70 + G, blocks)
    sh = np.array([700, 690, 33, 512, 600, 0, 250, 688, 64, 17], np.int32)
    maxq = 8 // G
    q_lens = [min(L, maxq) for L in lens]
    q_lens[5] = 0
    q_lens[2] = 1
    c = make_multi_query_case(base, q_lens, 70 + G)
    compare(c, [[0, 10]], sh, f"mq hand-made G={G}", ps)
    # the same call with no groups is the plain one
    got = run_mq_prefix(c, np.zeros((0, 2), np.int32), sh, ps)
    assert max_err(got, oracle(c)) <= REGRESS["bf16"]


def test_sparse_groups():
    """Groups of one and two members, and sequences in no group."""
    base = _shared_block_case([300, 300, 200, 50, 400], 4, 2, 16, 81, [18, 18, 12, 3, 0])
    c = make_multi_query_case(base, [2, 2, 1, 2, 2], 81)
    sh = np.array([290, 288, 192, 48, 0], np.int32)
    compare(c, [[0, 2], [2, 1], [3, 1]], sh, "mq sparse groups", 0)
    compare(c, [[0, 2], [2, 1], [3, 1]], sh, "mq sparse groups", 64)


@pytest.mark.parametrize("kind,n", [("bf16", 2), ("fp8", 2), ("int8", 2), ("bf16", 5)])
def test_full_size_spec_verify(kind, n):
    """The speculative-verification structure at full size (256 sequences,
    16-sequence groups sharing 1024-token prefixes) with n tokens per
    sequence: every output element against the oracle."""
    b = make_multi_query_workload("spec-verify").base
    c = make_multi_query_case(b, np.minimum(b.context_lens, n), 7)
    g, sh = host_groups(b)
    say(f"spec-verify prefix full size ({kind}, {n} tokens): S={b.num_seqs} groups={len(g)}")
    if kind == "bf16":
        got = run_mq_prefix(c, g, sh)
        ref = oracle(c)
    else:
        c8 = make_fp8_case(b, 7) if kind == "fp8" else make_int8_case(b, 7)
        got = run_mq_prefix(c, g, sh, pool=(c8.k8, c8.v8),
                            scales=(float(c8.k_scale), float(c8.v_scale)))
        fn = (fp8.paged_attention_multi_query_fp8 if kind == "fp8"
              else int8.paged_attention_multi_query_int8)
        ref = fn(c.q, c8.k8, c8.v8, b.block_tables, b.context_lens, c.query_start, b.scale,
                 b.block_size, "bf16", c8.k_scale, c8.v_scale)
    assert np.isfinite(got).all()
    err = max_err(got, ref)
    say(f"spec-verify prefix ({kind}): all {got.size} outputs, max abs err {err:.3e}")
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], err


def test_index_check_rejects_bad_groups():
    """With index checking on, a group of 17 members (above the multi-query
    limit), a group running past the batch and a shared length past the
    blocks the members have in common return PA_ERR_INDEX; valid groups
    run."""
    import paged_kv_cache_386_amd as pa
    blocks = [18] * 17
    blocks[3] = 10  # sequence 3 shares only its first 160 tokens
    base = _shared_block_case([300] * 17, 4, 2, 16, 91, blocks)
    c = make_multi_query_case(base, [2] * 17, 91)
    good = np.full(17, 288, np.int32)
    good[3] = 160
    past = good.copy()
    past[3] = 288
    was = pa.index_check()
    pa.set_index_check(True)
    try:
        for groups, sh in (([[0, 17]], good), ([[1, 17]], good), ([[0, 16], [16, 1]], past)):
            with pytest.raises(pa.PagedAttnError) as e:
                run_mq_prefix_unchecked(c, groups, sh)
            assert e.value.status == pa.PA_ERR_INDEX
        got = run_mq_prefix(c, [[0, 16], [16, 1]], good)
        assert max_err(got, oracle(c)) <= REGRESS["bf16"]
    finally:
        pa.set_index_check(was)


def run_mq_prefix_unchecked(c, groups, shared):
    """The call without the host-side consistency asserts (for inputs the
    library's index check must reject before launching anything)."""
    import paged_kv_cache_386_amd as pa
    b = c.base
    out = torch.full((c.num_tokens, b.num_q_heads, b.head_dim), 7.0, dtype=torch.float32,
                     device="cuda")
    pa.paged_attention_multi_query_prefix(
        to_torch(c.q, "bf16"), to_torch(b.k_cache, b.dtype), to_torch(b.v_cache, b.dtype),
        torch.from_numpy(np.ascontiguousarray(b.block_tables)).cuda(),
        torch.from_numpy(b.context_lens).cuda(), torch.from_numpy(c.query_start).cuda(),
        torch.from_numpy(np.asarray(groups, np.int32).reshape(-1, 2)).cuda(),
        torch.from_numpy(shared).cuda(), float(b.scale), out, max_query_len=c.max_query_len,
        max_context_len=int(b.context_lens.max()))
    torch.cuda.synchronize()
