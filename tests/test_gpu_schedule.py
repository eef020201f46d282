"""The longest-first dispatch list of decode and multi-query (needs an MI355X).

A launch of more than 1024 workgroups first sorts its (sequence, partition)
items by token count; the decode kernels then take their item from that list.
The order may change timing only: every item must run exactly once, so the
outputs with the list must equal, bit for bit, those of the fixed order (a
workspace with room for the partials but not the list), and both must match
the oracle.  The output buffer is filled with NaN before each run, so an item
that never ran shows up.  With shared prefixes the list also holds the
groups' prefix items, sized by the longest shared length they walk.
"""
import numpy as np
import pytest
import torch

from oracle import fp8 as F8
from oracle import oracle as O
from workloads import make_private_case
from workloads.generate import make_fp8_case

from gpu_helpers import TOL, DeviceCase, max_err, say, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()
    yield
    torch.cuda.synchronize()


def _mixed_lengths(S, seed, top):
    """Mixed lengths with the edge cases: empty, one token, one short of, at
    and one past a 16-token chunk, and a few long ones."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, top // 4, size=S)
    lens[:6] = [0, 1, 15, 16, 17, top]
    lens[rng.integers(6, S, size=S // 16)] = rng.integers(top // 2, top + 1, size=S // 16)
    return lens


def _partials_bytes(S, Hq, Hkv, D, max_ctx, ps):
    import paged_kv_cache_386_amd as pa
    P = pa.num_partitions(S, Hkv, max_ctx, ps)
    return S * Hq * P * (D + 2) * 4 if P > 1 else 0, P


def _run_both(run, S, Hq, Hkv, D, max_ctx, ps):
    """Outputs with the full workspace (dispatch list) and with only the
    partials (fixed order)."""
    import paged_kv_cache_386_amd as pa
    full = pa.workspace_size(S, Hq, Hkv, D, max_ctx, ps)
    partial, P = _partials_bytes(S, Hq, Hkv, D, max_ctx, ps)
    assert S * Hkv * P > 1024, "the case must be large enough for the list"
    assert full == partial + 4 * S * P
    outs = []
    for nbytes in (full, partial):
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda") if nbytes else None
        outs.append(run(ws))
        torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("dtype,D,G,Hkv,ps", [
    ("bf16", 128, 1, 16, 0),     # vector kernel, no split
    ("bf16", 128, 1, 16, 256),   # vector kernel, split
    ("bf16", 128, 4, 8, 0),      # matrix-core kernel, no split
    ("bf16", 128, 4, 8, 512),    # matrix-core kernel, split
    ("bf16", 128, 8, 8, 256),
    ("f32", 64, 2, 16, 128),     # fp32 vector kernel, split
])
def test_list_equals_fixed_order(dtype, D, G, Hkv, ps):
    S = 160
    top = 1200 if dtype == "bf16" else 400
    lens = _mixed_lengths(S, 11 + G, top)
    c = make_private_case("schedule", lens, G * Hkv, Hkv, D, 16, dtype, 5)
    say(f"schedule: {dtype} D={D} G={G} Hkv={Hkv} ps={ps} S={S} max_ctx={c.max_context_len}")
    dc = DeviceCase(c)

    def run(ws):
        dc.out.fill_(float("nan"))
        return dc.run_decode(ps, workspace=ws).cpu().numpy()

    with_list, fixed = _run_both(run, S, c.num_q_heads, Hkv, D, c.max_context_len, ps)
    assert np.array_equal(with_list.view(np.uint32), fixed.view(np.uint32))
    ref = O.paged_attention_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                   c.scale, c.block_size, c.dtype)
    err = max_err(with_list, ref)
    assert err <= TOL[dtype], f"max abs err {err}"


def test_list_equals_fixed_order_fp8():
    import paged_kv_cache_386_amd as pa
    S, Hkv, G, D, ps = 160, 8, 4, 128, 512
    lens = _mixed_lengths(S, 23, 1500)
    c8 = make_fp8_case(make_private_case("schedule-fp8", lens, G * Hkv, Hkv, D, 16, "bf16", 6), 6)
    b = c8.base
    say(f"schedule fp8: S={S} ps={ps} max_ctx={b.max_context_len}")
    q = to_torch(b.q, "bf16")
    k8 = torch.from_numpy(c8.k8).cuda()
    v8 = torch.from_numpy(c8.v8).cuda()
    tables = torch.from_numpy(b.block_tables).cuda()
    lens_d = torch.from_numpy(b.context_lens).cuda()
    out = torch.empty(b.q.shape, dtype=torch.float32, device="cuda")

    def run(ws):
        out.fill_(float("nan"))
        pa.paged_attention_decode_fp8(q, k8, v8, tables, lens_d, float(b.scale),
                                      float(c8.k_scale), float(c8.v_scale), out,
                                      max_context_len=b.max_context_len, partition_size=ps,
                                      workspace=ws)
        return out.cpu().numpy()

    with_list, fixed = _run_both(run, S, G * Hkv, Hkv, D, b.max_context_len, ps)
    assert np.array_equal(with_list.view(np.uint32), fixed.view(np.uint32))
    rows = [(s, h) for s in range(0, S, 7) for h in (0, G * Hkv - 1)]
    ref = F8.paged_attention_decode_fp8(b.q, c8.k8, c8.v8, b.block_tables, b.context_lens,
                                        b.scale, b.block_size, "bf16", c8.k_scale, c8.v_scale,
                                        rows=rows)
    got = np.stack([with_list[s, h] for s, h in rows])
    err = max_err(got, ref)
    assert err <= TOL["bf16"], f"max abs err {err}"


@pytest.mark.parametrize("S,G,Hkv,max_q,ps", [
    (160, 4, 8, 5, 256),    # decode walk (20 rows per KV head, two column sets), split
    (160, 4, 8, 5, -1),     # decode walk, no split
    (80, 4, 8, 40, 0),      # row tiles of 128 rows, no split
    (40, 2, 8, 64, 128),    # row tiles of 64 rows, split
])
def test_multi_query_list_equals_fixed_order(S, G, Hkv, max_q, ps):
    import paged_kv_cache_386_amd as pa
    from workloads import make_multi_query_case
    lens = np.maximum(_mixed_lengths(S, 31 + max_q, 1100), max_q)
    lens[0] = max_q  # a chunk that is the whole context
    rng = np.random.default_rng(max_q)
    q_lens = rng.integers(0, max_q + 1, size=S)
    q_lens[:3] = [max_q, 0, 1]
    base = make_private_case("schedule-mq", lens, G * Hkv, Hkv, 128, 16, "bf16", 8)
    c = make_multi_query_case(base, q_lens, 8)
    T, Hq, D = c.num_tokens, base.num_q_heads, base.head_dim
    max_ctx = int(base.context_lens.max())
    say(f"schedule mq: S={S} G={G} Hkv={Hkv} max_q={max_q} ps={ps} T={T} max_ctx={max_ctx}")
    P = pa.multi_query_partitions(S, Hq, Hkv, max_q, max_ctx, ps)
    full = pa.multi_query_workspace_size(S, T, Hq, Hkv, D, max_q, max_ctx, ps)
    partial = T * Hq * P * (D + 2) * 4 if P > 1 else 0
    assert full == partial + 4 * S * P, "the case must be large enough for the list"
    args = [to_torch(c.q, "bf16"), to_torch(base.k_cache, "bf16"), to_torch(base.v_cache, "bf16"),
            torch.from_numpy(base.block_tables).cuda(), torch.from_numpy(base.context_lens).cuda(),
            torch.from_numpy(c.query_start).cuda(), float(base.scale)]
    out = torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")
    outs = []
    for nbytes in (full, partial):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
        out.fill_(float("nan"))
        pa.paged_attention_multi_query(*args, out, max_query_len=max_q, max_context_len=max_ctx,
                                       partition_size=ps, workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    ref = O.paged_attention_multi_query(c.q, base.k_cache, base.v_cache, base.block_tables,
                                        base.context_lens, c.query_start, base.scale,
                                        base.block_size, base.dtype)
    err = max_err(outs[0], ref)
    assert err <= TOL["bf16"], f"max abs err {err}"


@pytest.mark.parametrize("S,Hkv,ps,top", [(256, 8, 0, 8192), (160, 8, 512, 1500), (600, 2, 0, 900)])
def test_list_is_longest_first_permutation(S, Hkv, ps, top):
    """The list in the workspace (after the partials) holds every (sequence,
    partition) item once, in non-increasing size class (tokens >> shift, the
    classes 2^shift tokens wide with fewer than 512 of them over a
    partition), items past a sequence's last partition at the end, listed
    as ~c (negative) so that their workgroups exit at once."""
    import paged_kv_cache_386_amd as pa
    G, D = 4, 128
    lens = _mixed_lengths(S, 41 + S, top)
    c = make_private_case("schedule-list", lens, G * Hkv, Hkv, D, 16, "bf16", 9)
    say(f"schedule list: S={S} Hkv={Hkv} ps={ps} max_ctx={c.max_context_len}")
    dc = DeviceCase(c)
    full = pa.workspace_size(S, G * Hkv, Hkv, D, c.max_context_len, ps)
    partial, P = _partials_bytes(S, G * Hkv, Hkv, D, c.max_context_len, ps)
    assert full == partial + 4 * S * P
    ws = torch.empty(full, dtype=torch.uint8, device="cuda")
    dc.run_decode(ps, workspace=ws)
    torch.cuda.synchronize()
    listed = ws[partial:].cpu().numpy().view(np.int32)
    order = np.where(listed < 0, ~listed, listed)
    assert np.array_equal(np.sort(order), np.arange(S * P))
    cap = c.block_tables.shape[1] * c.block_size
    tokens_per_part = pa.partition_tokens(S, Hkv, c.max_context_len, ps) if P > 1 else cap
    shift = 0
    while (tokens_per_part >> shift) >= 512:
        shift += 1
    s = order % S
    p = (P - 1) - order // S
    L = np.minimum(c.context_lens.astype(np.int64)[s], cap)
    nparts = np.minimum((L + tokens_per_part - 1) // tokens_per_part, P)
    tok = np.minimum(L, (p + 1) * tokens_per_part) - p * tokens_per_part
    key = np.where(p < np.maximum(nparts, 1), tok >> shift, -1)
    assert (np.diff(key) <= 0).all(), "not longest first"
    assert np.array_equal(listed < 0, key < 0), "empty items are the negative entries"


@pytest.mark.parametrize("ps", [512, 0])
def test_multi_query_prefix_list(ps):
    """A multi-query call with shared prefixes (2 tokens per sequence, G = 4:
    prefix items): its list holds the sequence items and the groups' prefix
    items once each, longest first -- a prefix item sized by its group's
    longest shared length, a sequence item by its private positions in its
    partition -- with empty items negative; and the outputs with the list
    equal, bit for bit, those of the fixed order."""
    import paged_kv_cache_386_amd as pa
    from workloads import make_multi_query_case, make_prefix_case
    from workloads.generate import settle_step
    S, G, Hkv, D, max_q = 160, 4, 8, 128, 2
    rng = np.random.default_rng(61)
    lens = rng.integers(3, 3000, size=S)
    lens[:4] = [1024, 1030, 700, 2]
    base = settle_step(make_prefix_case("schedule-mqp", lens, 16, 1024, G * Hkv, Hkv, D, 16,
                                        "bf16", 61))
    q_lens = np.minimum(base.context_lens, max_q)
    q_lens[5] = 0
    c = make_multi_query_case(base, q_lens, 61)
    g, sh = pa.prefix_groups(base.block_tables, base.context_lens, base.block_size,
                             G * Hkv, Hkv, 16)
    assert len(g) > 0 and (g[:, 1] <= 16).all()
    T, Hq = c.num_tokens, G * Hkv
    max_ctx = int(base.context_lens.max())
    P = pa.multi_query_partitions(S, Hq, Hkv, max_q, max_ctx, ps)
    ipg = -(-16 * max_q * G // 16)
    n_items = S * P + ipg * len(g)
    full = pa.multi_query_prefix_workspace_size(S, T, Hq, Hkv, D, max_q, max_ctx, ps, len(g),
                                                pa.PA_BF16)
    partial = T * Hq * (P + 1) * (D + 2) * 4
    assert full == partial + 4 * n_items, "the case must be large enough for the list"
    say(f"schedule mq prefix: S={S} P={P} groups={len(g)} items={n_items}")
    args = [to_torch(c.q, "bf16"), to_torch(base.k_cache, "bf16"), to_torch(base.v_cache, "bf16"),
            torch.from_numpy(base.block_tables).cuda(), torch.from_numpy(base.context_lens).cuda(),
            torch.from_numpy(c.query_start).cuda(), torch.from_numpy(g).cuda(),
            torch.from_numpy(sh).cuda(), float(base.scale)]
    out = torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")
    outs, listed = [], None
    for nbytes in (full, partial):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        out.fill_(float("nan"))
        pa.paged_attention_multi_query_prefix(*args, out, max_query_len=max_q,
                                              max_context_len=max_ctx, partition_size=ps,
                                              workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        if nbytes == full:
            listed = ws[partial:].cpu().numpy().view(np.int32).copy()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    # the list planned on the host: the same outputs, bit for bit
    plan = pa.multi_query_plan(base.context_lens, g, sh, num_q_heads=Hq, num_kv_heads=Hkv,
                               head_dim=D, block_size=base.block_size,
                               max_blocks_per_seq=base.block_tables.shape[1],
                               max_query_len=max_q, max_context_len=max_ctx,
                               kv_dtype=pa.PA_BF16, partition_size=ps)
    assert len(plan) == n_items
    out.fill_(float("nan"))
    pa.paged_attention_multi_query_prefix(*args, out, max_query_len=max_q, max_context_len=max_ctx,
                                          partition_size=ps,
                                          workspace=torch.empty(partial, dtype=torch.uint8,
                                                                device="cuda"),
                                          dispatch=torch.from_numpy(plan).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), outs[0].view(np.uint32))
    ref = O.paged_attention_multi_query(c.q, base.k_cache, base.v_cache, base.block_tables,
                                        base.context_lens, c.query_start, base.scale,
                                        base.block_size, base.dtype)
    assert max_err(outs[0], ref) <= TOL["bf16"]
    # the list: a permutation, longest first by the restated sizes
    order = np.where(listed < 0, ~listed, listed)
    assert np.array_equal(np.sort(order), np.arange(n_items))
    cap = base.block_tables.shape[1] * base.block_size
    pst = pa.partition_tokens(S, Hkv, max_ctx, ps) if P > 1 else cap
    if P > 1:
        pst = -(-pst // 64) * 64 if ps == 0 else ps
    shift = 0
    while (pst >> shift) >= 512:
        shift += 1
    L = np.minimum(np.maximum(base.context_lens.astype(np.int64), 0), cap)
    she = np.minimum(np.maximum(sh.astype(np.int64), 0), L) & ~15
    key = []
    for it in order.tolist():
        if it < S * P:
            s, p = it % S, (P - 1) - it // S
            nparts = min(-(-int(L[s]) // pst), P)
            if p >= max(nparts, 1) or p < she[s] // pst:
                key.append(-1)
                continue
            tok = max(0, min(int(L[s]), p * pst + pst) - max(p * pst, int(she[s])))
        else:
            f, m = g[(it - S * P) // ipg].tolist()
            tok = int(she[f:f + min(m, 16)].max())
            if tok == 0:
                key.append(-1)
                continue
        key.append(min(tok >> shift, 511))
    key = np.array(key)
    assert (np.diff(key) <= 0).all(), "not longest first"
    assert np.array_equal(listed < 0, key < 0), "empty items are the negative entries"


@pytest.mark.parametrize("S,G,Hkv,max_q,ps", [
    (160, 4, 8, 5, 256),    # decode walk, split
    (80, 4, 8, 40, 0),      # row tiles
    (40, 2, 8, 64, 128),    # row tiles, split
])
def test_multi_query_planned_list(S, G, Hkv, max_q, ps):
    """A list planned on the host (paged_attention_multi_query_plan, passed
    through the prefix entry with no groups) gives the device-sorted call's
    outputs bit for bit; a list holding an entry outside the launch skips it
    (that item's rows keep what they held)."""
    import paged_kv_cache_386_amd as pa
    from workloads import make_multi_query_case
    lens = np.maximum(_mixed_lengths(S, 51 + max_q, 1100), max_q)
    rng = np.random.default_rng(max_q + 7)
    q_lens = rng.integers(0, max_q + 1, size=S)
    q_lens[:2] = [max_q, 1]
    base = make_private_case("schedule-mq-plan", lens, G * Hkv, Hkv, 128, 16, "bf16", 12)
    c = make_multi_query_case(base, q_lens, 12)
    T, Hq, D = c.num_tokens, base.num_q_heads, base.head_dim
    max_ctx = int(base.context_lens.max())
    say(f"schedule mq plan: S={S} G={G} Hkv={Hkv} max_q={max_q} ps={ps}")
    args = [to_torch(c.q, "bf16"), to_torch(base.k_cache, "bf16"), to_torch(base.v_cache, "bf16"),
            torch.from_numpy(base.block_tables).cuda(), torch.from_numpy(base.context_lens).cuda(),
            torch.from_numpy(c.query_start).cuda()]
    out = torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")
    out.fill_(float("nan"))
    pa.paged_attention_multi_query(*args, float(base.scale), out, max_query_len=max_q,
                                   max_context_len=max_ctx, partition_size=ps)
    torch.cuda.synchronize()
    sorted_out = out.cpu().numpy()
    plan = pa.multi_query_plan(base.context_lens, None, None, num_q_heads=Hq, num_kv_heads=Hkv,
                               head_dim=D, block_size=16,
                               max_blocks_per_seq=base.block_tables.shape[1],
                               max_query_len=max_q, max_context_len=max_ctx,
                               kv_dtype=pa.PA_BF16, partition_size=ps)
    P = pa.multi_query_partitions(S, Hq, Hkv, max_q, max_ctx, ps)
    assert np.array_equal(np.sort(plan), np.arange(S * P))
    out.fill_(float("nan"))
    pa.paged_attention_multi_query_prefix(*args, None, None, float(base.scale), out,
                                          max_query_len=max_q, max_context_len=max_ctx,
                                          partition_size=ps,
                                          dispatch=torch.from_numpy(plan).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), sorted_out.view(np.uint32))
    # sequence 0's items replaced by an entry past the launch: its rows are
    # left as they were, every other row is the same
    P0 = [i for i, e in enumerate(plan.tolist()) if e % S == 0]
    bad = plan.copy()
    bad[P0] = S * P + 5
    out.fill_(7.0)
    pa.paged_attention_multi_query_prefix(*args, None, None, float(base.scale), out,
                                          max_query_len=max_q, max_context_len=max_ctx,
                                          partition_size=ps,
                                          dispatch=torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    r0 = slice(int(c.query_start[0]), int(c.query_start[1]))
    rest = slice(int(c.query_start[1]), T)
    if P == 1:
        assert (got[r0] == 7.0).all()
    assert np.array_equal(got[rest].view(np.uint32), sorted_out[rest].view(np.uint32))
