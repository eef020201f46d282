"""Index checking, the library's debug mode (needs an MI355X).

With checking on, a call whose indices are out of range -- a block-table
entry outside the pool among the entries a sequence uses, a context length
above max_context_len, a bad query_start, a slot or a copy-pair id outside
the pool -- returns PA_ERR_INDEX and launches nothing (the output and the
caches keep their contents); entries a sequence never reads may hold
anything.  Valid inputs give the same bits as with checking off.  Every bad
input here is also memory-safe without the check: the kernels clamp block
ids into the pool, bound context lengths by the table row and skip slots and
pairs outside the pool.
"""
import numpy as np
import pytest
import torch

from workloads import make_multi_query_case, make_private_case

from gpu_helpers import DeviceCase, say, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _checking():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_386_amd as pa
    pa.lib()
    was = pa.index_check()
    pa.set_index_check(True)
    yield
    pa.set_index_check(was)
    torch.cuda.synchronize()


def _expect_index_error(fn):
    import paged_kv_cache_386_amd as pa
    with pytest.raises(pa.PagedAttnError) as e:
        fn()
    assert e.value.status == pa.PA_ERR_INDEX


def _case():
    c = make_private_case("idx", [1, 17, 40, 100, 300], 16, 4, 128, 16, "bf16", 3)
    return c, DeviceCase(c)


@pytest.mark.parametrize("ps", [0, 64])
def test_valid_decode_is_unchanged(ps):
    import paged_kv_cache_386_amd as pa
    c, dc = _case()
    say(f"index check: valid decode ps={ps}")
    checked = dc.run_decode(ps).clone()
    pa.set_index_check(False)
    try:
        plain = dc.run_decode(ps).clone()
    finally:
        pa.set_index_check(True)
    torch.cuda.synchronize()
    assert torch.equal(checked.view(torch.int32), plain.view(torch.int32))


@pytest.mark.parametrize("bad", ["past_pool", "negative", "long_context"])
def test_bad_decode_index_launches_nothing(bad):
    c, dc = _case()
    tables = c.block_tables.copy()
    lens = c.context_lens.copy()
    if bad == "past_pool":
        tables[3, 2] = c.num_blocks          # a used entry (L = 100 uses 7)
    elif bad == "negative":
        tables[4, 18] = -5                   # the last used entry of L = 300
    else:
        lens[2] = c.max_context_len + 1      # above the host bound
    say(f"index check: bad decode ({bad})")
    d = DeviceCase(c, tables=tables)
    d.context_lens = torch.from_numpy(lens).cuda()
    d.out.fill_(7.0)
    _expect_index_error(lambda: d.run_decode(0))
    torch.cuda.synchronize()
    assert (d.out == 7.0).all()


def test_unused_table_entries_may_hold_anything():
    c, dc = _case()
    tables = c.block_tables.copy()
    tables[0, 1:] = -1                      # L = 1 uses entry 0 only
    tables[3, 7:] = c.num_blocks + 100      # L = 100 uses entries 0..6
    say("index check: junk in unused entries")
    ref = dc.run_decode(0).clone()
    got = DeviceCase(c, tables=tables).run_decode(0)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_fp8_decode_checks_tables():
    import paged_kv_cache_386_amd as pa
    c, dc = _case()
    tables = c.block_tables.copy()
    tables[1, 1] = c.num_blocks + 3
    k8 = torch.zeros(c.k_cache.shape, dtype=torch.uint8, device="cuda")
    v8 = torch.zeros_like(k8)
    out = torch.full(c.q.shape, 7.0, dtype=torch.float32, device="cuda")
    say("index check: bad FP8 decode")
    _expect_index_error(lambda: pa.paged_attention_decode_fp8(
        dc.q, k8, v8, torch.from_numpy(tables).cuda(), dc.context_lens, float(c.scale), 1.0, 1.0,
        out, max_context_len=c.max_context_len))
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("bad", [None, "decreasing", "past_tokens", "chunk_over_context",
                                 "chunk_over_max"])
def test_multi_query_checks(bad):
    import paged_kv_cache_386_amd as pa
    base = make_private_case("idx-mq", [40, 129, 300], 8, 2, 128, 16, "bf16", 5)
    mq = make_multi_query_case(base, [5, 10, 20], 5)
    qs = mq.query_start.copy()
    max_q = mq.max_query_len
    if bad == "decreasing":
        qs[1], qs[2] = qs[2], qs[1]
    elif bad == "past_tokens":
        qs[-1] = mq.num_tokens + 1
    elif bad == "chunk_over_context":
        base.context_lens[0] = 3             # a 5-token chunk over 3 positions
    elif bad == "chunk_over_max":
        max_q = 10                           # the third chunk has 20 rows
    say(f"index check: multi-query ({bad})")
    out = torch.full((mq.num_tokens, base.num_q_heads, base.head_dim), 7.0,
                     dtype=torch.float32, device="cuda")

    def run():
        pa.paged_attention_multi_query(
            to_torch(mq.q, "bf16"), to_torch(base.k_cache, "bf16"), to_torch(base.v_cache, "bf16"),
            torch.from_numpy(base.block_tables).cuda(), torch.from_numpy(base.context_lens).cuda(),
            torch.from_numpy(qs).cuda(), float(base.scale), out, max_query_len=max_q,
            max_context_len=int(base.context_lens.max()))

    if bad is None:
        run()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
    else:
        _expect_index_error(run)
        torch.cuda.synchronize()
        assert (out == 7.0).all()


def test_write_and_copy_check_their_indices():
    import paged_kv_cache_386_amd as pa
    c, dc = _case()
    NB, B = c.num_blocks, c.block_size
    T = 4
    k = torch.ones((T, c.num_kv_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")
    before = dc.k_cache.clone()
    say("index check: kv_cache_write / copy_blocks")
    # negative slots are padding; a slot past the pool is an error
    ok = torch.tensor([-1, 0, 5, NB * B - 1], dtype=torch.int32, device="cuda")
    pa.kv_cache_write(k, k, ok, dc.k_cache, dc.v_cache)
    torch.cuda.synchronize()
    dc.k_cache.copy_(before)
    bad = torch.tensor([-1, 0, NB * B, 3], dtype=torch.int32, device="cuda")
    _expect_index_error(lambda: pa.kv_cache_write(k, k, bad, dc.k_cache, dc.v_cache))
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache.view(torch.int16), before.view(torch.int16))
    pairs = torch.tensor([[0, 1], [2, NB]], dtype=torch.int32, device="cuda")
    _expect_index_error(lambda: pa.copy_blocks(pairs, dc.k_cache, dc.v_cache))
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache.view(torch.int16), before.view(torch.int16))
    pairs = torch.tensor([[0, 1], [-1, 2]], dtype=torch.int32, device="cuda")
    _expect_index_error(lambda: pa.copy_blocks(pairs, dc.k_cache, dc.v_cache))
    good = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device="cuda")
    pa.copy_blocks(good, dc.k_cache, dc.v_cache)
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache[1].view(torch.int16), before[0].view(torch.int16))
    assert np.array_equal(dc.k_cache[3].view(torch.int16).cpu().numpy(),
                          before[2].view(torch.int16).cpu().numpy())


def test_append_checks_pairs_and_slots():
    """kv_cache_append makes both checks: a bad pair or a bad slot returns
    PA_ERR_INDEX with nothing launched; valid indices run."""
    import paged_kv_cache_386_amd as pa
    c, dc = _case()
    NB, B = c.num_blocks, c.block_size
    T = 3
    k = torch.ones((T, c.num_kv_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")
    before = dc.k_cache.clone()
    say("index check: kv_cache_append")
    ok_slots = torch.tensor([-1, 1 * B + 2, 4 * B], dtype=torch.int32, device="cuda")
    bad_slots = torch.tensor([-1, NB * B, 4 * B], dtype=torch.int32, device="cuda")
    ok_pairs = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    bad_pairs = torch.tensor([[0, 1], [NB, 2]], dtype=torch.int32, device="cuda")
    _expect_index_error(lambda: pa.kv_cache_append(bad_pairs, k, k, ok_slots, dc.k_cache,
                                                   dc.v_cache))
    _expect_index_error(lambda: pa.kv_cache_append(ok_pairs, k, k, bad_slots, dc.k_cache,
                                                   dc.v_cache))
    torch.cuda.synchronize()
    assert torch.equal(dc.k_cache.view(torch.int16), before.view(torch.int16))
    pa.kv_cache_append(ok_pairs, k, k, ok_slots, dc.k_cache, dc.v_cache)
    torch.cuda.synchronize()
    # block 1 is block 0 except position 2, which holds the new token's ones
    got = dc.k_cache[1].view(torch.int16).cpu().numpy()
    want = before[0].view(torch.int16).cpu().numpy().copy()
    want[:, 2] = np.int16(0x3F80)  # bfloat16 1.0
    assert np.array_equal(got, want)
