"""FP8 (E4M3) KV cache through the C ABI against the oracle (needs an MI355X):
the quantising write bit for bit (every rounding case, saturation, NaN,
signed zeros, negative slots), every code read back exactly through decode,
FP8 decode against the oracle on private, prefix-shared and forked pools at
several block and partition sizes and at head_dim 64 and 128, and the
full-size GQA prefix workload (every output element)."""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import oracle as O
from workloads import make_case, make_fork_case, make_fp8_case, make_private_case
from workloads.generate import bf16_bits_from_f32, settle_step, E4M3_QNAN

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


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_decode_fp8(c8, ps=0):
    import paged_kv_cache_386_amd as pa
    b = c8.base
    NB, B = b.num_blocks, b.block_size
    for s, L in enumerate(b.context_lens.tolist()):
        nb = -(-L // B)
        assert ((b.block_tables[s, :nb] >= 0) & (b.block_tables[s, :nb] < NB)).all()
    out = torch.empty(b.q.shape, dtype=torch.float32, device="cuda")
    pa.paged_attention_decode_fp8(
        to_torch(b.q, "bf16"), _u8(c8.k8), _u8(c8.v8),
        torch.from_numpy(b.block_tables).cuda(), torch.from_numpy(b.context_lens).cuda(),
        float(b.scale), float(c8.k_scale), float(c8.v_scale), out,
        max_context_len=b.max_context_len, partition_size=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_decode(c8, rows=None):
    b = c8.base
    return fp8.paged_attention_decode_fp8(b.q, c8.k8, c8.v8, b.block_tables, b.context_lens,
                                          b.scale, b.block_size, "bf16", c8.k_scale,
                                          c8.v_scale, rows=rows)


# ---------------------------------------------------------------- write

def _special_values():
    pos = fp8.e4m3_decode(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2
    v = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [448, 449, 464, 465, 480, 1e6, np.inf, np.nan, 2.0 ** -10, 2.0 ** -12]])
    v = np.concatenate([v, -v, [0.0, -0.0]]).astype(np.float32)
    return v


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.25, 0.37])
def test_write_rounds_like_the_oracle(src, scale):
    import paged_kv_cache_386_amd as pa
    rng = np.random.default_rng(5)
    Hkv, D, B, NB = 2, 128, 16, 12
    vals = np.concatenate([_special_values() * np.float32(scale),
                           rng.standard_normal(4000).astype(np.float32) * 2])
    T = -(-len(vals) // (Hkv * D))
    flat = np.resize(vals, T * Hkv * D).astype(np.float32)
    k = flat.reshape(T, Hkv, D)
    v = np.roll(flat, 7).reshape(T, Hkv, D)
    if src == "bf16":
        k, v = bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    slots = rng.permutation(NB * B)[:T].astype(np.int32)
    slots[3] = -1
    kc = np.full((NB, Hkv, B, D), 0xA5, np.uint8)
    vc = kc.copy()
    say(f"fp8 write src={src} scale={scale} T={T}")
    dk, dv = _u8(kc), _u8(vc)
    pa.kv_cache_write_fp8(to_torch(k, src), to_torch(v, src), torch.from_numpy(slots).cuda(),
                          dk, dv, scale, scale * 2)
    torch.cuda.synchronize()
    wk, wv = fp8.kv_cache_write_fp8(k, v, slots, kc, vc, B, src, scale, scale * 2)
    assert np.array_equal(dk.cpu().numpy(), wk)
    assert np.array_equal(dv.cpu().numpy(), wv)


def test_raw_byte_edits_on_fp8_pools():
    """kv_cache_write (codes as bytes) and copy_blocks on uint8 pools."""
    import paged_kv_cache_386_amd as pa
    rng = np.random.default_rng(6)
    kc = rng.integers(0, 256, size=(10, 2, 16, 128), dtype=np.uint8)
    vc = rng.integers(0, 256, size=kc.shape, dtype=np.uint8)
    k = rng.integers(0, 256, size=(5, 2, 128), dtype=np.uint8)
    v = rng.integers(0, 256, size=(5, 2, 128), dtype=np.uint8)
    slots = np.array([3, 17, -1, 100, 159], np.int32)
    pairs = np.array([[1, 7], [2, 8]], np.int32)
    dk, dv = _u8(kc), _u8(vc)
    pa.copy_blocks(torch.from_numpy(pairs).cuda(), dk, dv, host_pairs=pairs)
    pa.kv_cache_write(_u8(k), _u8(v), torch.from_numpy(slots).cuda(), dk, dv)
    torch.cuda.synchronize()
    wk, wv = O.copy_blocks(pairs, kc, vc)
    wk, wv = O.kv_cache_write(k, v, slots, wk, wv, 16)
    assert np.array_equal(dk.cpu().numpy(), wk) and np.array_equal(dv.cpu().numpy(), wv)


# ---------------------------------------------------------------- decode

def test_every_code_reads_back_exactly():
    """1-token contexts return v_scale * e4m3(code) of their V row, for every
    finite code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)  # 254
    S = 2
    base = make_private_case("f8-codes", [1] * S, 8, 2, 128, 16, "bf16", 8)
    c8 = make_fp8_case(base, 8, k_scale=0.5, v_scale=0.25)
    row = np.resize(codes, S * 2 * 128).reshape(S, 2, 128)
    for s in range(S):
        c8.v8[base.block_tables[s, 0], :, 0] = row[s]
    got = run_decode_fp8(c8)
    for s in range(S):
        want = fp8.e4m3_decode(row[s]) * 0.25  # [Hkv, D]
        assert np.array_equal(got[s], np.repeat(want, 4, axis=0).astype(np.float32))


def test_every_code_reads_back_exactly_head_dim_64():
    """The same at head_dim 64 (the vector kernel, 16 codes per lane vector)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)  # 254
    S = 2
    base = make_private_case("f8-codes-64", [1] * S, 8, 2, 64, 16, "bf16", 9)
    c8 = make_fp8_case(base, 9, k_scale=0.5, v_scale=0.25)
    row = np.resize(codes, S * 2 * 64).reshape(S, 2, 64)
    for s in range(S):
        c8.v8[base.block_tables[s, 0], :, 0] = row[s]
    got = run_decode_fp8(c8)
    for s in range(S):
        want = fp8.e4m3_decode(row[s]) * 0.25
        assert np.array_equal(got[s], np.repeat(want, 4, axis=0).astype(np.float32))


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 2), (4, 2), (8, 1)])
@pytest.mark.parametrize("B", [1, 4, 16, 512])
def test_decode_head_dim_64(G, Hkv, B):
    """head_dim 64: the vector kernel, each 16-byte vector of codes widened to
    bfloat16 as it is computed; NaN-poisoned slots past every context."""
    lens = [1, 15, 16, 17, 63, 64, 65, 200, 513, 1030]
    base = make_private_case(f"f8-d64-{G}-{B}", lens, G * Hkv, Hkv, 64, B, "bf16", 70 + G + B)
    c8 = make_fp8_case(base, 70 + G + B)
    ref = oracle_decode(c8)
    for ps in (0, -1, 64):
        say(f"fp8 decode D=64 G={G} B={B} ps={ps}")
        err = max_err(run_decode_fp8(c8, ps), ref)
        assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"G={G} B={B} ps={ps}: {err}"


@pytest.mark.parametrize("ps", [-1, 0])
def test_decode_head_dim_64_long_contexts(ps):
    base = make_private_case("f8-d64-long", [9000, 20001, 3], 16, 4, 64, 16, "bf16", 77)
    c8 = make_fp8_case(base, 77)
    say(f"fp8 decode D=64 long contexts ps={ps}")
    err = max_err(run_decode_fp8(c8, ps), oracle_decode(c8))
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"ps={ps}: {err}"


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 2), (4, 2), (8, 1)])
@pytest.mark.parametrize("B", [1, 4, 16, 64, 512])
def test_decode_matches_oracle(G, Hkv, B):
    lens = [1, 15, 16, 17, 63, 64, 65, 200, 513, 1030]
    base = make_private_case(f"f8-{G}-{B}", lens, G * Hkv, Hkv, 128, B, "bf16", G + B)
    c8 = make_fp8_case(base, G + B)
    ref = oracle_decode(c8)
    for ps in (0, -1, 64):
        say(f"fp8 decode G={G} B={B} ps={ps}")
        err = max_err(run_decode_fp8(c8, ps), ref)
        assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"G={G} B={B} ps={ps}: {err}"


@pytest.mark.parametrize("G,Hkv", [(1, 2), (4, 2), (8, 1)])
@pytest.mark.parametrize("ps", [-1, 0])
def test_long_contexts_one_workgroup(G, Hkv, ps):
    """Contexts of 9,000 and 20,001 tokens: unsplit, a wave walks more than
    64 tiles, so its block ids come in several 64-tile chunks, with a ragged
    last tile (for G <= 4 through the three-buffer walk of 8-bit pools)."""
    base = make_private_case(f"f8-long-{G}", [9000, 20001], G * Hkv, Hkv, 128, 16, "bf16",
                             50 + G)
    c8 = make_fp8_case(base, 50 + G)
    say(f"fp8 long contexts G={G} ps={ps}")
    err = max_err(run_decode_fp8(c8, ps), oracle_decode(c8))
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"G={G} ps={ps}: {err}"


def test_decode_large_codes_and_prefix_sharing():
    """Codes over the whole E4M3 range (to 448) on a prefix-shared pool."""
    from workloads import make_prefix_case
    from workloads.generate import draw_e4m3_codes
    lens = [1, 5, 9, 16, 17, 18, 20, 33, 3, 40, 12, 300, 64, 65, 70, 1000]
    base = settle_step(make_prefix_case("f8-large", lens, 8, 32, 16, 2, 128, 16, "bf16", 31))
    c8 = make_fp8_case(base, 31, k_scale=0.01, v_scale=0.01)
    rng = np.random.default_rng(31)
    big = draw_e4m3_codes(rng, c8.k8.shape, max_exponent_field=15)
    big[(big & 0x7F) == 0x7F] = 0x7E  # no NaN codes in slots that are read
    c8.k8[:] = np.where(c8.k8 == E4M3_QNAN, c8.k8, big)
    c8.v8[:] = np.where(c8.v8 == E4M3_QNAN, c8.v8, np.roll(big, 1, axis=0))
    err = max_err(run_decode_fp8(c8), oracle_decode(c8))
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], err


def test_decode_forked_pool():
    base = settle_step(make_fork_case("f8-fork", [9, 9, 9, 9, 60, 60, 60, 60, 1, 130, 4, 300],
                                      2, 4, 32, 8, 128, 16, "bf16", 12))
    c8 = make_fp8_case(base, 12)
    err = max_err(run_decode_fp8(c8), oracle_decode(c8))
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], err


def test_full_size_prefix_workload():
    """The GQA prefix-sharing batch at full size over an FP8 pool, in
    the benchmark's launch configuration (automatic partitions, dispatch
    list): every output element against the oracle."""
    base = settle_step(make_case(2))
    c8 = make_fp8_case(base, 2)
    say("fp8 decode, GQA prefix-sharing batch at full size")
    got = run_decode_fp8(c8)
    assert np.isfinite(got).all()
    err = max_err(got, oracle_decode(c8))
    say(f"fp8 cfg2 full size: all {got.size} outputs, max abs err {err:.3e}")
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], err


# ---------------------------------------------------------------- multi-query

def _run_mq_fp8(c8, mq, ps=0, max_q=None):
    import paged_kv_cache_386_amd as pa
    b = c8.base
    out = torch.full((mq.num_tokens, b.num_q_heads, b.head_dim), 7.0, dtype=torch.float32,
                     device="cuda")
    pa.paged_attention_multi_query_fp8(
        to_torch(mq.q, "bf16"), _u8(c8.k8), _u8(c8.v8), torch.from_numpy(b.block_tables).cuda(),
        torch.from_numpy(b.context_lens).cuda(), torch.from_numpy(mq.query_start).cuda(),
        float(b.scale), float(c8.k_scale), float(c8.v_scale), out,
        max_query_len=mq.max_query_len if max_q is None else max_q,
        max_context_len=int(b.context_lens.max()), partition_size=ps)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("G,Hkv,q_lens", [(4, 2, [5, 1, 0, 16]), (8, 1, [8, 3, 1, 5]),
                                          (1, 4, [40, 64, 2, 17])])
@pytest.mark.parametrize("B", [16, 4])
@pytest.mark.parametrize("ps", [0, 64, -1])
def test_multi_query_matches_oracle(G, Hkv, q_lens, B, ps):
    from workloads import make_multi_query_case
    lens = [max(q, L) for q, L in zip(q_lens, [5, 40, 300, 1030])]
    base = make_private_case(f"f8mq-{G}-{B}", lens, G * Hkv, Hkv, 128, B, "bf16", 60 + G + B)
    c8 = make_fp8_case(base, 60 + G + B)
    mq = make_multi_query_case(base, q_lens, 60 + G)
    say(f"fp8 multi-query G={G} B={B} ps={ps} q_lens={q_lens}")
    got = _run_mq_fp8(c8, mq, ps)
    ref = fp8.paged_attention_multi_query_fp8(mq.q, c8.k8, c8.v8, base.block_tables,
                                              base.context_lens, mq.query_start, base.scale,
                                              base.block_size, "bf16", c8.k_scale, c8.v_scale)
    err = max_err(got, ref)
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"G={G} B={B} ps={ps}: {err}"


@pytest.mark.parametrize("G,Hkv,q_lens", [(4, 2, [512, 65, 0, 300]), (8, 1, [200, 9, 513, 64]),
                                          (1, 4, [512, 130, 1, 77])])
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("B,ps", [(16, 0), (4, -1), (16, 128)])
def test_multi_query_long_chunks(G, Hkv, q_lens, D, B, ps):
    """Chunks of more than 64 rows per KV head (chunked prefill) over an FP8
    pool, on the row-tile kernel: every output element."""
    from workloads import make_multi_query_case
    lens = [max(q, L) for q, L in zip(q_lens, [700, 1500, 513, 64])]
    base = make_private_case(f"f8cp-{G}-{D}", lens, G * Hkv, Hkv, D, B, "bf16", 90 + G + D)
    c8 = make_fp8_case(base, 90 + G)
    mq = make_multi_query_case(base, q_lens, 91 + G)
    say(f"fp8 chunked prefill G={G} D={D} B={B} ps={ps} q_lens={q_lens}")
    got = _run_mq_fp8(c8, mq, ps)
    ref = fp8.paged_attention_multi_query_fp8(mq.q, c8.k8, c8.v8, base.block_tables,
                                              base.context_lens, mq.query_start, base.scale,
                                              base.block_size, "bf16", c8.k_scale, c8.v_scale)
    err = max_err(got, ref)
    say(f"fp8 chunked prefill G={G} D={D} ps={ps}: max abs err {err:.3e}")
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"G={G} D={D} B={B} ps={ps}: {err}"


def test_multi_query_chunked_prefill_workload():
    """The chunked-prefill workload (16 sequences, contexts U[1024, 8192], a
    512-token chunk each) over an FP8 pool at full size in the benchmark's
    launch configuration; every output of four sequences against the oracle
    (the whole pool, tables and launch as run)."""
    from workloads import make_multi_query_workload
    from workloads.generate import subset_sequences, make_multi_query_case as mqc
    c = make_multi_query_workload("chunked-prefill")
    b = c.base
    c8 = make_fp8_case(b, 72)
    say(f"fp8 chunked prefill full size: S={b.num_seqs} T={c.num_tokens}")
    got = _run_mq_fp8(c8, c)
    assert np.isfinite(got).all()
    keep = [0, 5, 10, 15]
    sub = subset_sequences(b, keep)
    rows = np.concatenate([np.arange(c.query_start[s], c.query_start[s + 1]) for s in keep])
    sq = mqc(sub, np.diff(c.query_start)[keep], 72)
    sq.q = c.q[rows]
    ref = fp8.paged_attention_multi_query_fp8(sq.q, c8.k8, c8.v8, sub.block_tables,
                                              sub.context_lens, sq.query_start, b.scale,
                                              b.block_size, "bf16", c8.k_scale, c8.v_scale)
    err = max_err(got[rows], ref)
    say(f"fp8 chunked prefill full size: {len(rows)} rows, max abs err {err:.3e}")
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"max abs err {err}"


def test_multi_query_full_size_verification():
    """Speculative verification at full size (256 sequences, config-2
    contexts, 5 tokens each) over an FP8 pool, in the launch configuration
    of the benchmark: every output element against the oracle."""
    from workloads import make_multi_query_workload
    c = make_multi_query_workload("spec-verify", poison=False)
    b = c.base
    c8 = make_fp8_case(b, 71)
    say(f"fp8 multi-query full size: S={b.num_seqs} T={c.num_tokens}")
    got = _run_mq_fp8(c8, c)
    ref = fp8.paged_attention_multi_query_fp8(c.q, c8.k8, c8.v8, b.block_tables,
                                              b.context_lens, c.query_start, b.scale,
                                              b.block_size, "bf16", c8.k_scale, c8.v_scale)
    err = max_err(got, ref)
    say(f"fp8 spec-verify full size: all {got.size} outputs, max abs err {err:.3e}")
    assert err <= TOL["bf16"] and err <= REGRESS["bf16"], f"max abs err {err}"
