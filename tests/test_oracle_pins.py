"""The oracle pinned to things other than itself (runs on the CPU)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import oracle as O
from workloads import make_case, make_fork_case, make_prefix_case, make_private_case
from workloads.generate import bf16_bits_from_f32

import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- small cases

def small_prefix_case(poison=True, dtype="bf16", B=4):
    # config-2 structure scaled down: 3 groups of 4 sequences share a 16-token prefix
    lens = [1, 2, 5, 9, 16, 17, 18, 20, 33, 3, 40, 12]
    return make_prefix_case("small-prefix", lens, 4, 16, 4, 2, 8, B, dtype, 5,
                            poison=poison, keep_logical=True)


def small_fork_case(poison=True, dtype="bf16", B=4):
    lens = [9, 9, 9, 9, 6, 6, 6, 6, 1, 13, 4, 30]
    return make_fork_case("small-fork", lens, 2, 4, 6, 3, 8, B, dtype, 6,
                          poison=poison, keep_logical=True)


# ---------------------------------------------------------------- exact decoding

def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0001, 0x8000, 0x7F7F], np.uint16)
    want = [1.0, -2.0, 0.333984375, 2.0 ** -133, -0.0, 3.3895313892515355e38]
    got = O.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert np.signbit(got[4])


def test_generator_rounds_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -1.5], np.float32)
    assert bf16_bits_from_f32(x).tolist() == [0x3F80, 0x3F82, 0x3F80, 0xBFC0]


# ---------------------------------------------------------------- page examples

def test_page1_block_table_example():
    g = _golden("page1_block_table.json")
    B = g["block_size"]
    table = g["logical_to_physical"]
    for j, (lo, hi) in enumerate(g["token_ranges"]):
        for t in range(lo, hi + 1):
            slot = O.slot_of(table, t, B)
            assert slot // B == table[j]
            assert slot % B == t - lo
    # token 20 sits in logical block 1 -> physical block 3, offset 4
    assert O.slot_of(table, 20, B) == 3 * 16 + 4


def test_page3_pool_picture_gather_order():
    g = _golden("page3_pool_picture.json")
    B = g["block_size"]
    pool = g["pool"]
    NB = len(pool)
    # each block's K rows encode (request, ordinal, offset); free blocks are NaN
    kc = np.full((NB, 1, B, 3), np.nan, np.float32)
    for p, tag in enumerate(pool):
        if tag is None:
            continue
        for o in range(B):
            kc[p, 0, o] = [ord(tag[0]), int(tag[1:]), o]
    for req, table in g["tables"].items():
        assert [pool[p] for p in table] == [f"{req}{i + 1}" for i in range(len(table))]
        L = len(table) * B - 3  # last block partly used
        K, _ = O.gather_sequence(kc, kc, np.array(table), L, B, "f32", kv_head=0)
        assert K.shape == (L, 3)
        assert np.all(K[:, 0] == ord(req))
        assert K[:, 1].tolist() == [t // B + 1 for t in range(L)]
        assert K[:, 2].tolist() == [t % B for t in range(L)]
        assert not np.isnan(K).any()
    assert sorted(set(range(NB)) - {p for t in g["tables"].values() for p in t}) == g["free"]


def test_page3_fragmentation_bound_and_utilisation():
    g = _golden("page3_utilisation.json")
    used = sum(g["context_tokens"])
    reserved = sum(g["reserved_tokens"])
    assert round(used / reserved, 2) == g["utilisation_printed"]
    pic = _golden("page3_pool_picture.json")
    B = pic["block_size"]
    for L in list(g["context_tokens"]) + list(range(1, 200)):
        waste = -(-L // B) * B - L
        assert 0 <= waste <= pic["max_internal_fragmentation_tokens"]


def test_kv_byte_model_matches_pages():
    g = _golden("page1_kv_bytes.json")
    m = g["example_model"]
    per_token = 2 * m["layers"] * m["hidden"] * m["bytes_per_element"]
    assert per_token == 512 * 1024
    total = per_token * m["seq_len"]
    u = _golden("page3_utilisation.json")
    assert total == u["bytes_per_4096_tokens_printed_gb"] * 2 ** 30


# ---------------------------------------------------------------- pins

def test_dense_library_pin_config0():
    case = make_case(0, keep_logical=True)
    assert pins.dense_sdpa_error(case) <= 1e-12


@pytest.mark.parametrize("B", [1, 4, 16])
def test_dense_library_pin_prefix_step(B):
    assert pins.dense_sdpa_error(small_prefix_case(B=B)) <= 1e-12


@pytest.mark.parametrize("B", [2, 4, 8])
def test_dense_library_pin_fork_step(B):
    assert pins.dense_sdpa_error(small_fork_case(B=B)) <= 1e-12


def test_brute_force_pin_config0():
    assert pins.brute_error(make_case(0)) <= 1e-12


@settings(max_examples=25, deadline=None)
@given(st.integers(0, 10 ** 6), st.sampled_from([1, 2, 4, 16]), st.sampled_from([1, 2, 4]),
       st.sampled_from([1, 2]), st.sampled_from(["f32", "bf16"]),
       st.lists(st.integers(0, 40), min_size=1, max_size=3))
def test_brute_force_pin_random_shapes(seed, B, G, Hkv, dtype, lens):
    case = make_private_case("hyp", lens, G * Hkv, Hkv, 4, B, dtype, seed,
                             pool_blocks=sum(-(-L // B) for L in lens) + 2)
    assert pins.brute_error(case) <= 1e-12


def test_one_token_returns_v_exactly():
    case = make_case(0)
    assert case.context_lens[0] == 1
    assert pins.one_token_mismatches(case) == 0


@pytest.mark.parametrize("maker", [lambda: make_case(0), lambda: make_private_case(
    "bf16", [1, 7, 40], 4, 2, 16, 4, "bf16", 3)])
def test_identical_keys_give_mean_of_v(maker):
    assert pins.identical_keys_error(maker()) <= 1e-12


@pytest.mark.parametrize("maker", [lambda: make_case(0), lambda: small_prefix_case(),
                                   lambda: small_fork_case()])
def test_block_permutation_invariance(maker):
    assert pins.permutation_mismatches(maker()) == 0


def test_block_size_invariance():
    # the long-context workload at two block sizes holds the same logical tokens
    outs = []
    for B in (64, 4):
        c = make_private_case(f"B{B}", [256, 256], 8, 2, 16, B, "bf16", 3,
                              max_blocks_per_seq=256 // B)
        outs.append(O.paged_attention_decode(c.q, c.k_cache, c.v_cache, c.block_tables,
                                             c.context_lens, c.scale, B, c.dtype))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("ps", [1, 5, 16, 64, 1000])
def test_split_merge_equals_unsplit(ps):
    c = make_private_case("split", [1, 17, 100, 300], 8, 2, 16, 16, "bf16", 9)
    a = O.paged_attention_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                 c.scale, 16, c.dtype)
    b = O.paged_attention_decode_partitioned(c.q, c.k_cache, c.v_cache, c.block_tables,
                                             c.context_lens, c.scale, 16, c.dtype, ps)
    assert np.abs(a - b).max() <= 1e-12


def test_rows_variant_matches_full():
    c = small_prefix_case()
    kc, vc = O.copy_blocks(c.copy_pairs, c.k_cache, c.v_cache)
    kc, vc = O.kv_cache_write(c.k_new, c.v_new, c.slot_mapping, kc, vc, c.block_size)
    full = O.paged_attention_decode(c.q, kc, vc, c.block_tables, c.context_lens,
                                    c.scale, c.block_size, c.dtype)
    rows = [(0, 0), (5, 3), (11, 1)]
    part = O.paged_attention_decode_rows(c.q, kc, vc, c.block_tables,
                                         c.context_lens, c.scale, c.block_size, c.dtype, rows)
    assert np.isfinite(part).all()
    for i, (s, h) in enumerate(rows):
        assert np.abs(part[i] - full[s, h]).max() <= 1e-14


def test_empty_context_gives_zeros():
    c = make_private_case("empty", [0, 3], 2, 1, 8, 4, "f32", 1)
    out = O.paged_attention_decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens,
                                   c.scale, 4, c.dtype)
    assert np.all(out[0] == 0.0) and np.isfinite(out).all()


def test_oracle_never_reads_poison():
    for c in (make_case(0), small_prefix_case(), small_fork_case()):
        kc, vc = c.k_cache, c.v_cache
        if c.has_step:
            kc, vc = O.copy_blocks(c.copy_pairs, kc, vc)
            kc, vc = O.kv_cache_write(c.k_new, c.v_new, c.slot_mapping, kc, vc, c.block_size)
        out = O.paged_attention_decode(c.q, kc, vc, c.block_tables, c.context_lens, c.scale,
                                       c.block_size, c.dtype)
        assert np.isfinite(out).all()


# ---------------------------------------------------------------- cache edits

@pytest.mark.parametrize("maker", [small_prefix_case, small_fork_case])
def test_copy_then_write_rebuilds_logical_tokens(maker):
    c = maker()
    kc, vc = O.copy_blocks(c.copy_pairs, c.k_cache, c.v_cache)
    kc, vc = O.kv_cache_write(c.k_new, c.v_new, c.slot_mapping, kc, vc, c.block_size)
    for s in range(c.num_seqs):
        L = int(c.context_lens[s])
        pos = np.arange(L)
        phys = c.block_tables[s][pos // c.block_size]
        assert np.array_equal(kc[phys, :, pos % c.block_size], c.logical_k[s])
        assert np.array_equal(vc[phys, :, pos % c.block_size], c.logical_v[s])


def test_write_skips_negative_slots_and_is_bitwise():
    # pool [blocks=2][kv_heads=1][block_size=4][head_dim=2]; slot 5 = block 1, offset 1
    kc = np.arange(2 * 1 * 4 * 2, dtype=np.uint16).reshape(2, 1, 4, 2)
    k = np.array([[[0x7FC1, 0xFFFF]], [[1, 2]], [[3, 4]]], np.uint16)
    out_k, out_v = O.kv_cache_write(k, k, np.array([5, -1, 0]), kc, kc, 4)
    want = kc.copy()
    want[1, :, 1] = k[0]
    want[0, :, 0] = k[2]
    assert np.array_equal(out_k, want) and np.array_equal(out_v, want)
    assert np.array_equal(kc, np.arange(16, dtype=np.uint16).reshape(2, 1, 4, 2))  # input untouched


def test_copy_blocks_in_list_order():
    kc = np.arange(4 * 2, dtype=np.float32).reshape(4, 2, 1, 1)
    out_k, _ = O.copy_blocks(np.array([[0, 1], [1, 2]]), kc, kc)
    # list order: block 1 becomes block 0, then block 2 becomes the new block 1
    assert out_k[:, :, 0, 0].tolist() == [[0, 1], [0, 1], [0, 1], [6, 7]]
