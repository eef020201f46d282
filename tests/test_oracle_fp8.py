"""Pins of the FP8 (E4M3) oracle (CPU only): the element format against
torch's float8_e4m3fn conversions, the quantising write, and FP8 decode
against the bfloat16 decode oracle on pools whose dequantised values are
exact in bfloat16, plus closed forms."""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import oracle as O
from workloads import make_fp8_case, make_prefix_case, make_private_case
from workloads.generate import bf16_bits_from_f32, settle_step

from test_oracle_pins import small_prefix_case


def _torch_codes(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(y, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_every_code_decodes_like_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = fp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # a few values of the format itself
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    assert mine[0x38] == 1.0 and mine[0xB8] == -1.0 and np.isnan(mine[0x7F])


def test_encoding_matches_torch_with_saturation():
    rng = np.random.default_rng(0)
    vals = [rng.standard_normal(50000).astype(np.float32) * s for s in (1e-4, 1e-2, 1, 30, 1e3)]
    pos = fp8.e4m3_decode(np.arange(0x7F))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)  # every tie
    ties = [mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))]
    edge = np.array([0.0, -0.0, 448, 449, 464, 465, 480, 1e30, -1e30, np.inf, -np.inf, np.nan,
                     2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -6], np.float32)
    y = np.concatenate(vals + ties + [edge])
    assert np.array_equal(fp8.e4m3_encode(y), _torch_codes(y))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_divides_in_fp32(dtype):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32) * 3
    store = x if dtype == "f32" else bf16_bits_from_f32(x)
    xf = torch.from_numpy(O.to_f64(store, dtype).astype(np.float32))
    for scale in (0.25, 0.37, 3.0):
        want = _torch_codes((xf / torch.tensor(scale, dtype=torch.float32)).numpy())
        assert np.array_equal(fp8.quantize(store, dtype, scale), want)


def test_write_stores_codes_and_skips_negative_slots():
    rng = np.random.default_rng(2)
    kc = np.full((3, 2, 4, 8), 0x7F, np.uint8)
    vc = kc.copy()
    k = bf16_bits_from_f32(rng.standard_normal((3, 2, 8)).astype(np.float32))
    v = bf16_bits_from_f32(rng.standard_normal((3, 2, 8)).astype(np.float32))
    kc2, vc2 = fp8.kv_cache_write_fp8(k, v, np.array([5, -1, 8]), kc, vc, 4, "bf16", 0.5, 0.25)
    assert np.array_equal(kc2[1, :, 1], fp8.quantize(k[0], "bf16", 0.5))
    assert np.array_equal(vc2[2, :, 0], fp8.quantize(v[2], "bf16", 0.25))
    kc2[1, :, 1] = 0x7F
    kc2[2, :, 0] = 0x7F
    assert (kc2 == 0x7F).all()
    # values already on the grid come back as their own codes
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    exact = (fp8.e4m3_decode(codes) * 0.5).astype(np.float32)
    assert np.array_equal(fp8.quantize(exact, "f32", 0.5), codes)


def _bf16_twin(c8):
    """The bfloat16 workload whose pool holds the FP8 pool's dequantised
    values (exact in bfloat16 for power-of-two scales)."""
    b = c8.base
    kd = fp8.dequantize(c8.k8, c8.k_scale)
    vd = fp8.dequantize(c8.v8, c8.v_scale)
    kb = bf16_bits_from_f32(np.nan_to_num(kd, nan=0).astype(np.float32))
    vb = bf16_bits_from_f32(np.nan_to_num(vd, nan=0).astype(np.float32))
    assert np.array_equal(O.to_f64(kb, "bf16")[~np.isnan(kd)], kd[~np.isnan(kd)])
    kb[np.isnan(kd)] = b.k_cache[np.isnan(kd)]
    vb[np.isnan(vd)] = b.v_cache[np.isnan(vd)]
    return kb, vb


@pytest.mark.parametrize("maker", ["private", "prefix"])
def test_decode_equals_bf16_decode_on_exact_values(maker):
    if maker == "private":
        base = make_private_case("f8", [1, 15, 16, 17, 40, 100], 8, 2, 16, 4, "bf16", 3)
    else:
        base = settle_step(small_prefix_case(dtype="bf16"))
    c8 = make_fp8_case(base, 3, k_scale=0.25, v_scale=2.0)
    kb, vb = _bf16_twin(c8)
    want = O.paged_attention_decode(base.q, kb, vb, base.block_tables, base.context_lens,
                                    base.scale, base.block_size, "bf16")
    got = fp8.paged_attention_decode_fp8(base.q, c8.k8, c8.v8, base.block_tables,
                                         base.context_lens, base.scale, base.block_size, "bf16",
                                         c8.k_scale, c8.v_scale)
    assert np.abs(got - want).max() < 1e-12
    Hq = base.num_q_heads
    rows = [(0, 0), (3, Hq - 1), (5, Hq // 2)]
    part = fp8.paged_attention_decode_fp8(base.q, c8.k8, c8.v8, base.block_tables,
                                          base.context_lens, base.scale, base.block_size,
                                          "bf16", c8.k_scale, c8.v_scale, rows=rows)
    assert np.abs(part - np.array([got[s, h] for s, h in rows])).max() < 1e-13


def test_identical_keys_and_one_token():
    base = make_private_case("f8c", [1, 9, 33], 4, 2, 8, 4, "bf16", 4)
    c8 = make_fp8_case(base, 4, v_scale=0.75)
    k8 = c8.k8.copy()
    k8[k8 != 0x7F] = 0x38  # every key 1.0
    out = fp8.paged_attention_decode_fp8(base.q, k8, c8.v8, base.block_tables, base.context_lens,
                                         base.scale, base.block_size, "bf16", c8.k_scale,
                                         c8.v_scale)
    for s, L in enumerate(base.context_lens.tolist()):
        _, V = fp8.gather_sequence_fp8(k8, c8.v8, base.block_tables[s], L, base.block_size,
                                       c8.k_scale, c8.v_scale)
        assert np.abs(out[s] - np.repeat(V.mean(axis=0), 2, axis=0)).max() < 1e-12
    # the one-token sequence returns its dequantised V row exactly
    v0 = fp8.dequantize(c8.v8[base.block_tables[0, 0], :, 0], c8.v_scale)
    assert np.array_equal(out[0], np.repeat(v0, 2, axis=0))


def test_multi_query_fp8_pins():
    """The FP8 multi-query oracle against two pinned oracles: on pools whose
    dequantised values are exact in bf16 it equals the bf16 multi-query
    oracle on those values, and one query token per sequence (attending the
    whole context) equals the FP8 decode oracle."""
    from workloads import make_multi_query_case
    base = make_private_case("f8mq", [5, 17, 40, 100], 8, 2, 16, 4, "bf16", 6)
    c8 = make_fp8_case(base, 6, k_scale=0.25, v_scale=2.0)
    kb, vb = _bf16_twin(c8)
    mq = make_multi_query_case(base, [5, 3, 0, 7], 6)
    want = O.paged_attention_multi_query(mq.q, kb, vb, base.block_tables, base.context_lens,
                                         mq.query_start, base.scale, base.block_size, "bf16")
    got = fp8.paged_attention_multi_query_fp8(mq.q, c8.k8, c8.v8, base.block_tables,
                                              base.context_lens, mq.query_start, base.scale,
                                              base.block_size, "bf16", c8.k_scale, c8.v_scale)
    assert np.abs(got - want).max() < 1e-12
    one = make_multi_query_case(base, [1, 1, 1, 1], 7)
    got1 = fp8.paged_attention_multi_query_fp8(one.q, c8.k8, c8.v8, base.block_tables,
                                               base.context_lens, one.query_start, base.scale,
                                               base.block_size, "bf16", c8.k_scale, c8.v_scale)
    dec = fp8.paged_attention_decode_fp8(one.q, c8.k8, c8.v8, base.block_tables,
                                         base.context_lens, base.scale, base.block_size, "bf16",
                                         c8.k_scale, c8.v_scale)
    assert np.array_equal(got1, dec)
