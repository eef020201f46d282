"""Pins of the INT8 KV-cache oracle (CPU only): the quantiser against torch's
round-half-even and clamp, the write, and INT8 decode against the bf16
decode oracle on pools whose dequantised values are exact in bf16."""
import numpy as np
import pytest
import torch

from oracle import int8
from oracle import oracle as O
from workloads import make_int8_case, make_private_case
from workloads.generate import bf16_bits_from_f32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.02, 0.37])
def test_quantize_matches_torch(dtype, scale):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s
                        for s in (0.01, 1, 3, 100)])
    halves = (np.arange(-140, 140) + 0.5).astype(np.float32) * np.float32(scale)
    x = np.concatenate([x, halves, [0.0, -0.0, 1e30, -1e30, np.inf, -np.inf]]).astype(np.float32)
    store = x if dtype == "f32" else bf16_bits_from_f32(np.nan_to_num(x))
    xf = torch.from_numpy(O.to_f64(store, dtype).astype(np.float32))
    want = torch.round(xf / torch.tensor(scale, dtype=torch.float32)).clamp(-127, 127)
    assert np.array_equal(int8.quantize(store, dtype, scale), want.to(torch.int8).numpy())
    assert int8.quantize(np.array([np.nan], np.float32), "f32", scale)[0] == 0


def test_ties_go_to_even():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5], np.float32)
    assert int8.quantize(y, "f32", 1.0).tolist() == [0, 2, 2, 0, -2, -2, 126, -126]


def test_write_and_skip():
    rng = np.random.default_rng(2)
    kc = np.full((3, 2, 4, 16), -128, np.int8)
    vc = kc.copy()
    k = rng.standard_normal((2, 2, 16)).astype(np.float32)
    v = rng.standard_normal((2, 2, 16)).astype(np.float32)
    kc2, vc2 = int8.kv_cache_write_int8(k, v, np.array([6, -1]), kc, vc, 4, "f32", 0.05, 0.1)
    assert np.array_equal(kc2[1, :, 2], int8.quantize(k[0], "f32", 0.05))
    assert np.array_equal(vc2[1, :, 2], int8.quantize(v[0], "f32", 0.1))
    kc2[1, :, 2] = -128
    assert (kc2 == -128).all()


def test_decode_equals_bf16_decode_on_exact_values():
    base = make_private_case("i8", [1, 15, 16, 17, 40, 100], 8, 2, 16, 4, "bf16", 3)
    c8 = make_int8_case(base, 3, k_scale=2.0 ** -5, v_scale=2.0 ** -6)
    kd, vd = int8.dequantize(c8.k8, c8.k_scale), int8.dequantize(c8.v8, c8.v_scale)
    kb = bf16_bits_from_f32(kd.astype(np.float32))
    vb = bf16_bits_from_f32(vd.astype(np.float32))
    assert np.array_equal(O.to_f64(kb, "bf16"), kd)
    want = O.paged_attention_decode(base.q, kb, vb, base.block_tables, base.context_lens,
                                    base.scale, base.block_size, "bf16")
    got = int8.paged_attention_decode_int8(base.q, c8.k8, c8.v8, base.block_tables,
                                           base.context_lens, base.scale, base.block_size,
                                           "bf16", c8.k_scale, c8.v_scale)
    assert np.abs(got - want).max() < 1e-12
    rows = [(0, 0), (3, 7), (5, 4)]
    part = int8.paged_attention_decode_int8(base.q, c8.k8, c8.v8, base.block_tables,
                                            base.context_lens, base.scale, base.block_size,
                                            "bf16", c8.k_scale, c8.v_scale, rows=rows)
    assert np.abs(part - np.array([got[s, h] for s, h in rows])).max() < 1e-13


def test_one_token_returns_its_v_row():
    base = make_private_case("i8c", [1, 9], 4, 2, 8, 4, "bf16", 4)
    c8 = make_int8_case(base, 4)
    out = int8.paged_attention_decode_int8(base.q, c8.k8, c8.v8, base.block_tables,
                                           base.context_lens, base.scale, base.block_size,
                                           "bf16", c8.k_scale, c8.v_scale)
    v0 = int8.dequantize(c8.v8[base.block_tables[0, 0], :, 0], c8.v_scale)
    assert np.array_equal(out[0], np.repeat(v0, 2, axis=0))


def test_multi_query_int8_pins():
    """The INT8 multi-query oracle equals the bf16 multi-query oracle on the
    dequantised values (exact in bf16 at power-of-two scales), and one token
    per sequence equals the INT8 decode oracle."""
    from workloads import make_multi_query_case
    base = make_private_case("i8mq", [5, 17, 40, 100], 8, 2, 16, 4, "bf16", 8)
    c8 = make_int8_case(base, 8, k_scale=2.0 ** -5, v_scale=2.0 ** -6)
    kd, vd = int8.dequantize(c8.k8, c8.k_scale), int8.dequantize(c8.v8, c8.v_scale)
    kb = bf16_bits_from_f32(kd.astype(np.float32))
    vb = bf16_bits_from_f32(vd.astype(np.float32))
    mq = make_multi_query_case(base, [5, 3, 0, 7], 8)
    want = O.paged_attention_multi_query(mq.q, kb, vb, base.block_tables, base.context_lens,
                                         mq.query_start, base.scale, base.block_size, "bf16")
    got = int8.paged_attention_multi_query_int8(mq.q, c8.k8, c8.v8, base.block_tables,
                                                base.context_lens, mq.query_start, base.scale,
                                                base.block_size, "bf16", c8.k_scale, c8.v_scale)
    assert np.abs(got - want).max() < 1e-12
    one = make_multi_query_case(base, [1, 1, 1, 1], 9)
    got1 = int8.paged_attention_multi_query_int8(one.q, c8.k8, c8.v8, base.block_tables,
                                                 base.context_lens, one.query_start, base.scale,
                                                 base.block_size, "bf16", c8.k_scale,
                                                 c8.v_scale)
    dec = int8.paged_attention_decode_int8(one.q, c8.k8, c8.v8, base.block_tables,
                                           base.context_lens, base.scale, base.block_size,
                                           "bf16", c8.k_scale, c8.v_scale)
    assert np.array_equal(got1, dec)
