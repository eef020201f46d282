"""Pins of the oracle's multi-query (causal) paged attention (CPU only).

The oracle is checked against things other than itself: the library SDPA with
an explicit causal mask over the densely stored tokens (which never go
through a block table), pure-Python brute force on tiny inputs, the
identical-key closed form (row i returns the mean of V over positions
[0, p_i]), a one-token prefix returning its V row exactly, causality (tokens
after p_i never matter, token p_i does), agreement of a one-token chunk with
decode, and invariance under relabelling physical blocks.  Planted mistakes
at the end show that these pins catch an off-by-one mask, a dropped position
offset, a missing mask and interleaved GQA heads."""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import oracle as O
from workloads import make_multi_query_case, make_private_case
from workloads.generate import bf16_bits_from_f32, permute_pool


def _case(lens, q_lens, Hq=4, Hkv=2, D=8, B=4, dtype="bf16", seed=3, poison=True):
    base = make_private_case("mq", lens, Hq, Hkv, D, B, dtype, seed, keep_logical=True,
                             poison=poison)
    return make_multi_query_case(base, q_lens, seed)


def _run(c, fn=None):
    b = c.base
    fn = fn or O.paged_attention_multi_query
    return fn(c.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, c.query_start,
              b.scale, b.block_size, b.dtype)


def _sdpa(c):
    """torch SDPA (float64, CPU) per sequence on the logical tokens with an
    explicit boolean causal mask."""
    b = c.base
    G = b.num_q_heads // b.num_kv_heads
    out = np.zeros(c.q.shape)
    qf = O.to_f64(c.q, b.dtype)
    for s in range(b.num_seqs):
        a, e = int(c.query_start[s]), int(c.query_start[s + 1])
        n, L = e - a, int(b.context_lens[s])
        if n == 0:
            continue
        K = torch.from_numpy(O.to_f64(b.logical_k[s], b.dtype)).permute(1, 0, 2)  # [Hkv, L, D]
        V = torch.from_numpy(O.to_f64(b.logical_v[s], b.dtype)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        q = torch.from_numpy(qf[a:e]).permute(1, 0, 2)  # [Hq, n, D]
        pos = torch.arange(L)[None, :]
        mask = pos <= (L - n + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q, K, V, attn_mask=mask, scale=float(np.float64(np.float32(b.scale))))
        out[a:e] = o.permute(1, 0, 2).numpy()
    return out


CASES = [
    ([1, 5, 9, 16, 17, 33], [1, 5, 3, 16, 4, 1]),
    ([40, 7, 23], [40, 0, 12]),
    ([64], [17]),
]


@pytest.mark.parametrize("lens,q_lens", CASES)
@pytest.mark.parametrize("G,Hkv", [(1, 2), (2, 2), (4, 1)])
def test_library_sdpa_pin(lens, q_lens, G, Hkv):
    c = _case(lens, q_lens, Hq=G * Hkv, Hkv=Hkv)
    assert np.abs(_run(c) - _sdpa(c)).max() < 1e-12


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_pin(dtype):
    c = _case([3, 6, 5], [2, 6, 1], Hq=4, Hkv=2, D=4, B=2, dtype=dtype)
    b = c.base
    want = brute.multi_query(c.q.tolist(), b.k_cache.tolist(), b.v_cache.tolist(),
                             b.block_tables.tolist(), b.context_lens.tolist(),
                             c.query_start.tolist(), float(b.scale), b.block_size, dtype)
    assert np.abs(_run(c) - np.array(want)).max() < 1e-12


def test_identical_keys_give_prefix_means():
    c = _case([12, 7], [12, 3], poison=False)
    b = c.base
    one = bf16_bits_from_f32(np.full(b.k_cache.shape[1:], 0.5, np.float32))
    b.k_cache[:] = one
    got = _run(c)
    for s in range(b.num_seqs):
        a, e = int(c.query_start[s]), int(c.query_start[s + 1])
        n, L = e - a, int(b.context_lens[s])
        V = O.to_f64(b.logical_v[s], b.dtype)  # [L, Hkv, D]
        G = b.num_q_heads // b.num_kv_heads
        for i in range(n):
            p = L - n + i
            mean = V[:p + 1].mean(axis=0)  # [Hkv, D]
            assert np.abs(got[a + i] - np.repeat(mean, G, axis=0)).max() < 1e-12


def test_first_position_returns_its_v_row():
    # a whole prompt as the chunk: its first token sees only itself
    c = _case([9, 20], [9, 20], dtype="f32")
    got = _run(c)
    b = c.base
    G = b.num_q_heads // b.num_kv_heads
    for s in range(2):
        v0 = b.logical_v[s][0].astype(np.float64)  # [Hkv, D]
        assert np.array_equal(got[c.query_start[s]], np.repeat(v0, G, axis=0))


def test_causality():
    """Changing position t changes exactly the rows at positions >= t."""
    c = _case([30], [10], dtype="f32", poison=False)
    b = c.base
    base_out = _run(c)
    L, n = 30, 10
    for t in (L - 1, L - 4, L - n):
        kc, vc = b.k_cache.copy(), b.v_cache.copy()
        phys, off = b.block_tables[0][t // b.block_size], t % b.block_size
        kc[phys, :, off] += 1.0
        vc[phys, :, off] -= 2.0
        got = O.paged_attention_multi_query(c.q, kc, vc, b.block_tables, b.context_lens,
                                            c.query_start, b.scale, b.block_size, b.dtype)
        for i in range(n):
            p = L - n + i
            same = np.array_equal(got[i], base_out[i])
            assert same == (p < t), (t, i)


def test_one_token_chunk_equals_decode():
    c = _case([1, 17, 40, 64], [1, 1, 1, 1])
    b = c.base
    dec = O.paged_attention_decode(c.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                   b.scale, b.block_size, b.dtype)
    assert np.abs(_run(c) - dec).max() < 1e-14


def test_block_relabelling_invariance():
    c = _case([33, 18, 5], [20, 18, 2])
    b = c.base
    kc, vc, tables, _, _, _ = permute_pool(b, 4)
    got = O.paged_attention_multi_query(c.q, kc, vc, tables, b.context_lens, c.query_start,
                                        b.scale, b.block_size, b.dtype)
    assert np.array_equal(got, _run(c))


def test_empty_chunks_and_bad_lengths():
    c = _case([5, 6], [0, 0])
    assert _run(c).shape == (0, 4, 8)
    with pytest.raises(ValueError):
        _case([5], [6])


# ---------------------------------------------------------------- planted mistakes

def _mutant(mask_extra=0, absolute=True, masked=True, interleave=False):
    def fn(q, kc, vc, tables, lens, qs, scale, B, dtype):
        T, Hq, D = q.shape
        Hkv = kc.shape[1]
        G = Hq // Hkv
        qf = O.to_f64(q, dtype)
        out = np.zeros((T, Hq, D))
        for s in range(len(qs) - 1):
            n = int(qs[s + 1] - qs[s])
            L = int(lens[s])
            K, V = O.gather_sequence(kc, vc, tables[s], L, B, dtype)
            for i in range(n):
                p = (L - n + i) if absolute else i
                last = min(p + mask_extra, L - 1) if masked else L - 1
                for h in range(Hq):
                    g = h % Hkv if interleave else h // G
                    x = np.float64(np.float32(scale)) * (K[:last + 1, g] @ qf[qs[s] + i, h])
                    w = np.exp(x - x.max())
                    out[qs[s] + i, h] = (w @ V[:last + 1, g]) / w.sum()
        return out
    return fn


@pytest.mark.parametrize("name,fn", [
    ("mask-one-late", _mutant(mask_extra=1)),
    ("position-from-zero", _mutant(absolute=False)),
    ("no-mask", _mutant(masked=False)),
    ("gqa-interleaved", _mutant(interleave=True)),
])
def test_pins_catch_planted_mistakes(name, fn):
    c = _case([9, 17, 33], [4, 17, 6], Hq=4, Hkv=2)
    assert np.abs(_run(c, fn) - _sdpa(c)).max() > 1e-6, name
    assert np.abs(_run(c) - _sdpa(c)).max() < 1e-12
