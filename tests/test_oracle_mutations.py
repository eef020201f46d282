"""Planted mistakes in copies of the oracle (CPU only): each must be caught by
at least one of the pins, which shows the pins can tell a wrong oracle apart.

Reading a sequence's tokens in another order is not among them: with no
positional term in decode attention the output depends only on the set of
attended tokens, so the gather order is checked directly instead (the page
picture test in ``test_oracle_pins.py``)."""
import numpy as np
import pytest

from oracle import oracle as O
from workloads import make_case, make_fork_case, make_prefix_case

import pins


def _decode_with(gather=None, kv_head_of=None, scale_mul=1.0, swap_kv=False, neg_exp=False,
                 row_shift=0):
    def decode(q, kc, vc, tables, lens, scale, B, dtype):
        S, Hq, D = q.shape
        Hkv = kc.shape[1]
        G = Hq // Hkv
        qf = O.to_f64(q, dtype)
        out = np.zeros((S, Hq, D))
        for s in range(S):
            row = tables[(s + row_shift) % S]
            if gather is None:
                K, V = O.gather_sequence(kc, vc, row, int(lens[s]), B, dtype)
            else:
                K, V = gather(kc, vc, row, int(lens[s]), B, dtype)
            if swap_kv:
                K, V = V, K
            for h in range(Hq):
                g = kv_head_of(h, G, Hkv) if kv_head_of else h // G
                if K.shape[0] == 0:
                    continue
                x = np.float64(np.float32(scale)) * scale_mul * (K[:, g] @ qf[s, h])
                w = np.exp((x.max() - x) if neg_exp else (x - x.max()))
                out[s, h] = (w @ V[:, g]) / w.sum()
        return out
    return decode


def _gather_drop_last(kc, vc, row, L, B, dtype):
    return O.gather_sequence(kc, vc, row, max(L - 1, 0), B, dtype)


def _gather_shifted_offset(kc, vc, row, L, B, dtype):
    pos = np.arange(L)
    phys = np.asarray(row)[pos // B]
    off = (pos + 1) % B
    return O.to_f64(kc[phys, :, off], dtype), O.to_f64(vc[phys, :, off], dtype)


MUTANTS = {
    "gqa-interleaved-heads": _decode_with(kv_head_of=lambda h, G, Hkv: h % Hkv),
    "dropped-last-token": _decode_with(gather=_gather_drop_last),
    "offset-off-by-one": _decode_with(gather=_gather_shifted_offset),
    "dropped-scale": _decode_with(scale_mul=1.0 / 0.125),
    "k-v-swapped": _decode_with(swap_kv=True),
    "exponent-sign": _decode_with(neg_exp=True),
    "wrong-table-row": _decode_with(row_shift=1),
}


def _caught(decode) -> bool:
    prefix = make_prefix_case("m-prefix", [1, 2, 5, 9, 16, 17, 18, 20], 4, 16, 4, 2, 8, 4,
                              "bf16", 5, keep_logical=True)
    fork = make_fork_case("m-fork", [9, 9, 9, 9, 6, 13, 4, 30], 1, 4, 6, 3, 8, 4, "bf16", 6,
                          keep_logical=True)
    cfg0 = make_case(0, keep_logical=True)
    checks = [
        lambda: pins.dense_sdpa_error(cfg0, decode) > 1e-9,
        lambda: pins.dense_sdpa_error(prefix, decode) > 1e-9,
        lambda: pins.dense_sdpa_error(fork, decode) > 1e-9,
        lambda: pins.one_token_mismatches(cfg0, decode) > 0,
    ]
    for c in checks:
        with np.errstate(all="ignore"):
            r = c()
        if r or r is np.True_:
            return True
    return False


def test_unmutated_oracle_passes_the_same_checks():
    assert not _caught(O.paged_attention_decode)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _caught(MUTANTS[name]), name


def test_write_mutant_is_caught():
    # a write that lands one slot late must break the rebuilt logical tokens
    c = make_fork_case("m-fork", [9, 9, 9, 9, 6, 13], 1, 4, 6, 3, 8, 4, "bf16", 6,
                       keep_logical=True)
    kc, vc = O.copy_blocks(c.copy_pairs, c.k_cache, c.v_cache)
    kc, vc = O.kv_cache_write(c.k_new, c.v_new, c.slot_mapping + 1, kc, vc, c.block_size)
    s, L = 4, int(c.context_lens[4])
    pos = np.arange(L)
    phys = c.block_tables[s][pos // c.block_size]
    assert not np.array_equal(kc[phys, :, pos % c.block_size], c.logical_k[s])
