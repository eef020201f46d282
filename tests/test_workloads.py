"""Structure of the seeded workloads (CPU only)."""
import numpy as np
import pytest

from oracle import oracle as O
from workloads import make_case, make_fork_case, make_prefix_case
from workloads.generate import config_lengths


def _used_entries(c):
    B = c.block_size
    return [c.block_tables[s, : -(-int(L) // B)] for s, L in enumerate(c.context_lens)]


def test_documented_length_statistics():
    # totals quoted in the design notes for seed = config index
    sums = {c: int(config_lengths(c, np.random.default_rng(c)).sum()) for c in range(5)}
    assert sums == {0: 151, 1: 143905, 2: 403707, 3: 262144, 4: 540693}
    L2 = config_lengths(2, np.random.default_rng(2))
    assert (L2.min(), L2.max(), int((L2 == 8192).sum())) == (89, 8192, 5)


def test_config0_structure():
    c = make_case(0)
    assert c.context_lens.tolist() == [1, 17, 33, 100]
    assert c.num_blocks == 64 and c.max_blocks_per_seq == 7
    used = np.concatenate(_used_entries(c))
    assert len(used) == 13 and len(set(used.tolist())) == 13
    assert c.poison_block not in used
    assert np.isnan(c.k_cache[c.poison_block]).all()
    assert c.scale == np.float32(0.125)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_prefix_structure(B):
    lens = [1, 2, 5, 9, 16, 17, 18, 20, 33, 3, 40, 12]
    c = make_prefix_case("p", lens, 4, 16, 4, 2, 8, B, "bf16", 5)
    pb = 16 // B
    for s, L in enumerate(lens):
        n = L - 1
        jn = n // B
        shared = min(jn, pb)
        g0 = (s // 4) * 4
        # the shared prefix blocks are the same physical ids for every group member
        for t in range(g0, g0 + 4):
            m = min(shared, min((lens[t] - 1) // B, pb))
            assert np.array_equal(c.block_tables[s, :m], c.block_tables[t, :m])
        # the new token's block is never shared
        others = [c.block_tables[t, : -(-lens[t] // B)] for t in range(len(lens)) if t != s]
        assert c.block_tables[s, jn] not in np.concatenate(others)
        # slot mapping of the new token follows the table
        assert c.slot_mapping[s] == O.slot_of(c.block_tables[s], n, B)
    # copy pairs: one per sequence whose new token lands in a partly filled prefix block
    want = sum(1 for L in lens if (L - 1) // B < pb and (L - 1) % B != 0)
    assert len(c.copy_pairs) == want
    dst = c.copy_pairs[:, 1].tolist()
    assert len(set(dst)) == len(dst) and not set(dst) & set(c.copy_pairs[:, 0].tolist())


def test_fork_structure():
    lens = [9, 9, 9, 9, 6, 6, 6, 6, 1, 13, 4, 30]
    c = make_fork_case("f", lens, 2, 4, 6, 3, 8, 4, "bf16", 6)
    B = 4
    assert len(c.copy_pairs) == 2 * 3
    for g in range(2):
        sib = range(4 * g, 4 * g + 4)
        L = int(c.context_lens[4 * g])
        assert all(int(c.context_lens[s]) == L for s in sib)
        assert (L - 1) % B != 0
        nb = -(-L // B)
        pre = [c.block_tables_pre[s, :nb] for s in sib]
        assert all(np.array_equal(pre[0], p) for p in pre)
        post = [c.block_tables[s, :nb] for s in sib]
        assert len({int(p[-1]) for p in post}) == 4  # every sibling ends in its own block
        assert int(post[3][-1]) == int(pre[0][-1])  # the last sibling keeps the original
    slots = c.slot_mapping.tolist()
    assert len(set(slots)) == len(slots)


def test_config4_counts():
    c = make_case(4, poison=False)
    assert c.num_seqs == 512 and len(c.copy_pairs) == 48 and len(c.slot_mapping) == 512
    assert c.max_blocks_per_seq == 128
    assert int(c.context_lens.max()) <= 128 * 16
