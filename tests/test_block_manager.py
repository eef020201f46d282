"""The host block manager (include/pagedattn_blocks.h) on the CPU, against the
pages' worked examples and the invariants of paging and copy-on-write:

* the after-paging pool picture of the devpress.csdn.net/amd walkthrough
  ("关键设计一"): A's table [0, 2, 5, 8], B's [1, 4, 9], blocks 3, 6, 7 free;
* slots = table[t // B] * B + t % B (chenxutan.com deep-dive, section 2.1),
  checked against the oracle's slot_of;
* a sequence wastes less than one block (same two places);
* the 64% utilisation of contiguous reservation ("先理解问题") against the
  paged pool's;
* forks share every block; appending into a shared last block copies it
  first, n-1 copies for n siblings ("关键设计二");
* blocks return to the pool when no table holds them; out of memory leaves
  the state unchanged.
"""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_cache_386_amd", "libpagedattn.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpagedattn.so not built")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bm(nb, B):
    from paged_kv_cache_386_amd import BlockManager
    return BlockManager(nb, B)


def _status(e):
    return e.value.status


def test_free_list_hands_out_the_last_block_first():
    bm = _bm(8, 16)
    bm.add_sequence(1, 40)
    assert bm.block_table(1).tolist() == [7, 6, 5]
    assert bm.num_free_blocks() == 5


def test_page3_pool_picture():
    g = json.load(open(os.path.join(GOLDEN, "page3_pool_picture.json")))
    B = g["block_size"]
    NB = len(g["pool"])
    bm = _bm(NB, B)
    # reverse the free list so that blocks are handed out 0, 1, 2, ...: one
    # sequence takes all blocks (NB-1 first) and gives them back in order
    bm.add_sequence(99, NB * B)
    bm.free_sequence(99)
    # the interleaving of the picture: A1 B1 A2 C B2 A3 D D A4 B3, then C, D end
    bm.add_sequence(ord("A"), B)
    bm.add_sequence(ord("B"), B)
    for _ in range(B):
        bm.append_slot(ord("A"))
    bm.add_sequence(ord("C"), B)
    for _ in range(B):
        bm.append_slot(ord("B"))
    for _ in range(B):
        bm.append_slot(ord("A"))
    bm.add_sequence(ord("D"), 2 * B)
    for _ in range(B):
        bm.append_slot(ord("A"))
    for _ in range(B):
        bm.append_slot(ord("B"))
    bm.free_sequence(ord("C"))
    bm.free_sequence(ord("D"))
    assert bm.block_table(ord("A")).tolist() == g["tables"]["A"]
    assert bm.block_table(ord("B")).tolist() == g["tables"]["B"]
    assert bm.num_free_blocks() == len(g["free"])
    # the free blocks are exactly the picture's holes: allocating them back
    bm.add_sequence(7, len(g["free"]) * B)
    assert sorted(bm.block_table(7).tolist()) == g["free"]


@pytest.mark.parametrize("B", [1, 4, 16, 512])
def test_slots_follow_the_block_table(B):
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 3000, size=6).tolist()
    bm = _bm(sum(-(-(L + 2 * B + 3) // B) for L in lens), B)
    for sid, L in enumerate(lens):
        slots = bm.add_sequence(sid, L)
        table = bm.block_table(sid)
        assert len(table) == -(-L // B)  # ceil: waste below one block
        assert len(table) * B - L < B
        assert slots.tolist() == [O.slot_of(table, t, B) for t in range(L)]
        for t in range(L, L + 2 * B + 3):
            slot, src, dst = bm.append_slot(sid)
            assert (src, dst) == (-1, -1)
            table = bm.block_table(sid)
            assert slot == O.slot_of(table, t, B)
            assert len(table) == t // B + 1  # a new block exactly when t % B == 0
        assert bm.context_len(sid) == L + 2 * B + 3


def test_page1_block_table_example():
    g = json.load(open(os.path.join(GOLDEN, "page1_block_table.json")))
    B = g["block_size"]
    want = g["logical_to_physical"]
    # make the free list hand out #7, #3, #21 next: hold every block in a
    # one-block sequence, then free them with those three last (the last
    # freed block is handed out first)
    bm2 = _bm(32, B)
    ids = {}
    for sid in range(2000, 2032):
        bm2.add_sequence(sid, B)
        ids[int(bm2.block_table(sid)[0])] = sid
    order = [b for b in range(32) if b not in want] + want[::-1]
    for b in order:
        bm2.free_sequence(ids[b])
    slots = bm2.add_sequence(1, 48)
    assert bm2.block_table(1).tolist() == want
    for j, (lo, hi) in enumerate(g["token_ranges"]):
        assert slots[lo] == want[j] * B and slots[hi] == want[j] * B + B - 1
    assert slots[20] == 3 * B + 4  # token 20: logical block 1 -> #3, offset 4


def test_utilisation_against_contiguous_reservation():
    g = json.load(open(os.path.join(GOLDEN, "page3_utilisation.json")))
    used, reserved = g["context_tokens"], g["reserved_tokens"]
    contiguous = sum(used) / sum(reserved)
    assert round(contiguous, 2) == g["utilisation_printed"]
    B = 16
    bm = _bm(sum(-(-r // B) for r in reserved), B)
    for sid, L in enumerate(used):
        bm.add_sequence(sid, L)
    st = bm.stats()
    blocks = sum(-(-L // B) for L in used)
    assert st.slots_allocated == blocks * B
    assert st.tokens_stored == sum(used) == st.tokens_logical
    assert st.utilisation == pytest.approx(sum(used) / (blocks * B))
    assert st.utilisation > 0.99 > contiguous
    assert st.free_blocks == bm.num_blocks - blocks


@pytest.mark.parametrize("n", [2, 3, 4])
@pytest.mark.parametrize("L", [37, 48])
def test_fork_shares_then_copies_on_write(n, L):
    B = 16
    bm = _bm(64, B)
    bm.add_sequence(0, L)
    for c in range(1, n):
        bm.fork(0, c)
    parent = bm.block_table(0).tolist()
    st = bm.stats()
    assert st.free_blocks == 64 - len(parent)  # forking takes no block
    assert st.shared_blocks == len(parent)
    assert st.tokens_stored == L and st.tokens_logical == n * L
    copies = []
    for c in range(n):
        slot, src, dst = bm.append_slot(c)
        table = bm.block_table(c).tolist()
        assert slot == O.slot_of(table, L, B)
        if (src, dst) != (-1, -1):
            copies.append((src, dst))
            assert src == parent[-1] and dst == table[-1] != parent[-1]
        assert table[:-1] == parent[:-1] if L % B else table[:-1] == parent
    if L % B:
        # a partly filled shared last block: every sibling but the last copies it
        assert len(copies) == n - 1
        assert len({d for _, d in copies}) == n - 1
        assert bm.num_free_blocks() == 64 - len(parent) - (n - 1)
    else:
        # the new position opens a block: each sibling takes its own, no copy
        assert copies == []
        assert bm.num_free_blocks() == 64 - len(parent) - n
    # the history blocks stay shared by all n
    assert bm.stats().shared_blocks == len(parent) - (1 if L % B else 0)


def test_free_returns_blocks_only_when_unreferenced():
    bm = _bm(16, 4)
    bm.add_sequence(1, 10)  # 3 blocks
    bm.fork(1, 2)
    bm.free_sequence(1)
    assert bm.num_free_blocks() == 13  # still held by the child
    bm.free_sequence(2)
    assert bm.num_free_blocks() == 16
    from paged_kv_cache_386_amd import PagedAttnError
    with pytest.raises(PagedAttnError) as e:
        bm.free_sequence(2)
    assert _status(e) == -9


def test_out_of_memory_changes_nothing():
    from paged_kv_cache_386_amd import PagedAttnError
    bm = _bm(4, 4)
    assert bm.can_allocate(16) and not bm.can_allocate(17)
    with pytest.raises(PagedAttnError) as e:
        bm.add_sequence(1, 17)
    assert _status(e) == -8 and bm.num_free_blocks() == 4
    bm.add_sequence(1, 16)
    with pytest.raises(PagedAttnError) as e:
        bm.append_slot(1)
    assert _status(e) == -8 and bm.context_len(1) == 16
    with pytest.raises(PagedAttnError) as e:
        bm.add_sequence(1, 0)
    assert _status(e) == -10


def test_prepare_decode_is_all_or_nothing():
    from paged_kv_cache_386_amd import PagedAttnError
    B = 4
    bm = _bm(10, B)
    bm.add_sequence(1, 6)   # 2 blocks, last one half full
    bm.fork(1, 2)
    bm.fork(1, 3)
    bm.add_sequence(4, 8)   # 2 blocks, full: its append opens a block
    assert bm.num_free_blocks() == 6
    # siblings 1 and 2 copy (3 writes in place), 4 takes a block: 3 blocks
    slots, pairs, tables, lens = bm.prepare_decode([1, 2, 3, 4], max_blocks=5, pad_block=9)
    assert len(pairs) == 2 and bm.num_free_blocks() == 3
    assert lens.tolist() == [7, 7, 7, 9]
    for i, sid in enumerate([1, 2, 3, 4]):
        t = bm.block_table(sid).tolist()
        assert tables[i, :len(t)].tolist() == t and (tables[i, len(t):] == 9).all()
        assert slots[i] == O.slot_of(t, lens[i] - 1, B)
    assert len(set(slots.tolist())) == 4
    # a step that needs more blocks than are free fails and changes nothing
    for sid in (5, 6, 7):
        bm.add_sequence(sid, 4)  # one full block each: the pool is now empty
    assert bm.num_free_blocks() == 0
    before = [(s, bm.context_len(s)) for s in (1, 2, 3, 4)]
    free = bm.num_free_blocks()
    with pytest.raises(PagedAttnError) as e:
        bm.prepare_decode([4, 5, 6], max_blocks=5)
    assert _status(e) == -8
    assert [(s, bm.context_len(s)) for s in (1, 2, 3, 4)] == before
    assert bm.num_free_blocks() == free
    with pytest.raises(PagedAttnError) as e:
        bm.prepare_decode([1, 1], max_blocks=5)
    assert _status(e) == -10
    with pytest.raises(PagedAttnError) as e:
        bm.prepare_decode([42], max_blocks=5)
    assert _status(e) == -9
    with pytest.raises(PagedAttnError) as e:
        bm.prepare_decode([1], max_blocks=1)
    assert _status(e) == -2


def test_random_workload_keeps_every_invariant():
    """Random admissions, forks, appends and frees: slots stay unique across
    live sequences (no two tokens share a slot unless their blocks are shared
    history), reference counts match the tables, and the pool is conserved."""
    rng = np.random.default_rng(5)
    B, NB = 8, 400
    bm = _bm(NB, B)
    live = {}
    nxt = 0
    from paged_kv_cache_386_amd import PagedAttnError
    for step in range(400):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                L = int(rng.integers(0, 60))
                bm.add_sequence(nxt, L)
                live[nxt] = L
                nxt += 1
            elif op == 1:
                p = int(rng.choice(list(live)))
                bm.fork(p, nxt)
                live[nxt] = live[p]
                nxt += 1
            elif op == 2:
                ids = list(live)
                rng.shuffle(ids)
                ids = ids[:int(rng.integers(1, len(ids) + 1))]
                slots, pairs, tables, lens = bm.prepare_decode(ids, max_blocks=64)
                for sid, L in zip(ids, lens.tolist()):
                    live[sid] += 1
                    assert live[sid] == L
                # the step's new tokens never share a slot
                assert len(set(slots.tolist())) == len(ids)
                # copies go to blocks no other live table holds
                dsts = set(pairs[:, 1].tolist())
                holders = {}
                for sid in live:
                    for b in bm.block_table(sid).tolist():
                        holders.setdefault(b, []).append(sid)
                for d in dsts:
                    assert len(holders[d]) == 1
            else:
                sid = int(rng.choice(list(live)))
                bm.free_sequence(sid)
                del live[sid]
        except PagedAttnError as e:
            assert e.status == -8  # out of memory is the only expected failure
        held = set()
        for sid, L in live.items():
            t = bm.block_table(sid).tolist()
            assert len(t) == -(-L // B) and bm.context_len(sid) == L
            held |= set(t)
        assert bm.num_free_blocks() == NB - len(held)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B,NB,seed", [
    ("bf16", 4, 2, 16, 4, 400, 1),
    ("f32", 2, 1, 8, 8, 200, 2),
    ("bf16", 4, 2, 16, 4, 40, 3),   # small pool: steps preempt
])
def test_serving_loop_on_the_oracle(dtype, Hq, Hkv, D, B, NB, seed):
    """The block manager drives the oracle's cache edits and decode through a
    continuously batched loop: the pool read through the tables holds every
    sequence's tokens, and paged decode equals dense attention over them."""
    from serving_loop import Loop, OracleBackend, drive
    loop = Loop(OracleBackend(), dtype, Hq, Hkv, D, B, NB, max_blocks=64, seed=seed)
    drive(loop, steps=16, partition_size=0, max_prompt=60, admit_p=0.8 if NB < 100 else 0.3)
    assert loop.copies > 0 and loop.steps == 16
    if NB < 100:
        assert loop.preempted > 0


@pytest.mark.parametrize("dtype,Hq,Hkv,D,B,NB,max_batch,seed", [
    ("bf16", 4, 2, 64, 4, 300, 16, 1),
    ("f32", 2, 1, 64, 8, 120, 32, 2),
    ("bf16", 4, 2, 64, 4, 60, 12, 3),   # small pool: preemption
])
def test_engine_plans_on_the_oracle(dtype, Hq, Hkv, D, B, NB, max_batch, seed):
    """The engine's scheduler and planning (plan-only mode) drive the oracle's
    edits and decode: FCFS admission, forks for parallel samples, finishes,
    preemption with recompute; every request gets exactly its tokens."""
    from serving_loop import EngineHarness, drive_engine
    h = EngineHarness("oracle", dtype, Hq, Hkv, D, B, NB, max_batch, max_ctx=96, seed=seed)
    drive_engine(h, num_requests=40, seed=seed, max_prompt=60, max_new=30)
    assert h.copies > 0 and h.admitted >= 40
    if NB < 100:
        assert h.preempted > 0


def _plan_engine(**kw):
    import paged_kv_cache_386_amd as pa
    args = dict(num_q_heads=4, max_batch=8, max_context_len=64, num_blocks=40, block_size=4,
                num_kv_heads=2, head_dim=64)
    args.update(kw)
    return pa.Engine(**args)


def test_engine_submit_checks():
    from paged_kv_cache_386_amd import PagedAttnError
    e = _plan_engine()
    e.submit(1, 10, 5)
    for args, status in [((1, 10, 5), -10),        # id in use
                         ((-1, 10, 5), -10),       # id out of range
                         ((2, 0, 5), -2),          # empty prompt
                         ((2, 60, 5), -2),         # longer than max_context_len
                         ((2, 10, 0), -2),         # no decode step
                         ((2, 10, 5, 9), -2),      # more samples than max_batch
                         ((2, 8, 56, 8), -2)]:     # cannot run alone: 2 + 8*14 blocks
        with pytest.raises(PagedAttnError) as ex:
            e.submit(*args)
        assert _status(ex) == status, args
    assert e.num_waiting() == 1


def test_engine_admits_first_come_first_served():
    e = _plan_engine(max_batch=4)
    e.submit(7, 5, 3)
    e.submit(3, 5, 3, 2)
    e.submit(9, 5, 3, 2)   # does not fit the batch beside the first two
    e.submit(4, 1, 3)      # would fit, but admission stops at the first miss
    info = e.step()
    assert info.admitted_seq_ids.tolist() == [7 << 8, 3 << 8]
    assert info.batch_seq_ids.tolist() == [7 << 8, 3 << 8, (3 << 8) | 1]
    assert e.num_waiting() == 2
    # the fork copies the shared partial prompt block once (5 % 4 != 0)
    assert info.num_copies == 1
    for _ in range(2):
        info = e.step()
    assert sorted(info.finished_seq_ids.tolist()) == [3 << 8, (3 << 8) | 1, 7 << 8]
    info = e.step()
    assert info.admitted_seq_ids.tolist() == [9 << 8, 4 << 8]


def test_engine_preemption_requeues_the_newest_and_admits_nothing():
    # 12 blocks of 4 (watermark 0); two requests of 8 + 20 tokens (7 blocks
    # each at the end) run together until their 25th tokens need 14 blocks
    e = _plan_engine(num_blocks=12, max_batch=4, max_context_len=40)
    e.submit(1, 8, 20)
    e.submit(2, 8, 20)
    preempt_step = readmit = None
    last_len = {}
    for step in range(200):
        if step == 10:
            e.submit(3, 1, 1)  # waits behind nothing, admitted at once
        info = e.step()
        for sid, L in zip(info.batch_seq_ids.tolist(), info.context_lens.tolist()):
            last_len[sid] = L
        if info.preempted:
            assert preempt_step is None
            preempt_step = step
            assert info.preempted_seq_ids.tolist() == [2 << 8]
            assert info.admitted == 0
            assert info.batch_seq_ids.tolist() == [1 << 8]
            held = last_len[2 << 8]
        if preempt_step is not None and (2 << 8) in info.admitted_seq_ids.tolist():
            readmit = step
            rows = info.admitted_rows[info.admitted_seq_ids.tolist().index(2 << 8)]
            assert rows == held  # recomputed whole
        if e.num_running() == 0 and e.num_waiting() == 0:
            break
    assert preempt_step == 16 and readmit is not None and readmit > preempt_step
    assert last_len == {1 << 8: 28, 2 << 8: 28, 3 << 8: 2}
    assert e.block_stats().free_blocks == 12
