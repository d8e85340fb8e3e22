"""Pins of the reference block-manager model (CPU only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理"
"""
import json
import os

import numpy as np

from oracle.block_manager_model import BlockManagerModel, OK, EINVAL, ENOBLOCKS, ENOSEQ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_table_worked_example.json")


def test_worked_example_growth_p3_2_2_3():
    g = json.load(open(GOLDEN))
    bs = g["printed"]["block_size"]
    order = [7, 3, 9, 12] + [b for b in range(32) if b not in (7, 3, 9, 12)]
    m = BlockManagerModel(32, bs, order)
    assert m.add_seq(0, g["printed"]["seq_len"]) == OK
    assert m.table(0) == (g["printed"]["physical_blocks"], 35)
    assert m.slots(0, 0, 35) == g["derived_by_hand"]["slots_of_tokens_0_to_34"]
    got = [m.append_slot(0)[1] for _ in range(13)]
    assert got == g["derived_by_hand"]["slots_of_tokens_35_to_47"]
    assert m.table(0)[0] == [7, 3, 9]           # no new block before token 48
    st, slot, _, _ = m.append_slot(0)
    assert st == OK and slot == g["derived_by_hand"]["slot_of_token_48"]
    assert m.table(0)[0] == [7, 3, 9, 12]       # appended at the end, nothing moved


def test_fork_then_write_copies_exactly_one_block():
    """P1 §6.2: only the written block is copied; the original stays for the other users."""
    m = BlockManagerModel(16, 4)
    assert m.add_seq(1, 10) == OK               # blocks 0,1,2 ; last block holds 2 tokens
    assert m.fork(1, 2) == OK
    assert [m.refcount(b) for b in (0, 1, 2)] == [2, 2, 2]
    st, slot, src, dst = m.append_slot(2)
    assert st == 1 and src == 2 and dst == 3 and slot == 3 * 4 + 2
    assert m.table(1)[0] == [0, 1, 2] and m.table(2)[0] == [0, 1, 3]
    assert [m.refcount(b) for b in (0, 1, 2, 3)] == [2, 2, 1, 1]
    # the last holder writes in place
    st, slot, src, dst = m.append_slot(1)
    assert st == OK and slot == 2 * 4 + 2 and (src, dst) == (-1, -1)
    assert m.stats()["cow_copies"] == 1


def test_fork_at_block_boundary_needs_no_copy():
    m = BlockManagerModel(8, 4)
    m.add_seq(1, 8)
    m.fork(1, 2)
    st, slot, src, dst = m.append_slot(2)
    assert st == OK and src == -1 and slot == 2 * 4
    assert m.refcount(0) == 2 and m.refcount(1) == 2


def test_share_prefix_and_free():
    m = BlockManagerModel(10, 4)
    m.add_seq(1, 9)
    assert m.share_prefix(1, 2, 2) == OK
    assert m.table(2) == ([0, 1], 8)
    assert m.share_prefix(1, 3, 3) == EINVAL    # block 2 is only partly filled
    assert m.free_seq(1) == OK
    assert m.refcount(0) == 1 and m.refcount(2) == 0
    assert m.free_seq(1) == ENOSEQ
    # freed blocks return to the pool (P3 §2.2.2)
    assert m.stats()["free"] == 8


def test_exhaustion_fails_atomically():
    m = BlockManagerModel(4, 4)
    assert m.add_seq(1, 12) == OK
    before = (list(m.free), list(m.rc), {k: (list(v[0]), v[1]) for k, v in m.seqs.items()})
    assert m.add_seq(2, 8) == ENOBLOCKS
    after = (list(m.free), list(m.rc), {k: (list(v[0]), v[1]) for k, v in m.seqs.items()})
    assert before == after and m.stats()["alloc_failures"] == 1
    assert m.add_seq(2, 3) == OK
    assert m.append_slot(2)[0] == OK            # offset 3 of its own block: no allocation
    assert m.append_slot(2)[0] == ENOBLOCKS     # the block is full and the pool is empty
    assert m.stats()["alloc_failures"] == 2
    m2 = BlockManagerModel(2, 2)
    m2.add_seq(1, 2)
    m2.fork(1, 2)
    m2.add_seq(3, 1)
    assert m2.append_slot(1)[0] == ENOBLOCKS    # needs a fresh block, none free
    assert m2.stats()["alloc_failures"] == 1


def test_any_free_block_serves_any_request():
    """P1 §4.1: no external fragmentation. Free every other sequence and allocate a request as
    large as all the freed blocks together: it must succeed."""
    m = BlockManagerModel(64, 4)
    for s in range(16):
        m.add_seq(s, 16)
    for s in range(0, 16, 2):
        m.free_seq(s)
    assert m.stats()["free"] == 32
    assert m.add_seq(100, 128) == OK
    assert m.stats()["free"] == 0


def test_random_ops_keep_invariants():
    rng = np.random.default_rng(0)
    m = BlockManagerModel(48, 4, rng.permutation(48))
    live = []
    next_id = 0
    for _ in range(3000):
        op = rng.integers(0, 5)
        if op == 0:
            m.add_seq(next_id, int(rng.integers(0, 20)))
            if next_id in m.seqs:
                live.append(next_id)
            next_id += 1
        elif op == 1 and live:
            p = live[int(rng.integers(len(live)))]
            if m.fork(p, next_id) == OK:
                live.append(next_id)
            next_id += 1
        elif op == 2 and live:
            m.append_slot(live[int(rng.integers(len(live)))])
        elif op == 3 and live:
            s = live.pop(int(rng.integers(len(live))))
            assert m.free_seq(s) == OK
        elif op == 4 and live:
            src = live[int(rng.integers(len(live)))]
            nb = m.seqs[src][1] // 4
            if m.share_prefix(src, next_id, int(rng.integers(0, nb + 1))) == OK:
                live.append(next_id)
            next_id += 1
        # invariants
        refs = [0] * 48
        for blocks, n in m.seqs.values():
            assert len(blocks) == (n + 3) // 4        # waste below one block per sequence
            for b in blocks:
                refs[b] += 1
        assert refs == m.rc
        assert len(m.free) + sum(1 for r in m.rc if r > 0) == 48
        assert set(m.free).isdisjoint({b for b in range(48) if m.rc[b] > 0})
