"""The ticketed tail of a work list made private (pkv_decode_work_list_private_tail).

A launch over an initialised workspace hands the units of its last workgroups out by ticket,
so they may run on another XCD than their KV head's, away from the L2 that holds the blocks
their sequence shares with others (a common prefix: P1 §6.1, P3 §2.2.8). The reorder puts
private items there. These tests restate the rule by brute force: an item is shared when a
block its tokens read is read more than once by the whole list; if the old tail holds a shared
item, the list's last tail_items private items move to the end in their order, the walk back
stopping at the first private item longer than 5/4 of the old tail's longest; everything else
keeps its order. When no private item from before the tail qualifies, the list stays as it is.
"""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_402_amd as pk
from workloads import gen


def _tokens(item, lens, part, cap):
    b, p = item >> 16, item & 0xFFFF
    L = min(max(int(lens[b]), 0), cap)
    return max(0, min(part, L - p * part))


def _expected(items, tables, lens, bs, nb, part, tail):
    cap = tables.shape[1] * bs
    reads = []
    for it in items:
        b, p = it >> 16, it & 0xFFFF
        n = _tokens(it, lens, part, cap)
        ids = [int(tables[b][j]) for j in range(p * part // bs, (p * part + n + bs - 1) // bs)] \
            if n else []
        reads.append([i for i in ids if 0 <= i < nb])
    count = {}
    for r in reads:
        for i in r:
            count[i] = count.get(i, 0) + 1
    shared = [any(count[i] > 1 for i in r) for r in reads]
    T = min(tail, len(items))
    if T == 0 or not any(shared[len(items) - T:]):
        return list(items), 0
    longest = max(_tokens(it, lens, part, cap) for it in items[len(items) - T:])
    moved = []
    for i in range(len(items) - 1, -1, -1):
        if len(moved) == T:
            break
        if shared[i]:
            continue
        if _tokens(items[i], lens, part, cap) > longest + longest // 4:
            break
        moved.append(i)
    if len(moved) == T - sum(shared[len(items) - T:]):
        return list(items), 0                 # only the tail's own private items qualify
    mset = set(moved)
    out = [it for i, it in enumerate(items) if i not in mset] + \
          [items[i] for i in sorted(moved)]
    sh_after = sum(shared[items.index(it)] for it in out[len(out) - T:])
    return out, sum(shared[len(items) - T:]) - sh_after


def _batch(rng):
    """Random tables with a shared prefix for a random subset, shared single blocks, out-of-pool
    entries, and ragged lengths."""
    bs = int(rng.choice([8, 16, 32]))
    B = int(rng.integers(1, 60))
    W = int(rng.integers(1, 40))
    nb = int(rng.integers(W + 1, 4 * B * W + 2))
    tables = rng.integers(0, nb, size=(B, W)).astype(np.int32)
    pre = int(rng.integers(0, W + 1))
    tables[rng.random(B) < 0.5, :pre] = tables[0, :pre]
    tables[rng.random((B, W)) < 0.03] = -1
    tables[rng.random((B, W)) < 0.02] = nb + 3
    lens = rng.integers(0, W * bs + 1, size=B).astype(np.int32)
    return tables, lens, bs, nb


@pytest.mark.parametrize("seed", range(30))
def test_reorder_matches_the_rule(seed):
    rng = np.random.default_rng(9100 + seed)
    tables, lens, bs, nb = _batch(rng)
    part = int(rng.choice([p for p in (32, 64, 128, 256) if p % bs == 0]))
    items = pk.decode_work_list(lens, tables.shape[1], bs, part)
    for tail in (0, 1, 3, len(items) // 4, len(items) // 2, len(items), len(items) + 5):
        got, moved = pk.decode_work_list_private_tail(items, tables, lens, bs, nb, part, tail)
        want, wmoved = _expected(items.tolist(), tables, lens, bs, nb, part, tail)
        assert got.tolist() == want, tail
        assert moved == wmoved
        assert sorted(got.tolist()) == sorted(items.tolist())


def test_gqa_prefix_workload_tail_is_prefix_free():
    """The GQA 8B batch-256 workload at 2048-token partitions: its 64-item ticketed tail held 12
    items of partition 0 (which read the shared 512-token prefix); after the reorder it holds
    the 64 shortest items of later partitions, which read private blocks only."""
    c = gen.llama3_8b_gqa_prefix_case(values=False)
    items = pk.decode_work_list(c.seq_lens, c.table_width, c.block_size, 2048)
    assert ((items[-64:] & 0xFFFF) == 0).sum() == 12
    got, moved = pk.decode_work_list_private_tail(items, c.block_tables, c.seq_lens,
                                                  c.block_size, c.num_blocks, 2048, 64)
    assert moved == 12
    assert ((got[-64:] & 0xFFFF) >= 1).all()
    later = items[(items & 0xFFFF) >= 1]
    assert got[-64:].tolist() == later[-64:].tolist()
    # every other item keeps its order
    rest = [int(x) for x in items if x not in set(later[-64:].tolist())]
    assert got[:-64].tolist() == rest


def test_nothing_moves_without_private_items_or_shared_tail():
    bs, part = 16, 64
    tables = np.tile(np.arange(8, dtype=np.int32), (4, 1))      # every sequence shares all
    lens = np.array([100, 90, 30, 5], np.int32)
    items = pk.decode_work_list(lens, 8, bs, part)
    got, moved = pk.decode_work_list_private_tail(items, tables, lens, bs, 8, part, 3)
    assert moved == 0 and got.tolist() == items.tolist()
    private = np.arange(32, dtype=np.int32).reshape(4, 8)       # nothing shared
    got, moved = pk.decode_work_list_private_tail(items, private, lens, bs, 32, part, 3)
    assert moved == 0 and got.tolist() == items.tolist()


def test_long_private_items_stay_out_of_the_tail():
    """A shared 2-token item ends the list; the only private item before it holds 64 tokens,
    more than 5/4 of the tail's longest (2): it is not pulled to the end."""
    bs, part = 16, 64
    tables = np.array([[0, 1, 2, 3], [4, 5, 6, 7], [9, 8, 8, 8], [9, 10, 11, 12]], np.int32)
    lens = np.array([64, 30, 2, 2], np.int32)         # sequences 2 and 3 share block 9
    items = pk.decode_work_list(lens, 4, bs, part)
    assert [int(i) >> 16 for i in items] == [0, 1, 2, 3]
    got, moved = pk.decode_work_list_private_tail(items, tables, lens, bs, 16, part, 1)
    assert moved == 0 and got.tolist() == items.tolist()
    # with the private 30-token item a 2-token one (sequence 1 shortened), it moves last
    lens2 = np.array([64, 2, 2, 2], np.int32)
    items2 = pk.decode_work_list(lens2, 4, bs, part)
    got, moved = pk.decode_work_list_private_tail(items2, tables, lens2, bs, 16, part, 1)
    assert moved == 1 and int(got[-1]) >> 16 == 1


def test_bad_arguments_fail():
    L = pk._lib.lib
    P = ctypes.POINTER(ctypes.c_int32)
    tables = np.zeros((2, 2), np.int32)
    lens = np.array([3, 40], np.int32)
    items = pk.decode_work_list(lens, 2, 16, 32)
    tp, lp = tables.ctypes.data_as(P), lens.ctypes.data_as(P)
    ip = items.ctypes.data_as(P)
    n = items.shape[0]
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 16, 4, 32, 1, ip, n) >= 0
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 16, 4, 32, -1, ip, n) < 0
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 16, 0, 32, 1, ip, n) < 0
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 12, 4, 32, 1, ip, n) < 0
    assert L.pkv_decode_work_list_private_tail(None, lp, 2, 2, 16, 4, 32, 1, ip, n) < 0
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 16, 4, 32, 1, None, n) < 0
    bad = np.array([5 << 16], np.int32)                        # names sequence 5 of 2
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 16, 4, 32, 1,
                                               bad.ctypes.data_as(P), 1) < 0
    packed, rows = pk.decode_work_list_packed(lens, 2, 16, 32, 8)
    assert (packed < 0).any()                                   # holds a packed row
    assert L.pkv_decode_work_list_private_tail(tp, lp, 2, 2, 16, 4, 32, 1,
                                               packed.ctypes.data_as(P), packed.shape[0]) < 0
    with pytest.raises(ValueError):
        pk.decode_ticketed_items(np.float32, 128, 32, 8, 16, 2048, 10)
    with pytest.raises(ValueError):
        import torch
        pk.decode_ticketed_items(torch.bfloat16, 128, 32, 8, 16, 2048, 10, kind="other")
    # argument checks run before the occupancy query, so they fail without a device too
    for args in ((2, 96, 32, 8, 16, 2048, 10, 0, 1), (2, 128, 32, 8, 12, 2048, 10, 0, 1),
                 (2, 128, 32, 8, 16, 4096, 10, 0, 1), (2, 256, 64, 8, 16, 2048, 10, 0, 1),
                 (2, 128, 32, 8, 16, 2048, 10, 2, 3), (2, 128, 32, 8, 16, 2048, -1, 0, 1),
                 (2, 128, 32, 8, 16, 2048, 10, 5, 1), (7, 128, 32, 8, 16, 2048, 10, 0, 1)):
        assert L.pkv_decode_ticketed_items(*args) < 0, args
    assert L.pkv_decode_ticketed_items(2, 128, 32, 8, 16, 2048, 0, 0, 1) == 0   # empty list
