"""The host planner of the fork-group decode step (pkv_decode_plan_fork_groups).

Right after a fork (P2 §2.2), the branches of a prompt attend to the same tokens before their
own new one: the same length, the same blocks before the new token's block, and the same
block for that block's earlier rows (the copy source, P1 §6.2, or the block itself for the
branch that kept it). The planner groups exactly those sequences; these tests restate that
definition by brute force over block-manager runs.
"""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_402_amd as pk


def _key(tables, lens, cow, b, bs, nb):
    L = int(lens[b])
    if L <= 0:
        return ("alone", b)
    jb, r = (L - 1) // bs, (L - 1) % bs
    src = -1
    if r:
        c = int(cow[b]) if cow is not None else -1
        src = c if 0 <= c < nb else int(tables[b][jb])
    return (L, tuple(int(x) for x in tables[b][:jb]), src)


def _expected(tables, lens, cow, bs, nb, size):
    runs = {}
    for b in range(len(lens)):
        runs.setdefault(_key(tables, lens, cow, b, bs, nb), []).append(b)
    groups = []
    for members in runs.values():
        for i in range(0, len(members), size):
            groups.append(members[i:i + size])
    groups.sort(key=lambda g: g[0])
    return [g + [-1] * (size - len(g)) for g in groups], [int(lens[g[0]]) for g in groups]


def _fork_batch(rng, bs):
    """Prompts of random lengths forked into random branch counts, some branches grown by a few
    tokens first (so they no longer match their siblings), then one append each."""
    prompts = rng.integers(0, 5 * bs, size=int(rng.integers(1, 12))).tolist()
    branches = rng.integers(1, 6, size=len(prompts)).tolist()
    nb = 16 + sum((L // bs + 3) * br for L, br in zip(prompts, branches)) * 2
    bm = pk.BlockManager(nb, bs, rng.permutation(nb).astype(np.int32))
    seqs = []
    for g, (L, br) in enumerate(zip(prompts, branches)):
        bm.add_seq(100 * g, L)
        seqs.append(100 * g)
        for b in range(1, br):
            bm.fork(100 * g, 100 * g + b)
            seqs.append(100 * g + b)
    for s in seqs:
        if rng.random() < 0.15:
            bm.append_step([s])
    slots, pairs, cow_src = bm.append_step(seqs)
    W = max(5, max(len(bm.table(s)[0]) for s in seqs) + 1)
    tables, lens = bm.build_tables(seqs, W)
    return tables, lens, cow_src, nb


@pytest.mark.parametrize("seed", range(25))
def test_planner_matches_the_definition(seed):
    rng = np.random.default_rng(7700 + seed)
    bs = int(rng.choice([8, 16, 32]))
    tables, lens, cow, nb = _fork_batch(rng, bs)
    for size in (1, 2, 3, 4, 8):
        groups, glens = pk.plan_fork_groups(tables, lens, cow, bs, nb, size)
        want, wlens = _expected(tables, lens, cow, bs, nb, size)
        assert groups.tolist() == want, size
        assert glens.tolist() == wlens


def test_branches_of_one_fork_form_one_group():
    """Three branches of a 37-token prompt (block 16): two copy the shared partial block, the
    third keeps it; a two-branch fork of a 32-token prompt opens fresh blocks (no copy)."""
    bm = pk.BlockManager(40, 16, np.arange(40, dtype=np.int32))
    bm.add_seq(0, 37)
    bm.fork(0, 1)
    bm.fork(0, 2)
    bm.add_seq(5, 32)
    bm.fork(5, 6)
    seqs = [0, 1, 2, 5, 6]
    slots, pairs, cow = bm.append_step(seqs)
    assert (cow >= 0).sum() == 2
    tables, lens = bm.build_tables(seqs, 4)
    groups, glens = pk.plan_fork_groups(tables, lens, cow, 16, 40, 4)
    assert groups.tolist() == [[0, 1, 2, -1], [3, 4, -1, -1]]
    assert glens.tolist() == [38, 33]
    # without the copy sources the copies' last blocks differ: only the fresh-block pair groups
    groups, _ = pk.plan_fork_groups(tables, lens, None, 16, 40, 4)
    assert groups.tolist() == [[0, -1, -1, -1], [1, -1, -1, -1], [2, -1, -1, -1],
                               [3, 4, -1, -1]]


def test_empty_sequences_stay_alone_and_bad_arguments_fail():
    tables = np.zeros((3, 2), np.int32)
    lens = np.array([0, 0, 1], np.int32)
    groups, glens = pk.plan_fork_groups(tables, lens, None, 16, 4, 2)
    assert groups.tolist() == [[0, -1], [1, -1], [2, -1]] and glens.tolist() == [0, 0, 1]
    groups, glens = pk.plan_fork_groups(np.zeros((0, 2), np.int32), np.zeros(0, np.int32),
                                        None, 16, 4, 2)
    assert groups.shape == (0, 2)
    L = pk._lib.lib
    P = ctypes.POINTER(ctypes.c_int32)
    tp = tables.ctypes.data_as(P)
    lp = lens.ctypes.data_as(P)
    assert L.pkv_decode_plan_fork_groups(tp, lp, None, 3, 2, 12, 4, 2, None, None, 0) == -1
    assert L.pkv_decode_plan_fork_groups(tp, lp, None, 3, 2, 16, 0, 2, None, None, 0) == -1
    assert L.pkv_decode_plan_fork_groups(tp, lp, None, 3, 2, 16, 4, 0, None, None, 0) == -1
    assert L.pkv_decode_plan_fork_groups(None, lp, None, 3, 2, 16, 4, 2, None, None, 0) == -1
    assert L.pkv_decode_plan_fork_groups(tp, lp, None, 3, 2, 16, 4, 2, None, None, 0) == 3
    out = np.zeros(6, np.int32)
    gl = np.zeros(3, np.int32)
    assert L.pkv_decode_plan_fork_groups(tp, lp, None, 3, 2, 16, 4, 2, out.ctypes.data_as(P),
                                         gl.ctypes.data_as(P), 2) == -1       # capacity
    assert L.pkv_decode_plan_fork_groups(tp, lp, None, 3, 2, 16, 4, 2, out.ctypes.data_as(P),
                                         None, 3) == -1                       # one output
