"""The host rule that picks a decode launch's KV read cache policy (pkv_decode_kv_policy).

A launch reads, for each sequence b, the in-pool table entries its length reaches; the rule
takes the default cache policy (KV_CACHED) when those reads name at least twice as many
blocks as are distinct, i.e. at least half of them repeat a block another read names (forked
sequences, a long common prefix: P1 §6.1-6.2, P3 §2.2.8), and the non-temporal one otherwise.
"""
import numpy as np
import pytest

import paged_kv_cache_402_amd as pk
from workloads import gen


def _policy(tables, lens, bs, nb):
    return pk.decode_kv_policy(np.asarray(tables, np.int32), np.asarray(lens, np.int32), bs, nb)


def test_private_blocks_stream_and_an_empty_batch_streams():
    assert _policy(np.zeros((0, 4)), [], 16, 10) == pk.KV_STREAM
    assert _policy([[0, 1, 2], [3, 4, 5]], [48, 40], 16, 6) == pk.KV_STREAM


def test_two_sequences_on_the_same_blocks_are_exactly_half_repeats():
    # 6 reads of 3 distinct blocks: reads == 2 x distinct, the boundary case is cached
    assert _policy([[0, 1, 2], [0, 1, 2]], [48, 48], 16, 3) == pk.KV_CACHED
    # one block fewer repeated: 6 reads of 4 distinct blocks
    assert _policy([[0, 1, 2], [0, 1, 3]], [48, 48], 16, 4) == pk.KV_STREAM


def test_only_reads_within_the_length_and_the_pool_count():
    # sequence 1 lists sequence 0's blocks past its length (never read): 3 + 1 reads, 3 blocks
    assert _policy([[0, 1, 2], [0, 1, 2]], [48, 16], 16, 3) == pk.KV_STREAM
    # out-of-pool entries (-1 and NB) are skipped by the kernel and not counted: the reads
    # left are the same three blocks twice
    assert _policy([[0, 1, 2, -1], [0, 1, 2, 9]], [64, 64], 16, 9) == pk.KV_CACHED
    # lengths clamp to the table (as the kernel clamps them); negative lengths read nothing
    assert _policy([[0, 1], [0, 1], [2, 3]], [10_000, 32, -5], 16, 4) == pk.KV_CACHED


def test_three_sequences_two_of_them_forked():
    # 9 reads of 6 distinct blocks: a third repeats, so stream
    assert _policy([[0, 1, 2], [0, 1, 2], [3, 4, 5]], [48, 48, 48], 16, 6) == pk.KV_STREAM
    # a fourth branch of the fork: 12 reads of 6 blocks
    assert _policy([[0, 1, 2], [0, 1, 2], [3, 4, 5], [0, 1, 2]], [48] * 4, 16, 6) == pk.KV_CACHED


@pytest.mark.parametrize("seed", range(20))
def test_random_tables_against_a_count_of_distinct_reads(seed):
    rng = np.random.default_rng(9100 + seed)
    B, W, bs, nb = int(rng.integers(1, 30)), int(rng.integers(1, 12)), 8, int(rng.integers(1, 40))
    tables = rng.integers(-2, nb + 2, size=(B, W)).astype(np.int32)
    lens = rng.integers(-3, W * bs + 20, size=B).astype(np.int32)
    reads = []
    for b in range(B):
        n = -(-min(max(int(lens[b]), 0), W * bs) // bs)
        reads += [int(x) for x in tables[b, :n] if 0 <= x < nb]
    want = pk.KV_CACHED if reads and len(reads) >= 2 * len(set(reads)) else pk.KV_STREAM
    assert _policy(tables, lens, bs, nb) == want


def test_bad_arguments_are_rejected():
    from paged_kv_cache_402_amd import _lib
    L = _lib.lib
    t = np.zeros((2, 2), np.int32)
    n = np.zeros(2, np.int32)
    P = np.ctypeslib.as_ctypes_type(np.int32)
    import ctypes
    tp = t.ctypes.data_as(ctypes.POINTER(P))
    lp = n.ctypes.data_as(ctypes.POINTER(P))
    assert L.pkv_decode_kv_policy(tp, lp, 2, 2, 16, 0, None, 0, 0) == -1     # no pool
    assert L.pkv_decode_kv_policy(tp, lp, 2, 2, 12, 4, None, 0, 0) == -1     # block size not 2^k
    assert L.pkv_decode_kv_policy(tp, lp, -1, 2, 16, 4, None, 0, 0) == -1
    assert L.pkv_decode_kv_policy(None, lp, 2, 2, 16, 4, None, 0, 0) == -1
    assert L.pkv_decode_kv_policy(tp, lp, 2, 2, 16, 4, lp, -1, 32) == -1     # negative length
    assert L.pkv_decode_kv_policy(tp, lp, 2, 2, 16, 4, lp, 1, 24) == -1      # part % bs != 0
    assert L.pkv_decode_kv_policy(tp, lp, 2, 2, 16, 4, lp, 1, 0) == -1       # list, no part
    assert L.pkv_decode_kv_policy(None, None, 0, 2, 16, 4, None, 0, 0) == pk.KV_STREAM
    with pytest.raises(ValueError):
        pk.decode_kv_policy(np.zeros(4, np.int32), np.zeros(4, np.int32), 16, 4)


def test_the_bench_workloads_get_the_policy_their_sharing_calls_for():
    """GQA 8B (a 512-token prefix shared by all 256 sequences, private suffixes of mean 1824
    tokens: about a fifth of the reads repeat) streams; a 4096-token prefix under short
    suffixes, and four branches forked from each prompt, are mostly repeats and take the
    default policy; batches without sharing stream."""
    for name, want in (("llama3_8b_gqa_prefix", pk.KV_STREAM), ("llama2_7b_mha", pk.KV_STREAM),
                       ("long_context_splitk", pk.KV_STREAM),
                       ("llama3_8b_short_batch", pk.KV_STREAM),
                       ("llama3_8b_long_shared_prefix", pk.KV_CACHED)):
        c = gen.WORKLOADS[name](values=False)
        assert _policy(c.block_tables, c.seq_lens, c.block_size, c.num_blocks) == want, name
    c = gen.llama13b_longtail_case(values=False)
    bm = pk.BlockManager(c.num_blocks, c.block_size, c.free_order)
    for g, L in enumerate(c.decode_lens.tolist()):
        bm.add_seq(g * c.branches, L - 1)
        for br in range(1, c.branches):
            bm.fork(g * c.branches, g * c.branches + br)
    bm.append_step(range(c.num_seqs))
    tables, lens = bm.build_tables(range(c.num_seqs), c.table_width)
    assert _policy(tables, lens, c.block_size, c.num_blocks) == pk.KV_CACHED


def test_a_work_list_counts_only_the_partitions_it_names():
    # two sequences on the same four blocks (block 16, partitions of 32 tokens = 2 blocks)
    tab = [[0, 1, 2, 3], [0, 1, 2, 3]]
    lens = [64, 64]
    assert _policy(tab, lens, 16, 4) == pk.KV_CACHED
    both = np.array([(0 << 16) | 0, (0 << 16) | 1, (1 << 16) | 0, (1 << 16) | 1], np.int32)
    assert pk.decode_kv_policy(tab, lens, 16, 4, work_list=both, partition_size=32) == pk.KV_CACHED
    # sequence 1's first partition left to another pass: 6 reads of 4 blocks
    some = both[[0, 1, 3]]
    assert pk.decode_kv_policy(tab, lens, 16, 4, work_list=some, partition_size=32) == pk.KV_STREAM
    # items past a sequence's end or naming no sequence of the batch read nothing
    extra = np.concatenate([some, np.array([(0 << 16) | 5, (9 << 16) | 0], np.int32)])
    assert pk.decode_kv_policy(tab, lens, 16, 4, work_list=extra, partition_size=32) == pk.KV_STREAM


@pytest.mark.parametrize("seed", range(6))
def test_plain_and_packed_lists_count_the_same_reads_as_no_list(seed):
    rng = np.random.default_rng(9200 + seed)
    B, bs, part = int(rng.integers(2, 40)), 16, 256
    lens = rng.integers(0, 700, size=B).astype(np.int32)
    W = int(-(-max(int(lens.max()), 1) // bs))
    nb = int(rng.integers(W, 3 * B * W))
    tables = rng.integers(0, nb, size=(B, W)).astype(np.int32)
    want = _policy(tables, lens, bs, nb)
    plain = pk.decode_work_list(lens, W, bs, part)
    assert pk.decode_kv_policy(tables, lens, bs, nb, work_list=plain, partition_size=part) == want
    packed, rows = pk.decode_work_list_packed(lens, W, bs, part, 64)
    assert pk.decode_kv_policy(tables, lens, bs, nb, work_list=packed, partition_size=part) == want


def test_the_shared_prefix_plan_leaves_its_partitions_out():
    """The 4096-token common prefix under short suffixes: over every token it is mostly
    repeats (cached), but the per-partition pass of the shared-prefix plan reads only the
    private suffixes (stream)."""
    c = gen.llama3_8b_long_shared_prefix_case(values=False)
    part = 1024
    assert _policy(c.block_tables, c.seq_lens, c.block_size, c.num_blocks) == pk.KV_CACHED
    mem, pp, items = pk.plan_shared_prefix(c.block_tables, c.seq_lens, c.block_size, part)
    assert pp > 0 and mem.shape[0] == c.num_seqs
    assert pk.decode_kv_policy(c.block_tables, c.seq_lens, c.block_size, c.num_blocks,
                               work_list=items, partition_size=part) == pk.KV_STREAM
