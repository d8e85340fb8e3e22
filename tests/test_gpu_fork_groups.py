"""GPU parity of the fork-group decode step (MI355X only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html

The branches of a parallel-sampling fork (P2 §2.2) share their prompt's blocks until each
writes its own token; the first write into a shared partial block copies it (P1 §6.2). The
fork-group step reads the shared tokens once per group for all members' query rows. It must
leave bitwise the caches of the per-sequence one-pass step (itself bitwise copy_blocks, then
reshape_and_cache, then the decode, checked in test_gpu_cache_ops.py), and outputs that agree
with it to fp32 rounding and with the oracle within the parity gate.
"""
import numpy as np
import pytest
import torch

from workloads import gen
from tests.gpu_util import GATE, i32, max_err, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_402_amd  # noqa: F401


def pk():
    import paged_kv_cache_402_amd
    return paged_kv_cache_402_amd


def _forked_batch(P, rng, dtype, hkv, d, bs, prompts, branches):
    """Prompts written into a NaN-filled pool, forked into branches, then one append each.
    Returns (pool, seqs, slots, pairs, cow_src, tables, lens, W)."""
    nb = 8 + sum(-(-(L + 1) // bs) * br + 1 for L, br in zip(prompts, branches))
    bm = P.BlockManager(nb, bs, rng.permutation(nb).astype(np.int32))
    kd = to_dev(np.full((nb, hkv, bs, d), gen.nan_value(dtype),
                        dtype=gen.storage_numpy_dtype(dtype)), dtype)
    vd = kd.clone()
    seqs = []
    for g, (L, br) in enumerate(zip(prompts, branches)):
        parent = 10 * g
        bm.add_seq(parent, L)
        if L:
            P.reshape_and_cache(to_dev(gen.normal(rng, (L, hkv, d), dtype), dtype),
                                to_dev(gen.normal(rng, (L, hkv, d), dtype), dtype), kd, vd,
                                i32(bm.slots(parent, 0, L)))
        seqs.append(parent)
        for b in range(1, br):
            bm.fork(parent, parent + b)
            seqs.append(parent + b)
    slots, pairs, cow_src = bm.append_step(seqs)
    W = max(-(-(L + 1) // bs) for L in prompts) + 1
    tables, lens = bm.build_tables(seqs, W)
    return nb, kd, vd, seqs, slots, pairs, cow_src, tables, lens, W


def _work(P, glens, W, bs, part, form):
    if form == "list":
        return i32(P.decode_work_list(glens, W, bs, part))
    lst, rows = P.decode_work_list_packed(glens, W, bs, part, part // 4)
    return (i32(lst), rows)


@pytest.mark.parametrize("dtype,hq,hkv,bs,part,form,group,hd", [
    ("bf16", 32, 8, 16, 512, "list", 2, 0),      # 4 heads x 2 members: 8 rows
    ("f16", 40, 40, 32, 2048, "packed", 4, 0),   # MHA, 4 members
    ("f32", 8, 4, 8, 64, "list", 4, 0),          # 2 heads x 4 members, many partitions
    ("bf16", 16, 16, 16, 256, "packed", 8, 0),   # MHA, 8 members (groups of 4 padded)
    ("f16", 32, 8, 16, 512, "list", 1, 0),       # one member: the per-sequence rows
    ("bf16", 64, 8, 64, 1024, "list", 1, 0),     # 8 query heads per KV head, one member
    ("f32", 16, 8, 16, 256, "packed", 2, 0),     # head_dim 256 (f32 rows of 1 KiB), 2 x 2 rows
    ("bf16", 16, 8, 16, 256, "list", 2, 64),     # head_dim 64, 2 heads x 2 members
    ("f16", 8, 8, 16, 512, "packed", 2, 256),    # head_dim 256 16-bit rows, 2 members
])
def test_group_step_matches_the_per_sequence_step(dtype, hq, hkv, bs, part, form, group, hd):
    """Prompts of many lengths (a partial last block, a full one, empty, longer than a
    partition) forked into 1-4 branches, then one token each. The groups come from the
    planner; the group step must leave the per-sequence fused step's caches bit for bit, and
    outputs within fp32 rounding of it and within the gate of the oracle. Unwritten slots hold
    NaN, so a read of a row before it is written would show."""
    P = pk()
    rng = np.random.default_rng(90 + group + hq)
    d = hd or (128 if dtype != "f32" else (256 if hq == 16 else 64))
    prompts = [3 * bs - 3, 2 * bs, part + 5, 1, 0, bs + 1, 2 * part - 1, 7]
    branches = [4, 3, 2, 1, 2, 4, 3, 1]
    nb, kd, vd, seqs, slots, pairs, cow_src, tables, lens, W = _forked_batch(
        P, rng, dtype, hkv, d, bs, prompts, branches)
    B = len(seqs)
    groups, glens = P.plan_fork_groups(tables, lens, cow_src, bs, nb, group)
    # every sequence is in exactly one group, and the branches of a prompt share one
    members = groups[groups >= 0]
    assert sorted(members.tolist()) == list(range(B))
    if group >= 2:
        assert groups.shape[0] < B
    q = to_dev(gen.normal(rng, (B, hq, d), dtype), dtype)
    k_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    v_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    # per-sequence one-pass step
    k1, v1 = kd.clone(), vd.clone()
    o1 = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    P.paged_attention_decode_step(o1, q, k_new, v_new, i32(cow_src), k1, v1, i32(tables),
                                  i32(lens), scale, partition_size=part,
                                  work_list=i32(P.decode_work_list(lens, W, bs, part)))
    # fork groups
    k2, v2 = kd.clone(), vd.clone()
    o2 = torch.full_like(o1, float("nan"))
    P.paged_attention_decode_step_groups(o2, q, k_new, v_new, i32(cow_src), k2, v2, i32(tables),
                                         i32(lens), scale, i32(groups),
                                         _work(P, glens, W, bs, part, form),
                                         partition_size=part)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
    assert not torch.isnan(o2).any()
    assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)
    ref = gen.PagedDecodeCase("groups", dtype, hq, hkv, d, bs, nb, lens, tables, scale,
                              q=to_host(q, dtype), k_cache=to_host(k2, dtype),
                              v_cache=to_host(v2, dtype))
    assert max_err(o2.cpu().numpy().astype(np.float64), oracle(ref)) <= GATE[dtype]


def test_out_of_pool_shared_entries_are_left_out_for_every_member():
    """A table entry outside the pool in a fork's shared blocks (every member lists it, as forks
    share their entries): the group step leaves that block's tokens out for all members, as the
    per-sequence step does for each."""
    P = pk()
    rng = np.random.default_rng(97)
    dtype, hq, hkv, bs, d, part = "f16", 8, 8, 16, 128, 256
    nb, kd, vd, seqs, slots, pairs, cow_src, tables, lens, W = _forked_batch(
        P, rng, dtype, hkv, d, bs, [5 * bs + 3, 3 * bs + 7], [4, 3])
    B = len(seqs)
    for b in range(4):
        tables[b, 1] = -1                 # the first fork's second block, in every member
    for b in range(4, B):
        tables[b, 0] = nb + 3             # the second fork's first block, past the pool
    groups, glens = P.plan_fork_groups(tables, lens, cow_src, bs, nb, 4)
    assert groups.shape[0] == 2
    q = to_dev(gen.normal(rng, (B, hq, d), dtype), dtype)
    k_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    v_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    outs, caches = [], []
    for grouped in (False, True):
        k2, v2 = kd.clone(), vd.clone()
        o = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
        if grouped:
            P.paged_attention_decode_step_groups(o, q, k_new, v_new, i32(cow_src), k2, v2,
                                                 i32(tables), i32(lens), 0.09, i32(groups),
                                                 i32(P.decode_work_list(glens, W, bs, part)),
                                                 partition_size=part)
        else:
            P.paged_attention_decode_step(o, q, k_new, v_new, i32(cow_src), k2, v2, i32(tables),
                                          i32(lens), 0.09, partition_size=part,
                                          work_list=i32(P.decode_work_list(lens, W, bs, part)))
        torch.cuda.synchronize()
        outs.append(o)
        caches.append((k2, v2))
    assert not torch.isnan(outs[1]).any()
    assert torch.allclose(outs[0], outs[1], rtol=1e-5, atol=1e-6)
    assert torch.equal(caches[0][0].view(torch.uint8), caches[1][0].view(torch.uint8))
    assert torch.equal(caches[0][1].view(torch.uint8), caches[1][1].view(torch.uint8))


def test_sequences_outside_every_group_are_left_alone():
    """A group list naming only some sequences (all of one partition, so the merge has nothing
    to do for the others): the listed sequences' rows and the caches they hold are written, the
    other sequences' outputs are not, and the padded places of a short group (-1, or a sequence
    index past the batch) are skipped."""
    P = pk()
    rng = np.random.default_rng(95)
    dtype, hq, hkv, bs, d, part = "bf16", 8, 8, 16, 128, 256
    nb, kd, vd, seqs, slots, pairs, cow_src, tables, lens, W = _forked_batch(
        P, rng, dtype, hkv, d, bs, [37, 20], [3, 2])
    B = len(seqs)
    groups, glens = P.plan_fork_groups(tables, lens, cow_src, bs, nb, 4)
    assert groups.tolist() == [[0, 1, 2, -1], [3, 4, -1, -1]]
    g = groups[:1].copy()
    g[0, 3] = B + 7                       # outside the batch: skipped like -1
    q = to_dev(gen.normal(rng, (B, hq, d), dtype), dtype)
    k_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    v_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    o = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    k2, v2 = kd.clone(), vd.clone()
    P.paged_attention_decode_step_groups(o, q, k_new, v_new, i32(cow_src), k2, v2, i32(tables),
                                         i32(lens), 0.125, i32(g),
                                         i32(P.decode_work_list(glens[:1], W, bs, part)),
                                         partition_size=part)
    torch.cuda.synchronize()
    assert not torch.isnan(o[:3]).any() and torch.isnan(o[3:]).all()
    # sequences 3 and 4 wrote nothing: their new-token slots still hold the NaN fill, bit for
    # bit; the members' slots hold their new K rows
    before, after, new = to_host(kd, dtype), to_host(k2, dtype), to_host(k_new, dtype)
    for b in (3, 4):
        s = int(slots[b])
        assert np.array_equal(after[s // bs, :, s % bs], before[s // bs, :, s % bs])
    for b in (0, 1, 2):
        s = int(slots[b])
        assert np.array_equal(after[s // bs, :, s % bs], new[b])


def test_group_step_long_tail_parallel_sampling():
    """The long-tail serving step at full size (32 prompts x 4 branches, 40 MHA heads, fp16,
    block 32) over the packed list of its groups, the launch the bench times: caches bitwise
    those of the per-sequence step, outputs within fp32 rounding of it, sampled rows against
    the oracle."""
    P = pk()
    c = gen.llama13b_longtail_case(values=False)
    nb, bs, H, d, B = c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim, c.num_seqs
    bm = P.BlockManager(nb, bs, c.free_order)
    for g, L in enumerate(c.decode_lens.tolist()):
        bm.add_seq(g * c.branches, L - 1)
        for br in range(1, c.branches):
            bm.fork(g * c.branches, g * c.branches + br)
    slots, pairs, cow_src = bm.append_step(range(B))
    tables, lens = bm.build_tables(range(B), c.table_width)
    groups, glens = P.plan_fork_groups(tables, lens, cow_src, bs, nb, c.branches)
    assert groups.shape == (len(c.decode_lens), c.branches) and (groups >= 0).all()
    shape = (nb, H, bs, d)
    kd, vd = gen.device_normal(shape, "f16", 81, "cuda"), gen.device_normal(shape, "f16", 82, "cuda")
    q = gen.device_normal((B, H, d), "f16", 83, "cuda")
    k_new, v_new = gen.device_normal((B, H, d), "f16", 84, "cuda"), gen.device_normal((B, H, d), "f16", 85, "cuda")
    k1, v1 = kd.clone(), vd.clone()
    o1 = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    P.paged_attention_decode_step(o1, q, k_new, v_new, i32(cow_src), k1, v1, i32(tables),
                                  i32(lens), c.scale, partition_size=2048,
                                  work_list=i32(P.decode_work_list(lens, c.table_width, bs, 2048)))
    lst, rows = P.decode_work_list_packed(glens, c.table_width, bs, 2048, 256)
    for policy in (P.KV_STREAM, P.KV_CACHED):
        k2, v2 = kd.clone(), vd.clone()
        o2 = torch.empty_like(o1)
        P.paged_attention_decode_step_groups(o2, q, k_new, v_new, i32(cow_src), k2, v2,
                                             i32(tables), i32(lens), c.scale, i32(groups),
                                             (i32(lst), rows), partition_size=2048,
                                             kv_policy=policy)
        torch.cuda.synchronize()
        assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
        assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
        assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)
    # sampled sequences against the oracle (the caches after the step)
    kh, vh = to_host(k2, "f16"), to_host(v2, "f16")
    qh = to_host(q, "f16")
    pick = [0, 1, 2, 3, int(np.argmax(lens)), B - 1]
    sub = gen.PagedDecodeCase("groups_sample", "f16", H, H, d, bs, nb, lens[pick], tables[pick],
                              c.scale, q=qh[pick], k_cache=kh, v_cache=vh)
    assert max_err(o2[pick].cpu().numpy().astype(np.float64), oracle(sub)) <= GATE["f16"]


def test_group_step_long_prompt_forks_full_size():
    """The long-prompt fork workload at full size (32 prompts x 4 branches of mean 1432 tokens,
    40 MHA heads, fp16, block 32) in the launch the bench times (the groups' plain list with
    its ticketed tail made private, 1024-token partitions, late units by ticket, the merge):
    caches bitwise those of the per-sequence step, outputs within fp32 rounding of it, sampled
    sequences against the oracle."""
    P = pk()
    c = gen.llama13b_fork_long_case(values=False)
    nb, bs, H, d, B = c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim, c.num_seqs
    bm = P.BlockManager(nb, bs, c.free_order)
    for g, L in enumerate(c.decode_lens.tolist()):
        bm.add_seq(g * c.branches, L - 1)
        for br in range(1, c.branches):
            bm.fork(g * c.branches, g * c.branches + br)
    slots, pairs, cow_src = bm.append_step(range(B))
    tables, lens = bm.build_tables(range(B), c.table_width)
    groups, glens = P.plan_fork_groups(tables, lens, cow_src, bs, nb, c.branches)
    assert groups.shape == (len(c.decode_lens), c.branches)
    shape = (nb, H, bs, d)
    kd, vd = gen.device_normal(shape, "f16", 91, "cuda"), gen.device_normal(shape, "f16", 92, "cuda")
    q = gen.device_normal((B, H, d), "f16", 93, "cuda")
    k_new, v_new = gen.device_normal((B, H, d), "f16", 94, "cuda"), gen.device_normal((B, H, d), "f16", 95, "cuda")
    part = 1024
    k1, v1 = kd.clone(), vd.clone()
    o1 = torch.empty((B, H, d), dtype=torch.float16, device="cuda")
    P.paged_attention_decode_step(o1, q, k_new, v_new, i32(cow_src), k1, v1, i32(tables),
                                  i32(lens), c.scale, partition_size=part,
                                  work_list=i32(P.decode_work_list(lens, c.table_width, bs, part)))
    k2, v2 = kd.clone(), vd.clone()
    o2 = torch.empty_like(o1)
    ws = torch.empty(P.decode_workspace_bytes(B, H, c.table_width, bs, d, part), dtype=torch.uint8,
                     device="cuda")
    P.decode_workspace_init(ws)          # the bench's ticketed late units
    lst = P.decode_work_list(glens, c.table_width, bs, part)
    tail = P.decode_ticketed_items(torch.float16, d, H, H, bs, part, lst.shape[0], "fork_groups",
                                   c.branches)
    lst, _ = P.decode_work_list_private_tail(lst, tables[groups[:, 0]], glens, bs, nb, part, tail)
    P.paged_attention_decode_step_groups(o2, q, k_new, v_new, i32(cow_src), k2, v2, i32(tables),
                                         i32(lens), c.scale, i32(groups), i32(lst),
                                         partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
    # fp16 outputs: the two orders of summation may round to neighbouring halves
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-3
    kh, vh, qh = to_host(k2, "f16"), to_host(v2, "f16"), to_host(q, "f16")
    pick = [0, 1, int(np.argmax(lens)), int(np.argmin(lens)), B - 1]
    sub = gen.PagedDecodeCase("fork_long_sample", "f16", H, H, d, bs, nb, lens[pick], tables[pick],
                              c.scale, q=qh[pick], k_cache=kh, v_cache=vh)
    assert max_err(o2[pick].float().cpu().numpy().astype(np.float64), oracle(sub)) <= GATE["f16"]
