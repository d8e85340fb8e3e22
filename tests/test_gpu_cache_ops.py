"""GPU bit-exactness of the cache write and block copy, and whole decode steps driven by the
C++ block manager against the oracle's independent path (MI355X only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理"

The product side runs: C++ manager -> copy_blocks -> reshape_and_cache -> decode (HIP).
The oracle side runs: Python manager model -> reference copy -> reference cache write ->
fp64 attention. They share only the generated inputs.
"""
import hashlib

import numpy as np
import pytest
import torch

from oracle import cache_ops as ref_ops
from oracle.block_manager_model import BlockManagerModel
from workloads import gen
from tests.gpu_util import GATE, i32, max_err, oracle, run_decode, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_402_amd  # noqa: F401


def pk():
    import paged_kv_cache_402_amd
    return paged_kv_cache_402_amd


def _bits_equal(dev, host, dtype):
    return np.array_equal(to_host(dev, dtype).view(np.uint8), np.ascontiguousarray(host).view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_reshape_and_cache_bit_exact(dtype, d):
    rng = np.random.default_rng(3 + d)
    nb, H, bs = 64, 4, 16
    kc = gen.normal(rng, (nb, H, bs, d), dtype)
    vc = gen.normal(rng, (nb, H, bs, d), dtype)
    T = 200
    slots = rng.choice(nb * bs, T, replace=False).astype(np.int32)
    slots[::17] = -1
    kn = gen.normal(rng, (T, H, d), dtype)
    vn = gen.normal(rng, (T, H, d), dtype)
    kd, vd = to_dev(kc, dtype), to_dev(vc, dtype)
    pk().reshape_and_cache(to_dev(kn, dtype), to_dev(vn, dtype), kd, vd, i32(slots))
    torch.cuda.synchronize()
    kr, vr = ref_ops.reshape_and_cache(kn, vn, kc, vc, slots)
    assert _bits_equal(kd, kr, dtype) and _bits_equal(vd, vr, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_copy_blocks_bit_exact(dtype):
    rng = np.random.default_rng(4)
    nb, H, bs, d = 80, 8, 32, 128
    kc = gen.normal(rng, (nb, H, bs, d), dtype)
    vc = gen.normal(rng, (nb, H, bs, d), dtype)
    kc[5, :, 3:] = gen.nan_value(dtype)   # NaN payloads are copied as bits too
    ids = rng.permutation(nb)
    pairs = np.stack([ids[:20], ids[20:40]], axis=1).astype(np.int32)
    pairs[0, 0] = 5
    kd, vd = to_dev(kc, dtype), to_dev(vc, dtype)
    pk().copy_blocks(kd, vd, i32(pairs))
    torch.cuda.synchronize()
    kr, vr = ref_ops.copy_blocks(kc, vc, pairs)
    assert _bits_equal(kd, kr, dtype) and _bits_equal(vd, vr, dtype)


def test_copy_blocks_skips_pairs_outside_the_pool():
    rng = np.random.default_rng(5)
    kc = gen.normal(rng, (8, 2, 16, 64), "f32")
    kd, vd = to_dev(kc, "f32"), to_dev(kc.copy(), "f32")
    pk().copy_blocks(kd, vd, i32([[1, 2], [9, 3], [4, -1]]))
    torch.cuda.synchronize()
    kr, _ = ref_ops.copy_blocks(kc, kc, [[1, 2]])
    assert _bits_equal(kd, kr, "f32")


def _fused_copy_expected(apart, before, pairs, slots, bs):
    """The caches a one-pass decode step leaves: those of copy_blocks then reshape_and_cache
    (`apart`), except that in each copied block the rows past the new token's keep what the
    block held before the step (`before`): the fused copy writes the rows the sequence holds,
    the block's earlier rows, and no row past its new token."""
    want = apart.clone() if hasattr(apart, "clone") else apart.copy()
    new_row = {int(x) // bs: int(x) % bs for x in np.asarray(slots).reshape(-1)}
    for _, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        r = new_row[dst]
        want[dst, :, r + 1:] = before[dst, :, r + 1:]
    return want


def _hash_blocks(pool_dev, dtype):
    h = to_host(pool_dev, dtype)
    return [hashlib.sha256(np.ascontiguousarray(h[b]).tobytes()).hexdigest() for b in range(h.shape[0])]


def test_tiny_decode_step_with_cow():
    """Four sequences (1, 15, 16, 35 tokens; the last one on blocks 7, 3, 9 as in P3 §2.2.3):
    decode, write one token each (the 16-token sequence opens a new block), decode again, then
    fork the 36-token sequence and append to the child: its shared last block is copied first
    (P1 §6.2), the source block is unchanged and the sibling's output does not change."""
    P = pk()
    case = gen.tiny_case(pin_worked_example=True)
    bm = P.BlockManager(32, 16, case.free_order)
    model = BlockManagerModel(32, 16, case.free_order)
    for s, L in enumerate(case.seq_lens.tolist()):
        bm.add_seq(s, L)
        model.add_seq(s, L)
    tables, lens = bm.build_tables(range(4), 4)
    assert np.array_equal(tables, case.block_tables) and np.array_equal(lens, case.seq_lens)
    assert bm.table(3)[0] == [7, 3, 9]
    kd, vd = to_dev(case.k_cache, "f32"), to_dev(case.v_cache, "f32")
    got, _ = run_decode(case, k=kd, v=vd)
    assert max_err(got, oracle(case)) <= GATE["f32"]

    # one new token per sequence
    slots, pairs = bm.append_slots([0, 1, 2, 3])
    mres = [model.append_slot(s) for s in range(4)]
    assert slots.tolist() == [r[1] for r in mres] and pairs.shape[0] == 0
    assert slots[3] == 147                       # token 35 of the worked example
    assert len(bm.table(2)[0]) == 2              # 16 tokens -> the 17th opens a block
    k_new, v_new = case.meta["k_new"], case.meta["v_new"]
    P.reshape_and_cache(to_dev(k_new, "f32"), to_dev(v_new, "f32"), kd, vd, i32(slots))
    kc1, vc1 = ref_ops.reshape_and_cache(k_new, v_new, case.k_cache, case.v_cache,
                                         [r[1] for r in mres])
    torch.cuda.synchronize()
    assert _bits_equal(kd, kc1, "f32") and _bits_equal(vd, vc1, "f32")
    tables, lens = bm.build_tables(range(4), 4)
    step2 = gen.PagedDecodeCase("tiny2", "f32", 4, 4, 64, 16, 32, lens, tables, case.scale,
                                q=case.meta["q_next"], k_cache=kc1, v_cache=vc1)
    got2, out2 = run_decode(step2, k=kd, v=vd)
    ref2 = oracle(step2)
    assert max_err(got2, ref2) <= GATE["f32"]

    # fork the 36-token sequence, append to the child: copy-on-write of block 9
    bm.fork(3, 4)
    model.fork(3, 4)
    before = _hash_blocks(kd, "f32")
    slots_c, pairs_c = bm.append_slots([4])
    st, slot_m, cs, cd = model.append_slot(4)
    assert st == 1 and pairs_c.tolist() == [[cs, cd]] and cs == 9 and slots_c[0] == slot_m
    assert bm.stats()["cow_copies"] == 1
    P.copy_blocks(kd, vd, i32(pairs_c))
    kn2 = gen.normal(np.random.default_rng(99), (1, 4, 64), "f32")
    vn2 = gen.normal(np.random.default_rng(98), (1, 4, 64), "f32")
    P.reshape_and_cache(to_dev(kn2, "f32"), to_dev(vn2, "f32"), kd, vd, i32(slots_c))
    torch.cuda.synchronize()
    after = _hash_blocks(kd, "f32")
    changed = [b for b in range(32) if before[b] != after[b]]
    assert changed == [cd]                        # only the private copy changed
    kc2, vc2 = ref_ops.copy_blocks(kc1, vc1, [[cs, cd]])
    kc2, vc2 = ref_ops.reshape_and_cache(kn2, vn2, kc2, vc2, [slot_m])
    assert _bits_equal(kd, kc2, "f32") and _bits_equal(vd, vc2, "f32")
    kh = to_host(kd, "f32")
    assert np.array_equal(kh[cd, :, :4], kh[cs, :, :4])  # the copy holds the shared tokens

    tables, lens = bm.build_tables(range(5), 4)
    q5 = np.concatenate([case.meta["q_next"], case.meta["q_next"][3:4]])
    step3 = gen.PagedDecodeCase("tiny3", "f32", 4, 4, 64, 16, 32, lens, tables, case.scale,
                                q=q5, k_cache=kc2, v_cache=vc2)
    got3, out3 = run_decode(step3, k=kd, v=vd)
    assert max_err(got3, oracle(step3)) <= GATE["f32"]
    assert torch.equal(out3[:4].cpu(), out2.cpu())   # siblings untouched, bit for bit


def test_longtail_parallel_sampling_step():
    """32 prompts x 4 branches, fp16, block 32, geometric lengths (mean 200): each branch
    shares its prompt's blocks, appends one token (copy-on-write of the shared partial block
    for 3 of the 4 branches, in place for the last), then decode over all 128 sequences."""
    P = pk()
    c = gen.llama13b_longtail_case()
    nb, bs, H, d = c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim
    bm = P.BlockManager(nb, bs, c.free_order)
    model = BlockManagerModel(nb, bs, c.free_order)
    host_k = np.full((nb, H, bs, d), gen.nan_value("f16"), dtype=np.float16)
    host_v = host_k.copy()
    kd, vd = to_dev(host_k, "f16"), to_dev(host_v, "f16")
    B = c.num_seqs
    for g, L in enumerate(c.decode_lens.tolist()):
        parent = g * c.branches
        bm.add_seq(parent, L - 1)
        model.add_seq(parent, L - 1)
        if L - 1 > 0:
            s_dev = bm.slots(parent, 0, L - 1)
            s_ref = model.slots(parent, 0, L - 1)
            assert s_dev.tolist() == s_ref
            P.reshape_and_cache(to_dev(c.prompt_k[g], "f16"), to_dev(c.prompt_v[g], "f16"), kd, vd,
                                i32(s_dev))
            host_k, host_v = ref_ops.reshape_and_cache(c.prompt_k[g], c.prompt_v[g], host_k,
                                                       host_v, s_ref)
        for br in range(1, c.branches):
            bm.fork(parent, parent + br)
            model.fork(parent, parent + br)
    slots, pairs = bm.append_slots(range(B))
    res = [model.append_slot(s) for s in range(B)]
    assert slots.tolist() == [r[1] for r in res]
    ref_pairs = [[r[2], r[3]] for r in res if r[0] == 1]
    assert pairs.tolist() == ref_pairs
    partial = sum(1 for L in c.decode_lens if (L - 1) % bs != 0)
    assert len(ref_pairs) == 3 * partial
    P.copy_blocks(kd, vd, i32(pairs.reshape(-1, 2)))
    P.reshape_and_cache(to_dev(c.new_k, "f16"), to_dev(c.new_v, "f16"), kd, vd, i32(slots))
    host_k, host_v = ref_ops.copy_blocks(host_k, host_v, ref_pairs)
    host_k, host_v = ref_ops.reshape_and_cache(c.new_k, c.new_v, host_k, host_v,
                                               [r[1] for r in res])
    torch.cuda.synchronize()
    assert _bits_equal(kd, host_k, "f16") and _bits_equal(vd, host_v, "f16")
    tables, lens = bm.build_tables(range(B), c.table_width)
    assert lens.tolist() == np.repeat(c.decode_lens, c.branches).tolist()
    step = gen.PagedDecodeCase("longtail", "f16", H, H, d, bs, nb, lens, tables, c.scale, q=c.q,
                               k_cache=host_k, v_cache=host_v)
    got, _ = run_decode(step, k=kd, v=vd)
    assert max_err(got, oracle(step)) <= GATE["f16"]
    got16, _ = run_decode(step, k=kd, v=vd, out_dtype="f16")
    ref = oracle(step)
    from tests.gpu_util import out_gate
    assert (np.abs(got16 - ref) <= out_gate(ref, "f16", "f16")).all()


def test_prefix_cached_requests_decode_over_shared_blocks():
    """P1 §7.4 / P3 §2.2.8: a second request with the same system prompt reuses the cached
    blocks and writes K/V only for its own tokens; both decode to the attention over their own
    logically contiguous K/V."""
    from oracle import paged_attention as ref_pa
    P = pk()
    rng = np.random.default_rng(77)
    bs, H, d, NB = 16, 4, 128, 40
    bm = P.BlockManager(NB, bs)
    system = rng.integers(0, 50000, 48).tolist()                 # 3 full blocks
    users = [rng.integers(0, 50000, n).tolist() for n in (10, 23)]
    sys_k = gen.normal(rng, (48, H, d), "bf16")
    sys_v = gen.normal(rng, (48, H, d), "bf16")
    user_kv = [(gen.normal(rng, (len(u), H, d), "bf16"), gen.normal(rng, (len(u), H, d), "bf16"))
               for u in users]
    kd = to_dev(np.full((NB, H, bs, d), gen.nan_value("bf16"), np.uint16), "bf16")
    vd = to_dev(np.full((NB, H, bs, d), gen.nan_value("bf16"), np.uint16), "bf16")
    cached = []
    for s, u in enumerate(users):
        toks = system + u
        c = bm.add_seq_cached(s, toks)
        cached.append(c)
        k_all = np.concatenate([sys_k, user_kv[s][0]])
        v_all = np.concatenate([sys_v, user_kv[s][1]])
        slots = bm.slots(s, c, len(toks) - c)
        P.reshape_and_cache(to_dev(k_all[c:], "bf16"), to_dev(v_all[c:], "bf16"), kd, vd, i32(slots))
    assert cached == [0, 48]
    assert bm.stats()["prefix_hits"] == 3
    tables, lens = bm.build_tables([0, 1], 8)
    assert tables[0, :3].tolist() == tables[1, :3].tolist()
    q = gen.normal(rng, (2, H, d), "bf16")
    out = torch.empty((2, H, d), dtype=torch.float32, device="cuda")
    P.paged_attention_decode(out, to_dev(q, "bf16"), kd, vd, i32(tables), i32(lens), 0.088)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for s in range(2):
        k_all = np.concatenate([sys_k, user_kv[s][0]])
        v_all = np.concatenate([sys_v, user_kv[s][1]])
        ref = ref_pa.contiguous_attention(q[s], k_all, v_all, 0.088, "bf16")
        assert max_err(got[s], ref) <= GATE["bf16"]


@pytest.mark.parametrize("width,part,fused", [(4, 512, False), (3, 32, False), (4, 512, True),
                                              (3, 32, True)])
def test_beam_search_loop_decodes_every_step(width, part, fused):
    """P2 §2.2 / P1 §6.2: beam search over 40 steps on a tight pool (finished beams' blocks are
    handed out again): every step frees the dropped beams, forks the kept ones, appends one
    token per beam (copy-on-write of shared partial blocks), writes the new K/V and decodes all
    beams, as three launches or (fused) as one decode step. Device caches stay bit-identical
    to the oracle's, and every decode matches it."""
    from workloads import traces
    P = pk()
    rng = np.random.default_rng(402700 + width)
    bs, Hq, H, d, NB, W, dt = 16, 8, 2, 128, 40, 8, "bf16"
    trace = traces.beam_search_trace(rng, 37, width, 40)
    order = rng.permutation(NB).astype(np.int32)
    bm, model = P.BlockManager(NB, bs, order), BlockManagerModel(NB, bs, order)
    host_k = np.full((NB, H, bs, d), gen.nan_value(dt), dtype=np.uint16)
    host_v = host_k.copy()
    kd, vd = to_dev(host_k, dt), to_dev(host_v, dt)
    bm.add_seq(trace.root, trace.prompt_len)
    model.add_seq(trace.root, trace.prompt_len)
    pk_, pv_ = gen.normal(rng, (37, H, d), dt), gen.normal(rng, (37, H, d), dt)
    slots = bm.slots(trace.root, 0, 37)
    assert slots.tolist() == model.slots(trace.root, 0, 37)
    P.reshape_and_cache(to_dev(pk_, dt), to_dev(pv_, dt), kd, vd, i32(slots))
    host_k, host_v = ref_ops.reshape_and_cache(pk_, pv_, host_k, host_v, slots.tolist())
    worst = 0.0
    for step in trace.steps[:-1]:
        for s in step.frees:
            bm.free_seq(s)
            model.free_seq(s)
        for p_, c_ in step.forks:
            bm.fork(p_, c_)
            model.fork(p_, c_)
        seqs = step.appends
        sl, pairs, cow_src = bm.append_step(seqs)
        res = [model.append_slot(s) for s in seqs]
        assert sl.tolist() == [r[1] for r in res]
        ref_pairs = [[r[2], r[3]] for r in res if r[0] == 1]
        assert pairs.reshape(-1, 2).tolist() == ref_pairs
        if ref_pairs:
            if not fused:
                P.copy_blocks(kd, vd, i32(pairs.reshape(-1, 2)))
            host_k, host_v = ref_ops.copy_blocks(host_k, host_v, ref_pairs)
        nk, nv = gen.normal(rng, (len(seqs), H, d), dt), gen.normal(rng, (len(seqs), H, d), dt)
        if not fused:
            P.reshape_and_cache(to_dev(nk, dt), to_dev(nv, dt), kd, vd, i32(sl))
        host_k, host_v = ref_ops.reshape_and_cache(nk, nv, host_k, host_v, sl.tolist())
        tables, lens = bm.build_tables(seqs, W)
        for i, s in enumerate(seqs):
            blocks, n = model.table(s)
            assert lens[i] == n and tables[i, :len(blocks)].tolist() == blocks
        q = gen.normal(rng, (len(seqs), Hq, d), dt)
        case = gen.PagedDecodeCase("beam", dt, Hq, H, d, bs, NB, lens, tables, 0.0884, q=q,
                                   k_cache=host_k, v_cache=host_v)
        if fused:
            out = torch.full((len(seqs), Hq, d), float("nan"), dtype=torch.float32,
                             device="cuda")
            kb, vb = to_host(kd, dt), to_host(vd, dt)
            P.paged_attention_decode_step(out, to_dev(q, dt), to_dev(nk, dt), to_dev(nv, dt),
                                          i32(cow_src), kd, vd, i32(tables), i32(lens), 0.0884,
                                          partition_size=part)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            # rows of a copied block past the new token are not copied by the fused step
            host_k = _fused_copy_expected(host_k, kb, ref_pairs, sl, bs)
            host_v = _fused_copy_expected(host_v, vb, ref_pairs, sl, bs)
        else:
            got, _ = run_decode(case, k=kd, v=vd, partition_size=part)
        worst = max(worst, max_err(got, oracle(case)))
        torch.cuda.synchronize()
        assert _bits_equal(kd, host_k, dt) and _bits_equal(vd, host_v, dt)
    assert worst <= GATE[dt]
    assert model.stats()["cow_copies"] > 0


def test_continuous_batching_loop_decodes_every_step():
    """P1 §8.2 / P3 §2.2.12: requests arrive, are admitted, write their prompt, decode one token
    per step, finish or get preempted (a tight pool) and are recomputed; every step the C++
    scheduler agrees with the reference model, the device caches stay bit-identical to the
    oracle's, and every decode matches the oracle's attention."""
    from oracle.scheduler_model import SchedulerModel
    from workloads import traces
    P = pk()
    rng = np.random.default_rng(402800)
    bs, Hq, H, d, NB, W, dt = 16, 8, 2, 128, 16, 12, "bf16"
    reqs = traces.request_stream(rng, 24, 1.5, (1, 80), 10, 40)
    # K/V of every (request, position): a recomputed token gets the same values again
    kv = {r.req_id: (gen.normal(rng, (r.prompt_len + r.output_len, H, d), dt),
                     gen.normal(rng, (r.prompt_len + r.output_len, H, d), dt)) for r in reqs}
    order = rng.permutation(NB).astype(np.int32)
    bm, model_bm = P.BlockManager(NB, bs, order), BlockManagerModel(NB, bs, order)
    sched, model = P.Scheduler(bm, 6, 256, 1), SchedulerModel(model_bm, 6, 256, 1)
    host_k = np.full((NB, H, bs, d), gen.nan_value(dt), dtype=np.uint16)
    host_v = host_k.copy()
    kd, vd = to_dev(host_k, dt), to_dev(host_v, dt)
    pending = sorted(reqs, key=lambda r: r.arrival)
    worst, steps, preempted = 0.0, 0, 0
    while (pending or sched.stats()["waiting"] or sched.stats()["running"]) and steps < 400:
        while pending and pending[0].arrival <= steps:
            r = pending.pop(0)
            sched.add_request(r.req_id, r.prompt_len, r.output_len)
            model.add_request(r.req_id, r.prompt_len, r.output_len)
        st, ref = sched.step(), model.step()
        assert st.batch.tolist() == ref["batch"] and st.slots.tolist() == ref["slots"]
        preempted += len(st.preempted)
        if st.cow_pairs.shape[0]:
            P.copy_blocks(kd, vd, i32(st.cow_pairs))
            host_k, host_v = ref_ops.copy_blocks(host_k, host_v, st.cow_pairs.tolist())
        if st.slots.shape[0]:
            nk = np.stack([kv[s][0][p] for s, p in zip(st.slot_seq.tolist(), st.slot_pos.tolist())])
            nv = np.stack([kv[s][1][p] for s, p in zip(st.slot_seq.tolist(), st.slot_pos.tolist())])
            P.reshape_and_cache(to_dev(nk, dt), to_dev(nv, dt), kd, vd, i32(st.slots))
            host_k, host_v = ref_ops.reshape_and_cache(nk, nv, host_k, host_v, st.slots.tolist())
        if st.batch.shape[0]:
            tables, lens = bm.build_tables(st.batch, W)
            q = gen.normal(rng, (st.batch.shape[0], Hq, d), dt)
            case = gen.PagedDecodeCase("serve", dt, Hq, H, d, bs, NB, lens, tables, 0.0884, q=q,
                                       k_cache=host_k, v_cache=host_v)
            got, _ = run_decode(case, k=kd, v=vd, partition_size=64)
            worst = max(worst, max_err(got, oracle(case)))
        steps += 1
    torch.cuda.synchronize()
    assert _bits_equal(kd, host_k, dt) and _bits_equal(vd, host_v, dt)
    assert worst <= GATE[dt]
    assert sched.stats()["finished"] == len(reqs) and preempted > 0


# ------------------------------------------------------------------------------------------
# one decode step in one pass: copy-on-write, cache write and attention fused
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,hq,hkv,bs,part,form", [
    ("bf16", 32, 8, 16, 512, "list"),
    ("f16", 40, 40, 32, 2048, "packed"),
    ("bf16", 64, 8, 64, 1024, "full"),         # G 8: matrix-core scores
    ("f32", 8, 4, 8, 64, "list"),
])
def test_decode_step_is_copy_then_cache_write_then_decode(dtype, hq, hkv, bs, part, form):
    """Prompts forked into 1-4 branches, then one token each: branches of a partial last
    block copy it (all but the last writer), full ones open a fresh block. The fused step
    (decode_step with the manager's per-sequence copy sources) must leave bitwise the caches
    and the output of copy_blocks, reshape_and_cache and the decode run apart. Unwritten slots
    hold NaN, so a read of a copy before it is made would show."""
    P = pk()
    rng = np.random.default_rng(80)
    d = 128 if dtype != "f32" else 64
    prompts = [3 * bs - 3, 2 * bs, part + 5, 1, 0, bs + 1, 2 * part - 1, 7]
    branches = [4, 3, 2, 1, 2, 4, 3, 1]
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
    B = len(seqs)
    slots, pairs, cow_src = bm.append_step(seqs)
    assert pairs.shape[0] == sum(br - 1 for L, br in zip(prompts, branches) if L % bs)
    W = max(-(-(L + 1) // bs) for L in prompts) + 1
    tables, lens = bm.build_tables(seqs, W)
    q = to_dev(gen.normal(rng, (B, hq, d), dtype), dtype)
    k_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    v_new = to_dev(gen.normal(rng, (B, hkv, d), dtype), dtype)
    scale = float(np.float32(1 / np.sqrt(d)))
    if form == "full":
        work = None
    elif form == "list":
        work = i32(P.decode_work_list(lens, W, bs, part))
    else:
        lst, rows = P.decode_work_list_packed(lens, W, bs, part, part // 4)
        assert rows < len(lst)
        work = (i32(lst), rows)
    # apart
    k1, v1 = kd.clone(), vd.clone()
    if pairs.shape[0]:
        P.copy_blocks(k1, v1, i32(pairs.reshape(-1, 2)))
    P.reshape_and_cache(k_new, v_new, k1, v1, i32(slots))
    o1 = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    P.paged_attention_decode(o1, q, k1, v1, i32(tables), i32(lens), scale, partition_size=part,
                             work_list=work)
    # fused
    k2, v2 = kd.clone(), vd.clone()
    o2 = torch.full_like(o1, float("nan"))
    P.paged_attention_decode_step(o2, q, k_new, v_new, i32(cow_src), k2, v2, i32(tables),
                                  i32(lens), scale, partition_size=part, work_list=work)
    torch.cuda.synchronize()
    want_k = _fused_copy_expected(k1, kd, pairs, slots, bs)
    want_v = _fused_copy_expected(v1, vd, pairs, slots, bs)
    assert torch.equal(want_k.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(want_v.view(torch.uint8), v2.view(torch.uint8))
    assert torch.equal(o1, o2)
    ref = gen.PagedDecodeCase("step", dtype, hq, hkv, d, bs, nb, lens, tables, scale,
                              q=to_host(q, dtype), k_cache=to_host(k2, dtype),
                              v_cache=to_host(v2, dtype))
    assert max_err(o2.cpu().numpy().astype(np.float64), oracle(ref)) <= GATE[dtype]


def test_decode_step_long_tail_parallel_sampling():
    """The long-tail serving step at full size (32 prompts x 4 branches, 40 MHA heads, fp16,
    block 32): the fused step over the work list against the separate copy, cache write and
    decode, bitwise."""
    P = pk()
    c = gen.llama13b_longtail_case(values=False)
    nb, bs, H, d, B = c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim, c.num_seqs
    bm = P.BlockManager(nb, bs, c.free_order)
    for g, L in enumerate(c.decode_lens.tolist()):
        bm.add_seq(g * c.branches, L - 1)
        for br in range(1, c.branches):
            bm.fork(g * c.branches, g * c.branches + br)
    slots, pairs, cow_src = bm.append_step(range(B))
    assert (cow_src >= 0).sum() == pairs.shape[0] > 0
    tables, lens = bm.build_tables(range(B), c.table_width)
    shape = (nb, H, bs, d)
    kd, vd = gen.device_normal(shape, "f16", 81, "cuda"), gen.device_normal(shape, "f16", 82, "cuda")
    q = gen.device_normal((B, H, d), "f16", 83, "cuda")
    k_new, v_new = gen.device_normal((B, H, d), "f16", 84, "cuda"), gen.device_normal((B, H, d), "f16", 85, "cuda")
    work = i32(P.decode_work_list(lens, c.table_width, bs, 2048))
    k1, v1 = kd.clone(), vd.clone()
    P.copy_blocks(k1, v1, i32(pairs.reshape(-1, 2)))
    P.reshape_and_cache(k_new, v_new, k1, v1, i32(slots))
    o1 = torch.empty((B, H, d), dtype=torch.float16, device="cuda")
    P.paged_attention_decode(o1, q, k1, v1, i32(tables), i32(lens), c.scale, partition_size=2048,
                             work_list=work)
    k2, v2 = kd.clone(), vd.clone()
    o2 = torch.empty_like(o1)
    P.paged_attention_decode_step(o2, q, k_new, v_new, i32(cow_src), k2, v2, i32(tables),
                                  i32(lens), c.scale, partition_size=2048, work_list=work)
    torch.cuda.synchronize()
    want_k = _fused_copy_expected(k1, kd, pairs, slots, bs)
    want_v = _fused_copy_expected(v1, vd, pairs, slots, bs)
    assert torch.equal(want_k.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(want_v.view(torch.uint8), v2.view(torch.uint8))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # the four branches read the same prompt blocks: the policy helper picks the default cache
    # policy for this batch, and the step under it leaves the same bits
    assert P.decode_kv_policy(tables, lens, bs, nb) == P.KV_CACHED
    k3, v3 = kd.clone(), vd.clone()
    o3 = torch.empty_like(o1)
    P.paged_attention_decode_step(o3, q, k_new, v_new, i32(cow_src), k3, v3, i32(tables),
                                  i32(lens), c.scale, partition_size=2048, work_list=work,
                                  kv_policy=P.KV_CACHED)
    torch.cuda.synchronize()
    assert torch.equal(k2.view(torch.uint8), k3.view(torch.uint8))
    assert torch.equal(v2.view(torch.uint8), v3.view(torch.uint8))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


# ------------------------------------------------------------------------------------------
# pool sizing on the device (P3 §2.2.5: the memory fraction fixes the KV pool at start-up;
# §2.2.7: the pool left after the weights, divided by what one request's KV takes)
# ------------------------------------------------------------------------------------------

def test_pool_plan_sizes_a_real_pool_and_decodes_over_it():
    """The plan is taken from the device's free memory (torch.cuda.mem_get_info), with all but
    768 MiB of it standing for the weights, so the pool stays small. It must equal the
    exact-rational oracle, its cache-tensor size must be what the allocated caches take, the
    manager must admit exactly its number of requests before ENOBLOCKS, and decoding over the
    whole pool must match the fp64 oracle."""
    from fractions import Fraction

    from oracle import pool_plan as ref_plan
    free, _total = torch.cuda.mem_get_info()
    weights, reserve = free - (768 << 20), 64 << 20
    Hq, Hkv, D, bs, ctx = 32, 8, 128, 16, 1024
    kw = dict(num_layers=1, num_kv_heads=Hkv, head_dim=D, elem_bytes=2, block_size=bs,
              context_tokens=ctx)
    plan = pk().kv_pool_plan(free, weights, utilization=0.9, reserve_bytes=reserve, **kw)
    want = ref_plan.plan(free, weights, Fraction(900000, 10 ** 6), "remainder", reserve,
                         1, Hkv, D, 2, bs, ctx, ctx)
    for key in ("pool_bytes", "bytes_per_token", "bytes_per_block", "num_blocks",
                "blocks_per_request", "max_requests", "cache_tensor_bytes",
                "max_requests_contiguous"):
        assert plan[key] == want[key], key
    nb, nreq = plan["num_blocks"], plan["max_requests"]
    assert nreq >= 64
    k = gen.device_normal((nb, Hkv, bs, D), "bf16", 7701, "cuda")
    v = gen.device_normal((nb, Hkv, bs, D), "bf16", 7702, "cuda")
    assert k.numel() * k.element_size() == plan["cache_tensor_bytes"]
    assert v.numel() * v.element_size() == plan["cache_tensor_bytes"]
    bm = pk().BlockManager(nb, bs)
    for r in range(nreq):
        bm.add_seq(r, ctx)
    assert bm.add_seq_status(nreq, ctx) == -3           # PKV_ENOBLOCKS: the plan's limit
    assert bm.stats()["free"] == nb - nreq * plan["blocks_per_request"]
    W = plan["blocks_per_request"]
    tables, lens = bm.build_tables(range(nreq), W)
    q = gen.device_normal((nreq, Hq, D), "bf16", 7703, "cuda")
    out = torch.full((nreq, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pk().paged_attention_decode(out, q, k, v, i32(tables), i32(lens), float(np.float32(D ** -0.5)))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    seqs = [0, 1, nreq // 2, nreq - 1]
    ids = np.unique(tables[seqs].reshape(-1))
    remap = {int(b): i for i, b in enumerate(ids)}
    idx = torch.from_numpy(ids.astype(np.int64)).cuda()
    sub = gen.PagedDecodeCase("pool", "bf16", Hq, Hkv, D, bs, len(ids), lens[seqs],
                              np.vectorize(remap.get)(tables[seqs]).astype(np.int32), float(np.float32(D ** -0.5)),
                              q=to_host(q[seqs], "bf16"), k_cache=to_host(k[idx], "bf16"),
                              v_cache=to_host(v[idx], "bf16"))
    ref = oracle(sub)
    assert max_err(got[seqs], ref) <= GATE["bf16"]


def test_library_imported_before_torch_still_reaches_the_device():
    """A process that imports the package before torch: the library must bind to the HIP
    runtime torch uses (torch's wheel carries its own), or its launches find no device. Run in a
    child process, so the import order is the child's own."""
    import os
    import subprocess
    import sys
    code = (
        "import paged_kv_cache_402_amd as pk\n"
        "import torch\n"
        "k = torch.zeros((8, 2, 16, 64), dtype=torch.float32, device='cuda')\n"
        "v = k.clone()\n"
        "kn = torch.ones((4, 2, 64), dtype=torch.float32, device='cuda')\n"
        "pk.reshape_and_cache(kn, kn, k, v, torch.tensor([0, 1, 17, 33], dtype=torch.int32,\n"
        "                                                device='cuda'))\n"
        "torch.cuda.synchronize()\n"
        "print(int(k.sum().item()))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=180,
                       env=env, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == str(4 * 2 * 64)
