"""GPU parity of the HIP decode path against the fp64 oracle (MI355X only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理"

Gates: max |HIP - oracle| <= 1e-5 (fp32 KV) or 2e-3 (fp16/bf16 KV) with fp32 output; with a
16-bit output, max(2e-3, half an ulp of the output format at |oracle| + 1e-5), which is 2e-3
wherever one rounding of the result fits inside it (tests/gpu_util.py: out_gate). Pools hold
NaN in every slot no sequence may read, so any stray read shows.
"""
import math

import numpy as np
import pytest
import torch

from workloads import gen
from tests.gpu_util import (GATE, i32, max_err, oracle, out_gate, run_decode, to_dev, to_host,
                            TORCH_DT)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_402_amd  # noqa: F401  (fails loudly if the library is missing)


def _check(case, partition_size=512, out_dtype=None, seqs=None, ref=None):
    got, _ = run_decode(case, out_dtype=out_dtype, partition_size=partition_size)
    ref = oracle(case, seqs=seqs) if ref is None else ref
    rows = slice(None) if seqs is None else list(seqs)
    err = np.abs(got[rows] - ref[rows])
    gate = out_gate(ref[rows], case.dtype, out_dtype)
    assert np.isfinite(got[rows]).all()
    assert (err <= gate).all(), "max err %g" % float(err.max())
    return got, ref


# --------------------------------------------------------------------------------------------
# the five workloads (reduced batch where the oracle would take long; full sizes sampled)
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("pin", [False, True])
def test_tiny_fp32(pin):
    case = gen.tiny_case(pin_worked_example=pin)
    if pin:
        assert case.block_tables[3, :3].tolist() == [7, 3, 9]
    _check(case)
    _check(case, out_dtype="f32", partition_size=32)


@pytest.mark.parametrize("out_dtype", [None, "bf16"])
def test_llama2_7b_mha_reduced(out_dtype):
    case = gen.llama2_7b_mha_case(num_seqs=6)
    _check(case, out_dtype=out_dtype)


def test_llama3_8b_gqa_prefix_reduced():
    case = gen.llama3_8b_gqa_prefix_case(num_seqs=12)
    got, ref = _check(case)
    _check(case, out_dtype="bf16", ref=ref)


def test_long_context_splitk_reduced():
    case = gen.long_context_splitk_case(num_seqs=3, min_len=5000, max_len=20000)
    _check(case)


# --------------------------------------------------------------------------------------------
# shapes, dtypes, block sizes, group sizes, partition sizes, ragged tails
# --------------------------------------------------------------------------------------------

LENS = [1, 2, 7, 8, 9, 31, 32, 33, 255, 511, 512, 513, 1000, 1024, 1025, 2100]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_shapes_and_groups(dtype, d, group):
    rng = np.random.default_rng(1000 + d + group)
    hkv = 2
    case = gen.make_case("shape", rng, LENS, hkv * group, hkv, d, 16, dtype)
    if d == 256 and group == 8:
        # outside the supported shapes (head_dim 256 takes groups up to 4): refused on the host
        # before any launch, with the reason
        from paged_kv_cache_402_amd._lib import PagedKVError
        with pytest.raises(PagedKVError, match="head_dim 256"):
            run_decode(case)
        return
    _check(case)


@pytest.mark.parametrize("bs", [8, 16, 32, 64, 128, 256])
def test_block_sizes(bs):
    rng = np.random.default_rng(bs)
    part = max(512, bs)
    case = gen.make_case("bs", rng, [1, bs - 1, bs, bs + 1, 3 * bs + 5, 1500], 8, 2, 128, bs,
                         "bf16")
    _check(case, partition_size=part)


@pytest.mark.parametrize("part", [32, 64, 256, 512, 768, 1024, 1536, 2048])
def test_partition_sizes_agree(part):
    rng = np.random.default_rng(77)
    case = gen.make_case("part", rng, [1, 100, 700, 3000, 4500], 16, 4, 128, 16, "bf16")
    _check(case, partition_size=part)


@pytest.mark.parametrize("part", [1024, 1280, 1536])
def test_partition_sizes_agree_group8(part):
    """G = 8 on 64-token blocks (the long-context shape) at the partition sizes the default
    policy can pick there, with ragged last partitions and a sequence of one token."""
    rng = np.random.default_rng(78)
    case = gen.make_case("part8", rng, [1, 64, 1535, 1537, 4000, 9000], 64, 8, 128, 64, "bf16")
    _check(case, partition_size=part)


def test_zero_length_and_single_token():
    rng = np.random.default_rng(5)
    case = gen.make_case("edge", rng, [0, 1, 0, 600], 4, 4, 128, 16, "f32")
    got, out = run_decode(case)
    assert (got[0] == 0).all() and (got[2] == 0).all()
    # one token: exp(0) = 1, out = v exactly
    blk = case.block_tables[1, 0]
    assert np.array_equal(got[1], case.v_cache[blk, :, 0, :].astype(np.float64))
    _check(case)


def test_largest_batches():
    """The largest batches each launch form takes: 65535 sequences on the full grid (its
    sequence dimension) and 32767 over a work list (an item's top bit is reserved), one or two
    tokens each. A one-token sequence's output is its V row exactly (e^0 = 1); a two-token one
    is checked against the oracle on a sample."""
    import paged_kv_cache_402_amd as pk
    for B, use_list in ((65535, False), (32767, True)):
        rng = np.random.default_rng(B)
        lens = (1 + (np.arange(B) % 2)).astype(np.int32)
        case = gen.make_case("maxb", rng, lens, 2, 1, 64, 8, "f32", width=1, poison=False)
        q, k, v = to_dev(case.q, "f32"), to_dev(case.k_cache, "f32"), to_dev(case.v_cache, "f32")
        out = torch.full((B, 2, 64), float("nan"), dtype=torch.float32, device="cuda")
        work = i32(pk.decode_work_list(lens, 1, 8, 32)) if use_list else None
        pk.paged_attention_decode(out, q, k, v, i32(case.block_tables), i32(lens), case.scale,
                                  partition_size=32, work_list=work)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        one = np.nonzero(lens == 1)[0]
        rows = case.v_cache[case.block_tables[one, 0], 0, 0, :]          # [n][64]
        assert np.array_equal(got[one, 0], rows) and np.array_equal(got[one, 1], rows)
        seqs = [1, 3, B // 2 | 1, B - 2 if (B - 2) % 2 else B - 1]
        ref = oracle(case, seqs=seqs)
        assert max_err(got[seqs].astype(np.float64), ref[seqs]) <= GATE["f32"]


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations_match_oracle(seed):
    """Seeded draws over the supported space at once: dtype, head_dim, group, KV heads, block
    size, partition size, batch and lengths (with 0, 1 and block/partition edges), launch form
    (full grid, work list, packed list) and whether the step's new token is stored by the
    pass. Each draw is checked against the oracle; with the store fused, the caches must also
    be bitwise those of reshape_and_cache."""
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(9000 + seed)
    dtype = ["f32", "f16", "bf16"][seed % 3]
    d = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([1, 2, 4] if d == 256 else [1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([8, 16, 32, 64]))
    parts = [p for p in (32, 64, 128, 256, 512, 768, 1024, 1536, 2048) if p % bs == 0 and p >= bs]
    part = int(rng.choice(parts))
    B = int(rng.integers(1, 13))
    edges = [1, bs - 1, bs, bs + 1, part, part + 1, 2 * part + 3]
    lens = [int(rng.choice(edges)) if rng.random() < 0.5 else int(rng.integers(1, 3 * part))
            for _ in range(B)]
    form = ["full", "list", "packed"][(seed // 3) % 3]
    fused = bool(seed % 2)
    W = max(-(-L // bs) for L in lens) + 1
    case = gen.make_case("rnd", rng, lens, G * hkv, hkv, d, bs, dtype, width=W)
    q, k, v = to_dev(case.q, dtype), to_dev(case.k_cache, dtype), to_dev(case.v_cache, dtype)
    tables, lns = i32(case.block_tables), i32(case.seq_lens)
    if form == "full":
        work = None
    elif form == "list":
        work = i32(pk.decode_work_list(case.seq_lens, W, bs, part))
    else:
        lst, rows = pk.decode_work_list_packed(case.seq_lens, W, bs, part, part // 4)
        work = (i32(lst), rows)
    out = torch.full((B, G * hkv, d), float("nan"), dtype=torch.float32, device="cuda")
    if fused:
        # the last token's K/V come in as new rows; its slot is poisoned beforehand
        nk = case.k_cache[case.block_tables[np.arange(B), (np.array(lens) - 1) // bs], :,
                          (np.array(lens) - 1) % bs, :].copy()
        nv = case.v_cache[case.block_tables[np.arange(B), (np.array(lens) - 1) // bs], :,
                          (np.array(lens) - 1) % bs, :].copy()
        want_k, want_v = k.clone(), v.clone()
        for b, L in enumerate(lens):
            blk = int(case.block_tables[b, (L - 1) // bs])
            k[blk, :, (L - 1) % bs, :] = float("nan")
            v[blk, :, (L - 1) % bs, :] = float("nan")
        pk.paged_attention_decode_append(out, q, to_dev(nk, dtype), to_dev(nv, dtype), k, v,
                                         tables, lns, case.scale, partition_size=part,
                                         work_list=work)
    else:
        pk.paged_attention_decode(out, q, k, v, tables, lns, case.scale, partition_size=part,
                                  work_list=work)
    torch.cuda.synchronize()
    if fused:
        assert torch.equal(k.view(torch.uint8), want_k.view(torch.uint8))
        assert torch.equal(v.view(torch.uint8), want_v.view(torch.uint8))
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert max_err(got, oracle(case)) <= GATE[dtype], (dtype, d, G, hkv, bs, part, form, fused)


def test_seq_lens_beyond_table_are_clamped():
    rng = np.random.default_rng(6)
    case = gen.make_case("clamp", rng, [48, 20], 4, 4, 64, 16, "f32", width=3)
    lens_big = i32([10 ** 6, 20])
    got, _ = run_decode(case, lens=lens_big)
    clamped = gen.PagedDecodeCase(**{**case.__dict__, "seq_lens": np.array([48, 20], np.int32)})
    ref = oracle(clamped)
    assert max_err(got, ref) <= 1e-5


def test_invalid_table_entries_are_skipped_without_faulting():
    """Table entries outside the pool are skipped with their tokens (the kernel never
    addresses memory through them). Sequence 2 lists only valid blocks and must match the
    oracle exactly as usual; sequences 0 and 1 must match the oracle over the tokens of their
    valid blocks (attention is invariant to which tokens sit where, so dropping a logical block
    is the same as a shorter table without it)."""
    rng = np.random.default_rng(8)
    case = gen.make_case("bad", rng, [40, 40, 40], 4, 4, 128, 16, "bf16")
    bad = case.block_tables.copy()
    bad[0, 1] = case.num_blocks + 5     # out of the pool
    bad[1, 0] = -7
    got, _ = run_decode(case, tables=i32(bad))
    assert np.isfinite(got).all()
    ref = oracle(case)
    assert max_err(got[2], ref[2]) <= GATE["bf16"]
    kept = np.full_like(case.block_tables, -1)
    kept[0, :2] = case.block_tables[0, [0, 2]]    # 16 + 8 tokens
    kept[1, :2] = case.block_tables[1, [1, 2]]
    kept[2] = case.block_tables[2]
    short = gen.PagedDecodeCase(**{**case.__dict__, "block_tables": kept,
                                   "seq_lens": np.array([24, 24, 40], np.int32)})
    ref_kept = oracle(short)
    assert max_err(got[:2], ref_kept[:2]) <= GATE["bf16"]


def test_scale_zero_gives_mean_of_values():
    rng = np.random.default_rng(9)
    case = gen.make_case("s0", rng, [37, 600], 8, 2, 128, 16, "f32")
    case.scale = 0.0
    _check(case)


# --------------------------------------------------------------------------------------------
# invariances the pages state, bit for bit on the device
# --------------------------------------------------------------------------------------------

def _scatter_logical(keys, bs, ids, num_blocks, dtype):
    """[L][Hkv][d] rows -> pool with the rows placed through `ids` (test-side placement)."""
    L, H, d = keys.shape
    pool = np.full((num_blocks, H, bs, d), gen.nan_value(dtype), dtype=keys.dtype)
    nb = -(-L // bs)
    padded = np.full((nb * bs, H, d), gen.nan_value(dtype), dtype=keys.dtype)
    padded[:L] = keys
    pool[ids] = padded.reshape(nb, bs, H, d).transpose(0, 2, 1, 3)
    return pool


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_placement_does_not_change_a_bit(dtype):
    """P1 §4.2: the kernel sees the same logical sequence wherever its blocks sit."""
    rng = np.random.default_rng(21)
    bs, H, G, d = 16, 2, 4, 128
    lens = [35, 700, 1500]
    nbp = 400
    keys = [gen.normal(rng, (L, H, d), dtype) for L in lens]
    vals = [gen.normal(rng, (L, H, d), dtype) for L in lens]
    q = to_dev(gen.normal(rng, (3, H * G, d), dtype), dtype)
    outs = []
    for trial in range(3):
        perm = rng.permutation(nbp)
        pos = 0
        kpool = np.full((nbp, H, bs, d), gen.nan_value(dtype), dtype=keys[0].dtype)
        vpool = np.full_like(kpool, gen.nan_value(dtype))
        table = np.full((3, 100), -1, np.int32)
        for s, L in enumerate(lens):
            nb = -(-L // bs)
            ids = perm[pos:pos + nb]
            pos += nb
            table[s, :nb] = ids
            kp = _scatter_logical(keys[s], bs, ids, nbp, dtype)
            vp = _scatter_logical(vals[s], bs, ids, nbp, dtype)
            kpool[ids] = kp[ids]
            vpool[ids] = vp[ids]
        case = gen.PagedDecodeCase("perm", dtype, H * G, H, d, bs, nbp, np.array(lens, np.int32),
                                   table, 0.09)
        got, out = run_decode(case, q=q, k=to_dev(kpool, dtype), v=to_dev(vpool, dtype))
        outs.append(out.cpu())
        case.q, case.k_cache, case.v_cache = to_host(q, dtype), kpool, vpool
        if trial == 0:
            ref = oracle(case)
            assert max_err(got, ref) <= GATE[dtype]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_shared_prefix_equals_private_copies_bitwise():
    """P3 §2.2.3 key point / P1 §6.1: sequences pointing at one set of prefix blocks get
    exactly what they would get from private copies of those blocks."""
    case = gen.llama3_8b_gqa_prefix_case(num_seqs=6)
    got_shared, out_shared = run_decode(case)
    prefix = case.meta["prefix_blocks"]
    # sequences 1.. get their own copy of the prefix, in blocks appended past the pool
    extra = (case.num_seqs - 1) * len(prefix)
    pad = np.full((extra,) + case.k_cache.shape[1:], gen.nan_value("bf16"), dtype=np.uint16)
    kc = np.concatenate([case.k_cache, pad])
    vc = np.concatenate([case.v_cache, pad])
    tables = case.block_tables.copy()
    dst = case.num_blocks
    for s in range(1, case.num_seqs):
        for j, src in enumerate(prefix):
            kc[dst], vc[dst] = kc[src], vc[src]
            tables[s, j] = dst
            dst += 1
    got_priv, out_priv = run_decode(case, k=to_dev(kc, "bf16"), v=to_dev(vc, "bf16"),
                                    tables=i32(tables))
    assert torch.equal(out_shared.cpu(), out_priv.cpu())
    # equal queries over the prefix alone: identical rows
    q_same = np.repeat(case.q[:1], case.num_seqs, axis=0)
    lens = np.full(case.num_seqs, case.meta["prefix_tokens"], np.int32)
    got_p, out_p = run_decode(case, q=to_dev(q_same, "bf16"), lens=i32(lens))
    for s in range(1, case.num_seqs):
        assert torch.equal(out_p[s].cpu(), out_p[0].cpu())


def test_repeat_runs_are_bitwise_identical():
    case = gen.long_context_splitk_case(num_seqs=2, min_len=3000, max_len=9000)
    _, a = run_decode(case)
    _, b = run_decode(case)
    assert torch.equal(a.cpu(), b.cpu())


# --------------------------------------------------------------------------------------------
# full sizes in the benchmark's launch configuration, checked on sampled sequences
# --------------------------------------------------------------------------------------------

def _device_values(case, seed):
    """Full-size pools from the device generator; the sampled sequences' blocks are copied
    back for the oracle."""
    dt = case.dtype
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    k = gen.device_normal(shape, dt, seed, "cuda")
    v = gen.device_normal(shape, dt, seed + 1, "cuda")
    q = gen.device_normal((case.num_seqs, case.num_q_heads, case.head_dim), dt, seed + 2, "cuda")
    return q, k, v


def _sampled_reference(case, q, k, v, seqs):
    dt = case.dtype
    bs = case.block_size
    sub_tables, ids_all = [], []
    for s in seqs:
        nb = -(-int(case.seq_lens[s]) // bs)
        ids_all.extend(case.block_tables[s, :nb].tolist())
    uniq = sorted(set(ids_all))
    remap = {b: i for i, b in enumerate(uniq)}
    idx = torch.tensor(uniq, dtype=torch.long, device="cuda")
    ksub, vsub = to_host(k[idx], dt), to_host(v[idx], dt)
    width = case.block_tables.shape[1]
    tab = np.full((len(seqs), width), -1, np.int32)
    for r, s in enumerate(seqs):
        nb = -(-int(case.seq_lens[s]) // bs)
        tab[r, :nb] = [remap[int(b)] for b in case.block_tables[s, :nb]]
    sub = gen.PagedDecodeCase("sample", dt, case.num_q_heads, case.num_kv_heads, case.head_dim, bs,
                              len(uniq), case.seq_lens[list(seqs)], tab, case.scale,
                              q=to_host(q[list(seqs)], dt), k_cache=ksub, v_cache=vsub)
    return oracle(sub)


@pytest.mark.parametrize("form", ["bench", "bench_f32out", "grid512"])
@pytest.mark.parametrize("which", ["llama2_7b_mha", "llama3_8b_gqa_prefix", "long_context_splitk"])
def test_full_size_sampled(which, form):
    """form "bench" is the benchmark's launch exactly as timed: the default partition for the
    shapes, the host work list with its ticketed tail made private, an initialised workspace
    (late units by ticket), every sequence's newest K/V row (fresh values) stored by the
    per-partition pass itself, then the merge as its own launch, into an output of the KV
    dtype; the reference reads the caches the pass leaves. "bench_f32out": the same launches
    into an fp32 output (the arithmetic before the final rounding). "grid512": the one-call
    decode over the full grid at 512-token partitions."""
    import paged_kv_cache_402_amd as pk
    maker = gen.WORKLOADS[which]
    case = maker(values=False)
    q, k, v = _device_values(case, 4020)
    if form == "grid512":
        got, out = run_decode(case, q=q, k=k, v=v)
    else:
        B, Hq, D = q.shape
        W, bs, Hkv, dt = case.block_tables.shape[1], case.block_size, case.num_kv_heads, case.dtype
        part = pk.default_partition(B, Hq, Hkv, D, bs, W)
        need = pk.decode_workspace_bytes(B, Hq, W, bs, D, part)
        items = pk.decode_work_list(case.seq_lens, W, bs, part)
        if need:    # late units are ticketed only from an initialised workspace
            tail = pk.decode_ticketed_items(TORCH_DT[dt], D, Hq, Hkv, bs, part, items.shape[0])
            items, _ = pk.decode_work_list_private_tail(items, case.block_tables, case.seq_lens,
                                                        bs, case.num_blocks, part, tail)
        work = i32(items)
        k_new = gen.device_normal((B, Hkv, D), dt, 4030, "cuda")
        v_new = gen.device_normal((B, Hkv, D), dt, 4031, "cuda")
        odt = TORCH_DT[dt] if form == "bench" else torch.float32
        out = torch.full((B, Hq, D), float("nan"), dtype=odt, device="cuda")
        tables, lens_d = i32(case.block_tables), i32(case.seq_lens)
        ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
        if need:
            pk.decode_workspace_init(ws)
        policy = pk.decode_kv_policy(case.block_tables, case.seq_lens, bs, case.num_blocks)
        assert policy == pk.KV_STREAM          # no batch here mostly re-reads shared blocks
        pk.paged_attention_partitions_append(out, q, k_new, v_new, k, v, tables, lens_d,
                                             case.scale, partition_size=part, workspace=ws,
                                             work_list=work, kv_policy=policy)
        pk.paged_attention_reduce(out, lens_d, bs, W, ws, partition_size=part)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        # the new rows sit where each table puts token L - 1
        lens = case.seq_lens.astype(np.int64)
        blk = torch.from_numpy(case.block_tables[np.arange(B), (lens - 1) // bs].astype(np.int64))
        off = torch.from_numpy((lens - 1) % bs)
        for cache, new in ((k, k_new), (v, v_new)):
            rows = cache[blk.cuda(), :, off.cuda()]
            assert torch.equal(rows.view(torch.int16 if dt != "f32" else torch.int32),
                               new.view(torch.int16 if dt != "f32" else torch.int32))
    assert np.isfinite(got).all()
    rng = np.random.default_rng(1)
    nsamp = 2 if which == "long_context_splitk" else 6
    seqs = sorted(rng.choice(case.num_seqs, nsamp, replace=False).tolist())
    # always include the longest and the shortest sequence
    seqs = sorted(set(seqs) | {int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens))})
    ref = _sampled_reference(case, q, k, v, seqs)
    odt = case.dtype if form == "bench" else None
    for r, s in enumerate(seqs):
        assert (np.abs(got[s] - ref[r]) <= out_gate(ref[r], case.dtype, odt)).all(), "seq %d" % s
        if odt is not None:
            # the benchmarked rows' magnitudes keep one bf16 rounding inside the 2e-3 bar
            assert max_err(got[s], ref[r]) <= GATE[case.dtype], "seq %d" % s


# --------------------------------------------------------------------------------------------
# the KV read cache policy changes speed only
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("form", ["mha_f16_grid", "gqa_bf16_list_append", "g8_bf16_mfma_grid",
                                  "f32_g2_packed", "shared_prefix"])
def test_kv_read_policies_give_the_same_bits(form):
    """Every decode kernel exists in two builds, non-temporal KV loads and default-policy KV
    loads (kv_policy). The loaded bytes are the same, so outputs and caches must be bitwise
    the same; one of the two is checked against the oracle as well."""
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(7400)
    grid = form.endswith("grid")
    if form == "mha_f16_grid":
        case = gen.make_case("pol1", rng, [1, 31, 700, 2049, 4000], 16, 16, 128, 32, "f16")
        part, pack = 512, 0
    elif form == "gqa_bf16_list_append":
        case = gen.make_case("pol2", rng, [int(x) for x in rng.integers(1, 3000, 40)], 32, 8,
                             128, 16, "bf16")
        part, pack = 2048, 0
    elif form == "g8_bf16_mfma_grid":
        case = gen.make_case("pol3", rng, [5000, 17, 1536, 3100], 64, 8, 128, 16, "bf16")
        part, pack = 1536, 0
    elif form == "f32_g2_packed":
        case = gen.make_case("pol4", rng, [int(x) for x in rng.integers(1, 200, 60)], 16, 8, 64,
                             16, "f32")
        part, pack = 512, 64
    else:
        case = _share_case("pol5", 7401, [900, 1300, 700, 2000], 32, 8, 16, "bf16", 512,
                           [0, 1, 2, 3])
        part, pack = 256, 0
    dt, B, Hq, D = case.dtype, case.num_seqs, case.num_q_heads, case.head_dim
    W, bs, Hkv = case.block_tables.shape[1], case.block_size, case.num_kv_heads
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    q = to_dev(case.q, dt)
    if grid:
        work = None
    elif pack:
        lst, rows = pk.decode_work_list_packed(case.seq_lens, W, bs, part, pack)
        work = (i32(lst), rows)
    else:
        work = i32(pk.decode_work_list(case.seq_lens, W, bs, part))
    outs, caches = [], []
    for policy in (pk.KV_STREAM, pk.KV_CACHED):
        k, v = to_dev(case.k_cache, dt), to_dev(case.v_cache, dt)
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        if form == "gqa_bf16_list_append":
            k_new = gen.device_normal((B, Hkv, D), dt, 7402, "cuda")
            v_new = gen.device_normal((B, Hkv, D), dt, 7403, "cuda")
            pk.paged_attention_decode_append(out, q, k_new, v_new, k, v, tables, lens, case.scale,
                                             partition_size=part, work_list=work,
                                             kv_policy=policy)
        elif form == "shared_prefix":
            mem, pp, items = pk.plan_shared_prefix(case.block_tables, case.seq_lens, bs, part)
            assert pp > 0
            pk.paged_attention_decode(out, q, k, v, tables, lens, case.scale, partition_size=part,
                                      work_list=i32(items), shared_prefix=(i32(mem), pp),
                                      kv_policy=policy)
        else:
            pk.paged_attention_decode(out, q, k, v, tables, lens, case.scale, partition_size=part,
                                      work_list=work, kv_policy=policy)
        torch.cuda.synchronize()
        outs.append(out)
        caches.append((k, v))
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    ib = torch.int32 if dt == "f32" else torch.int16
    for c0, c1 in zip(caches[0], caches[1]):
        assert torch.equal(c0.view(ib), c1.view(ib))
    got = outs[1].cpu().numpy().astype(np.float64)
    if form == "gqa_bf16_list_append":
        # the reference reads the caches the pass left (the new rows stored in place)
        case.k_cache, case.v_cache = to_host(caches[1][0], dt), to_host(caches[1][1], dt)
    ref = oracle(case)
    assert np.isfinite(got).all()
    assert max_err(got, ref) <= GATE[dt]


# --------------------------------------------------------------------------------------------
# split-K: a reused caller workspace and the two-launch form (partitions, then the merge)
# --------------------------------------------------------------------------------------------

def test_caller_workspace_reused_bitwise():
    import paged_kv_cache_402_amd as pk
    case = gen.make_case("splitk", np.random.default_rng(31), [40, 1100, 2900, 513, 1024], 16, 4,
                         128, 16, "bf16", width=200)
    B, Hq, D = case.q.shape
    need = pk.decode_workspace_bytes(B, Hq, 200, 16, D, 512)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # stale contents
    q, k, v = to_dev(case.q, "bf16"), to_dev(case.k_cache, "bf16"), to_dev(case.v_cache, "bf16")
    outs = []
    for _ in range(3):
        o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        pk.paged_attention_decode(o, q, k, v, i32(case.block_tables), i32(case.seq_lens),
                                  case.scale, partition_size=512, workspace=ws)
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert max_err(outs[0].numpy().astype(np.float64), oracle(case)) <= GATE["bf16"]


def test_two_launch_split_matches_oracle():
    import paged_kv_cache_402_amd as pk
    case = gen.make_case("split2", np.random.default_rng(32), [7, 600, 3000, 1537], 32, 8, 128, 16,
                         "bf16", width=200)
    B, Hq, D = case.q.shape
    q, k, v = to_dev(case.q, "bf16"), to_dev(case.k_cache, "bf16"), to_dev(case.v_cache, "bf16")
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = pk.paged_attention_partitions(out, q, k, v, tables, lens, case.scale)
    pk.paged_attention_reduce(out, lens, 16, 200, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert max_err(got, oracle(case)) <= GATE["bf16"]


# --------------------------------------------------------------------------------------------
# the per-partition pass over a host work list: bitwise the full-grid result
# --------------------------------------------------------------------------------------------

def _decode_both(case, part, shuffle=None, extra=None):
    import paged_kv_cache_402_amd as pk
    dt = case.dtype
    B, Hq, D = case.q.shape
    W = case.block_tables.shape[1]
    q, k, v = to_dev(case.q, dt), to_dev(case.k_cache, dt), to_dev(case.v_cache, dt)
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    a = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    pk.paged_attention_decode(a, q, k, v, tables, lens, case.scale, partition_size=part)
    items = pk.decode_work_list(case.seq_lens, W, case.block_size, part)
    if shuffle is not None:
        items = shuffle.permutation(items)
    if extra is not None:
        items = np.concatenate([items, np.asarray(extra, np.int32)])
    pk.paged_attention_decode(b, q, k, v, tables, lens, case.scale, partition_size=part,
                              work_list=i32(items))
    torch.cuda.synchronize()
    return a.cpu(), b.cpu()


@pytest.mark.parametrize("part", [32, 512])
def test_work_list_decode_is_bitwise_the_grid_decode(part):
    rng = np.random.default_rng(40)
    case = gen.make_case("wl", rng, [0, 1, 15, 16, 17, 511, 512, 513, 1024, 1500, 3001], 16, 4,
                         128, 16, "bf16", width=200)
    a, b = _decode_both(case, part)
    assert torch.equal(a, b)
    assert max_err(b.numpy().astype(np.float64), oracle(case)) <= GATE["bf16"]


def test_work_list_order_and_skipped_items():
    """Any order of the items gives the same bits; items past a sequence's end or naming a
    sequence beyond the batch do nothing."""
    rng = np.random.default_rng(41)
    case = gen.make_case("wl2", rng, [5, 700, 2100, 64], 8, 8, 128, 16, "f16", width=160)
    junk = [(4 << 16) | 0, (0 << 16) | 3, (1 << 16) | 9]
    a, b = _decode_both(case, 512, shuffle=np.random.default_rng(3), extra=junk)
    assert torch.equal(a, b)


def test_work_list_full_size_gqa_prefix_bitwise():
    import paged_kv_cache_402_amd as pk
    case = gen.llama3_8b_gqa_prefix_case(values=False)
    q, k, v = _device_values(case, 4021)
    B, Hq, D = case.num_seqs, case.num_q_heads, case.head_dim
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    a = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    pk.paged_attention_decode(a, q, k, v, tables, lens, case.scale, partition_size=512)
    items = pk.decode_work_list(case.seq_lens, case.table_width, case.block_size, 512)
    pk.paged_attention_decode(b, q, k, v, tables, lens, case.scale, partition_size=512,
                              work_list=i32(items))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------------------------------------
# packed work lists: short partitions four to a workgroup, one wave each
# --------------------------------------------------------------------------------------------

def _packed_rows_items(lst, rows):
    u = np.asarray(lst, np.int32).view(np.uint32)
    packed = set()
    for r in u[:rows]:
        if r & 0x80000000:
            i = int(r & 0x7FFFFFFF)
            packed |= {(int(x >> 16), int(x & 0xFFFF)) for x in u[i:i + 4]}
    return packed


@pytest.mark.parametrize("dtype,hq,hkv,d,bs,part,pack", [
    ("bf16", 32, 32, 128, 16, 2048, 64),      # MHA, the long-tail serving shape
    ("f16", 40, 40, 128, 32, 2048, 512),      # every partition of <= 512 tokens packed
    ("bf16", 32, 8, 128, 16, 512, 128),       # G 4
    ("bf16", 64, 8, 128, 64, 1024, 64),       # G 8: matrix-core score product
    ("f32", 8, 4, 64, 8, 128, 32),
    ("bf16", 8, 2, 256, 16, 256, 64),
])
def test_packed_work_list_matches_oracle(dtype, hq, hkv, d, bs, part, pack):
    """Partitions of at most `pack` tokens run one wave each; the rest as in the plain list.
    Lengths cover empty sequences, single tokens, short sequences (packed, single partition),
    sequences whose short last partition is packed and merged with full ones (partials), a
    last group padded to four, and a row of NaN-poisoned slots past every end."""
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(70)
    lens = [0, 1, 2, 5, bs - 1, bs, pack, pack + 1, part, part + 1, part + pack, 2 * part + 3,
            3 * part, 700, 33, 17, 9]
    case = gen.make_case("pk", rng, lens, hq, hkv, d, bs, dtype, width=-(-max(lens) // bs) + 2)
    B, W = len(lens), case.block_tables.shape[1]
    q, k, v = to_dev(case.q, dtype), to_dev(case.k_cache, dtype), to_dev(case.v_cache, dtype)
    tables, lns = i32(case.block_tables), i32(case.seq_lens)
    lst, rows = pk.decode_work_list_packed(case.seq_lens, W, bs, part, pack)
    assert rows < len(lst)                      # something was packed
    a = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    pk.paged_attention_decode(a, q, k, v, tables, lns, case.scale, partition_size=part,
                              work_list=i32(pk.decode_work_list(case.seq_lens, W, bs, part)))
    pk.paged_attention_decode(b, q, k, v, tables, lns, case.scale, partition_size=part,
                              work_list=(i32(lst), rows))
    torch.cuda.synchronize()
    got = b.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert max_err(got, oracle(case)) <= GATE[dtype]
    # sequences none of whose partitions was packed are bitwise the plain list's
    packed = _packed_rows_items(lst, rows)
    for s, L in enumerate(lens):
        if not any(it[0] == s for it in packed):
            assert torch.equal(a[s], b[s]), s


def test_packed_work_list_fused_append():
    """The packed wave of a sequence's last partition stores the appended token: caches are
    bitwise those of reshape_and_cache + decode, outputs within the gate of the oracle."""
    import paged_kv_cache_402_amd as pk
    dtype, hq, hkv, d, bs, part, pack = "f16", 16, 16, 128, 32, 1024, 128
    rng = np.random.default_rng(71)
    lens = [1, 2, 31, 32, 33, 100, 1024, 1030, 2100, 64, 0]
    case = gen.make_case("pkapp", rng, lens, hq, hkv, d, bs, dtype, width=2100 // bs + 2)
    B, W = len(lens), case.block_tables.shape[1]
    k_new, v_new = gen.normal(rng, (B, hkv, d), dtype), gen.normal(rng, (B, hkv, d), dtype)
    slots = np.array([-1 if L == 0 else
                      int(case.block_tables[b, (L - 1) // bs]) * bs + (L - 1) % bs
                      for b, L in enumerate(lens)], np.int32)
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    for sl in slots:
        if sl >= 0:
            kc[sl // bs, :, sl % bs, :] = gen.nan_value(dtype)
            vc[sl // bs, :, sl % bs, :] = gen.nan_value(dtype)
    q, tables, lns = to_dev(case.q, dtype), i32(case.block_tables), i32(case.seq_lens)
    lst, rows = pk.decode_work_list_packed(case.seq_lens, W, bs, part, pack)
    k1, v1 = to_dev(kc, dtype), to_dev(vc, dtype)
    pk.reshape_and_cache(to_dev(k_new, dtype), to_dev(v_new, dtype), k1, v1, i32(slots))
    k2, v2 = to_dev(kc, dtype), to_dev(vc, dtype)
    out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode_append(out, q, to_dev(k_new, dtype), to_dev(v_new, dtype), k2, v2,
                                     tables, lns, case.scale, partition_size=part,
                                     work_list=(i32(lst), rows))
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
    ref = gen.PagedDecodeCase("pkapp", dtype, hq, hkv, d, bs, case.num_blocks, case.seq_lens,
                              case.block_tables, case.scale, q=case.q,
                              k_cache=to_host(k2, dtype), v_cache=to_host(v2, dtype))
    assert max_err(out.cpu().numpy().astype(np.float64), oracle(ref)) <= GATE[dtype]


def test_packed_work_list_long_tail_full_size_sampled():
    """The long-tail serving shape at full size (128 sequences, 40 MHA heads, fp16, block 32,
    geometric lengths of mean 200 clipped to [1, 2048]) with 2048-token partitions and
    partitions of at most 64 tokens packed, in the fp16 output the benchmark writes, against
    the oracle on sampled sequences (the shortest, the longest and random ones)."""
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(72)
    lens = np.clip(rng.geometric(1.0 / 200, size=128), 1, 2048).astype(np.int32)
    case = gen.make_case("pklt", rng, lens, 40, 40, 128, 32, "f16", width=64, values=False)
    q, k, v = _device_values(case, 4023)
    lst, rows = pk.decode_work_list_packed(case.seq_lens, 64, 32, 2048, 64)
    assert rows < len(lst)
    out = torch.full((128, 40, 128), float("nan"), dtype=torch.float16, device="cuda")
    pk.paged_attention_decode(out, q, k, v, i32(case.block_tables), i32(case.seq_lens),
                              case.scale, partition_size=2048, work_list=(i32(lst), rows))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    order = np.argsort(lens, kind="stable")
    seqs = sorted(set(order[:6].tolist()) | set(order[-3:].tolist())
                  | {int(x) for x in rng.choice(128, 5, replace=False)})
    ref = _sampled_reference(case, q, k, v, seqs)
    for r, s_ in enumerate(seqs):
        gate = out_gate(ref[r], "f16", "f16")
        assert (np.abs(got[s_] - ref[r]) <= gate).all(), "seq %d" % s_


def test_packed_work_list_short_batch_full_size_sampled():
    """2048 short GQA sequences (lengths 1..48), every partition packed (32 and 48 tokens),
    against the oracle on sampled sequences and against the plain list."""
    import paged_kv_cache_402_amd as pk
    case = gen.llama3_8b_short_batch_case(values=False)
    q, k, v = _device_values(case, 4024)
    B, W, bs = case.num_seqs, case.table_width, case.block_size
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    plain = torch.empty((B, 32, 128), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode(plain, q, k, v, tables, lens, case.scale, partition_size=2048,
                              work_list=i32(pk.decode_work_list(case.seq_lens, W, bs, 2048)))
    rng = np.random.default_rng(5)
    seqs = sorted(set(rng.choice(B, 8, replace=False).tolist())
                  | {int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens))})
    ref = _sampled_reference(case, q, k, v, seqs)
    for pack in (32, 48):
        lst, rows = pk.decode_work_list_packed(case.seq_lens, W, bs, 2048, pack)
        out = torch.full_like(plain, float("nan"))
        pk.paged_attention_decode(out, q, k, v, tables, lens, case.scale, partition_size=2048,
                                  work_list=(i32(lst), rows))
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        for r, s_ in enumerate(seqs):
            assert max_err(got[s_], ref[r]) <= GATE["bf16"], "seq %d pack %d" % (s_, pack)
        # the same attention up to fp32 rounding order
        assert float((out - plain).abs().max()) <= 1e-5


# --------------------------------------------------------------------------------------------
# shared-prefix decode: the members' shared partitions on the matrix cores
# --------------------------------------------------------------------------------------------

def _share_case(name, seed, lens, hq, hkv, bs, dtype, share_tokens, members, width=None):
    """A batch whose members list member 0's blocks for their first share_tokens tokens."""
    rng = np.random.default_rng(seed)
    case = gen.make_case(name, rng, lens, hq, hkv, 128, bs, dtype, width=width, values=False)
    nsh = share_tokens // bs
    for b in members[1:]:
        case.block_tables[b, :nsh] = case.block_tables[members[0], :nsh]
    case.q = gen.normal(rng, (len(lens), hq, 128), dtype)
    case.k_cache, case.v_cache = gen.fill_pool(rng, case.num_blocks, hkv, bs, 128, dtype,
                                               case.block_tables, case.seq_lens)
    return case


def _run_shared(case, part, min_members=2, members_override=None):
    import paged_kv_cache_402_amd as pk
    dt = case.dtype
    B, Hq, D = case.q.shape
    W = case.block_tables.shape[1]
    mem, pp, items = pk.plan_shared_prefix(case.block_tables, case.seq_lens, case.block_size,
                                           part, min_members)
    if members_override is not None:
        mem = np.asarray(members_override, np.int32)
    q, k, v = to_dev(case.q, dt), to_dev(case.k_cache, dt), to_dev(case.v_cache, dt)
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode(out, q, k, v, tables, lens, case.scale, partition_size=part,
                              work_list=i32(items), shared_prefix=(i32(mem), pp))
    plain = torch.full_like(out, float("nan"))
    pk.paged_attention_decode(plain, q, k, v, tables, lens, case.scale, partition_size=part)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64), plain.cpu().numpy().astype(np.float64), mem,
            pp)


@pytest.mark.parametrize("dtype,hq,hkv,bs,part,share,n", [
    ("bf16", 32, 8, 16, 512, 1024, 21),      # G 4: two shared partitions, a partial chunk
    ("f16", 64, 8, 32, 256, 768, 11),        # G 8: chunks of 8 sequences
    ("bf16", 8, 8, 8, 128, 384, 40),         # G 1: one partial chunk of 64
    ("bf16", 16, 8, 64, 64, 256, 9),         # G 2: four one-block partitions
])
def test_shared_prefix_decode_matches_oracle(dtype, hq, hkv, bs, part, share, n):
    rng = np.random.default_rng(50)
    lens = [int(x) for x in rng.integers(share + 1, share + 2500, size=n)]
    lens += [300, share + 7]                  # two sequences outside the group
    members = list(range(n))
    case = _share_case("shared", 51, lens, hq, hkv, bs, dtype, share, members, width=None)
    got, plain, mem, pp = _run_shared(case, part)
    assert mem.tolist() == members and pp == share // part
    ref = oracle(case)
    assert np.isfinite(got).all()
    assert max_err(got, ref) <= GATE[dtype]
    assert max_err(got, plain) <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_shared_prefix_rescales_on_rising_scores(dtype):
    """Scores that jump by far more than the pass's rescale slack in later steps of a shared
    partition (and one far below everything else): the weights are taken against a reference
    max that must move several times mid-partition. Every member's query heads of a group are
    one vector u; shared keys at four tokens are u scaled by 1, 4, 8 and 12 (scores of about
    15, 59, 119 and 178 in log2 units): kept against the first reference, the last weights
    would pass 2^128 and overflow fp32, so the test fails unless the reference moves. One key
    is -5 u."""
    from oracle.storage import to_f64
    hq, hkv, bs, part, share, n = 32, 8, 16, 512, 1024, 13
    G = hq // hkv
    rng = np.random.default_rng(52)
    lens = [int(x) for x in rng.integers(share + 1, share + 900, size=n)] + [700]
    case = _share_case("rise", 53, lens, hq, hkv, bs, dtype, share, list(range(n)))
    u = rng.standard_normal((hkv, 128)).astype(np.float32)
    q = np.repeat(u, G, axis=0)                               # [hq][128]: group heads equal
    case.q = np.broadcast_to(gen.round_to_storage(q, dtype), case.q.shape).copy()
    uq = to_f64(gen.round_to_storage(u, dtype), dtype)
    for tok, f in ((40, 1.0), (300, 4.0), (600, 8.0), (900, 12.0), (1000, -5.0)):
        blk = case.block_tables[0, tok // bs]
        case.k_cache[blk, :, tok % bs, :] = gen.round_to_storage((f * uq).astype(np.float32), dtype)
    got, plain, mem, pp = _run_shared(case, part)
    assert mem.tolist() == list(range(n)) and pp == share // part
    ref = oracle(case)
    assert np.isfinite(got).all()
    assert max_err(got, ref) <= GATE[dtype]
    assert max_err(got, plain) <= 1e-4


def test_shared_prefix_with_fused_append():
    """The shared-prefix pass, then the per-partition pass over the planner's list storing the
    step's new tokens, then the merge: caches bitwise those of reshape_and_cache, the output
    that of the plain decode over the written caches (each member's new token lies in its own
    partitions, which the shared pass never reads)."""
    import paged_kv_cache_402_amd as pk
    dtype, hq, hkv, bs, part, share, n = "bf16", 32, 8, 16, 256, 512, 12
    rng = np.random.default_rng(54)
    lens = [int(x) for x in rng.integers(share + 1, share + 700, size=n)] + [share + 1, 90]
    case = _share_case("shapp", 55, lens, hq, hkv, bs, dtype, share, list(range(n + 1)))
    B, W = len(lens), case.block_tables.shape[1]
    k_new, v_new = gen.normal(rng, (B, hkv, 128), dtype), gen.normal(rng, (B, hkv, 128), dtype)
    slots = np.array([int(case.block_tables[b, (L - 1) // bs]) * bs + (L - 1) % bs
                      for b, L in enumerate(lens)], np.int32)
    mem, pp, items = pk.plan_shared_prefix(case.block_tables, case.seq_lens, bs, part)
    assert pp == share // part and mem.size == n + 1
    q, tables, lns = to_dev(case.q, dtype), i32(case.block_tables), i32(case.seq_lens)
    kn, vn = to_dev(k_new, dtype), to_dev(v_new, dtype)
    k1, v1 = to_dev(case.k_cache, dtype), to_dev(case.v_cache, dtype)
    pk.reshape_and_cache(kn, vn, k1, v1, i32(slots))
    plain = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode(plain, q, k1, v1, tables, lns, case.scale, partition_size=part)
    k2, v2 = to_dev(case.k_cache, dtype), to_dev(case.v_cache, dtype)
    out = torch.full_like(plain, float("nan"))
    ws = torch.empty(pk.decode_workspace_bytes(B, hq, W, bs, 128, part), dtype=torch.uint8,
                     device="cuda")
    pk.paged_attention_prefix(out, q, k2, v2, tables, lns, case.scale, i32(mem), pp, ws,
                              partition_size=part)
    pk.paged_attention_partitions_append(out, q, kn, vn, k2, v2, tables, lns, case.scale,
                                         partition_size=part, workspace=ws, work_list=i32(items))
    pk.paged_attention_reduce(out, lns, bs, W, ws, partition_size=part)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
    assert float((out - plain).abs().max()) <= 1e-4
    ref = gen.PagedDecodeCase("shapp", dtype, hq, hkv, 128, bs, case.num_blocks, case.seq_lens,
                              case.block_tables, case.scale, q=case.q,
                              k_cache=to_host(k2, dtype), v_cache=to_host(v2, dtype))
    assert max_err(out.cpu().numpy().astype(np.float64), oracle(ref)) <= GATE[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_shared_prefix_skips_out_of_pool_entries_and_short_members(dtype):
    """The shared-prefix pass follows the per-partition kernel's rules for inputs the planner
    never produces: a shared table entry outside the pool is left out with its tokens, and
    every member attends only to its own tokens. Members here end inside the second shared
    partition (300), inside the first (100: one partition, so the pass writes its row), exactly
    at a partition end (256) and at 0 tokens (zero row). The reference is the oracle over the
    same tables with the out-of-pool logical block taken out (attention does not depend on
    which positions the remaining tokens hold)."""
    import paged_kv_cache_402_amd as pk
    hq, hkv, bs, part, share, n = 32, 8, 16, 256, 512, 9
    rng = np.random.default_rng(57)
    lens = [int(x) for x in rng.integers(share + 1, share + 900, size=n)]
    lens += [300, 100, 256, 0, 400]          # four short members, then one non-member
    members = list(range(n + 4))
    case = _share_case("shbad", 58, lens, hq, hkv, bs, dtype, share, members)
    B, W, NB = len(lens), case.block_tables.shape[1], case.num_blocks
    bad_col = 5                              # tokens 80..95, inside every member but the last
    tables = case.block_tables.copy()
    for b in members:
        tables[b, bad_col] = NB + 3
    pp = share // part
    items = []
    for b, L in enumerate(lens):
        npart = max(1, -(-L // part))
        first = pp if b in members else 0
        items += [(b << 16) | p for p in range(first, npart)]
    dt = case.dtype
    q, k, v = to_dev(case.q, dt), to_dev(case.k_cache, dt), to_dev(case.v_cache, dt)
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode(out, q, k, v, i32(tables), i32(case.seq_lens), case.scale,
                              partition_size=part, work_list=i32(np.array(items, np.uint32)
                                                                  .view(np.int32)),
                              shared_prefix=(i32(members), pp))
    plain = torch.full_like(out, float("nan"))
    pk.paged_attention_decode(plain, q, k, v, i32(tables), i32(case.seq_lens), case.scale,
                              partition_size=part)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert (got[n + 3] == 0).all()                        # the 0-token member
    kept = np.full_like(tables, -1)
    kept_lens = case.seq_lens.copy()
    for b in range(B):
        row = case.block_tables[b].tolist()
        if b in members and lens[b] > bad_col * bs:
            assert lens[b] >= (bad_col + 1) * bs       # the left-out block is a full one
            row = row[:bad_col] + row[bad_col + 1:] + [-1]
            kept_lens[b] -= bs
        kept[b] = row
    ref = oracle(gen.PagedDecodeCase(**{**case.__dict__, "block_tables": kept,
                                        "seq_lens": kept_lens}))
    assert max_err(got, ref) <= GATE[dtype]
    assert max_err(got, plain.cpu().numpy().astype(np.float64)) <= 1e-4


@pytest.mark.parametrize("seed", range(16))
def test_shared_prefix_random_configurations(seed):
    """Seeded draws of the shared-prefix pass: dtype, group, block and partition size, shared
    length (one to three partitions), group size, private lengths, plus sequences outside
    the group; against the oracle and the per-partition path."""
    rng = np.random.default_rng(9500 + seed)
    dtype = ["bf16", "f16"][seed % 2]
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 8]))
    bs = int(rng.choice([8, 16, 32, 64]))
    part = int(rng.choice([p for p in (64, 128, 256, 512, 1024) if p % bs == 0 and p // bs <= 256]))
    share = part * int(rng.integers(1, 4))
    n = int(rng.integers(2, 40))
    lens = [share + int(rng.integers(1, 700)) for _ in range(n)] + [int(rng.integers(1, 900))]
    case = _share_case("srnd", 9600 + seed, lens, G * hkv, hkv, bs, dtype, share, list(range(n)))
    got, plain, mem, pp = _run_shared(case, part)
    assert mem.tolist() == list(range(n)) and pp == share // part
    assert np.isfinite(got).all()
    assert max_err(got, oracle(case)) <= GATE[dtype], (dtype, G, hkv, bs, part, share, n)
    assert max_err(got, plain) <= 1e-4


def test_shared_prefix_full_size_gqa_prefix_sampled():
    import paged_kv_cache_402_amd as pk
    case = gen.llama3_8b_gqa_prefix_case(values=False)
    q, k, v = _device_values(case, 4022)
    B, Hq, D = case.num_seqs, case.num_q_heads, case.head_dim
    tables, lens = i32(case.block_tables), i32(case.seq_lens)
    mem, pp, items = pk.plan_shared_prefix(case.block_tables, case.seq_lens, case.block_size, 512)
    assert mem.size == B and pp == 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode(out, q, k, v, tables, lens, case.scale, partition_size=512,
                              work_list=i32(items), shared_prefix=(i32(mem), pp))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    seqs = sorted(set(np.random.default_rng(2).choice(B, 6, replace=False).tolist())
                  | {int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens))})
    ref = _sampled_reference(case, q, k, v, seqs)
    for r, s in enumerate(seqs):
        assert max_err(got[s], ref[r]) <= GATE["bf16"], "seq %d" % s


def test_shared_prefix_members_outside_the_batch_are_skipped():
    """A member index past the batch reads and writes nothing; the real members still get
    their shared partitions."""
    members = list(range(6))
    case = _share_case("skip", 52, [900] * 6 + [40], 32, 8, 16, "bf16", 512, members)
    got, plain, mem, pp = _run_shared(case, 512, members_override=members + [7, 1000])
    assert pp == 1
    assert max_err(got, oracle(case)) <= GATE["bf16"]


# --------------------------------------------------------------------------------------------
# the cache write of the new tokens fused into the decode pass
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,hq,hkv,d,bs,part,grid", [
    ("bf16", 32, 8, 128, 16, 512, "list"),
    ("bf16", 64, 8, 128, 16, 512, "list"),     # G 8: matrix-core score product
    ("f16", 16, 16, 128, 32, 1024, "full"),
    ("f32", 8, 4, 64, 8, 32, "list"),
    ("bf16", 8, 2, 256, 64, 256, "full"),
])
def test_append_decode_is_cache_write_then_decode(dtype, hq, hkv, d, bs, part, grid):
    """The fused pass stores each sequence's newest token where the table puts it and gives
    bitwise the output of reshape_and_cache followed by decode. The token's slot holds NaN
    beforehand, so reading it from the cache instead of from k_new would show."""
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(60)
    lens = [0, 1, 2, bs, bs + 1, 3 * bs, 700, 1025, 2048, 77]
    case = gen.make_case("app", rng, lens, hq, hkv, d, bs, dtype, width=2048 // bs + 2)
    B = len(lens)
    W = case.block_tables.shape[1]
    k_new, v_new = gen.normal(rng, (B, hkv, d), dtype), gen.normal(rng, (B, hkv, d), dtype)
    slots = np.array([-1 if L == 0 else
                      int(case.block_tables[b, (L - 1) // bs]) * bs + (L - 1) % bs
                      for b, L in enumerate(lens)], np.int32)
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    for b, sl in enumerate(slots):
        if sl >= 0:
            kc[sl // bs, :, sl % bs, :] = gen.nan_value(dtype)
            vc[sl // bs, :, sl % bs, :] = gen.nan_value(dtype)
    q = to_dev(case.q, dtype)
    tables, lns = i32(case.block_tables), i32(case.seq_lens)
    work = i32(pk.decode_work_list(case.seq_lens, W, bs, part)) if grid == "list" else None
    # unfused
    k1, v1 = to_dev(kc, dtype), to_dev(vc, dtype)
    pk.reshape_and_cache(to_dev(k_new, dtype), to_dev(v_new, dtype), k1, v1, i32(slots))
    o1 = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode(o1, q, k1, v1, tables, lns, case.scale, partition_size=part,
                              work_list=work)
    # fused
    k2, v2 = to_dev(kc, dtype), to_dev(vc, dtype)
    o2 = torch.full_like(o1, float("nan"))
    pk.paged_attention_decode_append(o2, q, to_dev(k_new, dtype), to_dev(v_new, dtype), k2, v2,
                                     tables, lns, case.scale, partition_size=part, work_list=work)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.uint8), k2.view(torch.uint8))
    assert torch.equal(v1.view(torch.uint8), v2.view(torch.uint8))
    assert torch.equal(o1, o2)
    # and both are the attention over the written caches
    ref = gen.PagedDecodeCase("app", dtype, hq, hkv, d, bs, case.num_blocks, case.seq_lens,
                              case.block_tables, case.scale, q=case.q,
                              k_cache=to_host(k2, dtype), v_cache=to_host(v2, dtype))
    assert max_err(o2.cpu().numpy().astype(np.float64), oracle(ref)) <= GATE[dtype]


def test_append_decode_skips_an_invalid_last_block():
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(61)
    case = gen.make_case("appbad", rng, [40, 40], 4, 4, 128, 16, "bf16")
    bad = case.block_tables.copy()
    bad[1, 2] = case.num_blocks + 3                  # block of token 39 of sequence 1
    k_new = gen.normal(rng, (2, 4, 128), "bf16")
    kd, vd = to_dev(case.k_cache, "bf16"), to_dev(case.v_cache, "bf16")
    before = kd.clone()
    out = torch.empty((2, 4, 128), dtype=torch.float32, device="cuda")
    pk.paged_attention_decode_append(out, to_dev(case.q, "bf16"), to_dev(k_new, "bf16"),
                                     to_dev(k_new, "bf16"), kd, vd, i32(bad), i32(case.seq_lens),
                                     case.scale)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    changed = (kd.view(torch.int16) != before.view(torch.int16)).any(dim=(1, 2, 3))
    # only sequence 0's last block took a store
    assert changed.nonzero().flatten().tolist() == [int(case.block_tables[0, 2])]


# --------------------------------------------------------------------------------------------
# work-list launches with an initialised workspace: late workgroups take their units in list
# order from the workspace's scheduling word
# --------------------------------------------------------------------------------------------

def _sched_word(ws):
    return int(ws[:8].cpu().numpy().view(np.uint64)[0])


@pytest.mark.parametrize("shape", ["gqa_short", "mha_mixed", "packed", "append_step"])
def test_scheduled_units_are_each_taken_once_and_bitwise_static(shape):
    """Units handed out by the scheduling word: every (row, KV head) unit of the list is taken
    by exactly one workgroup (read from the per-workgroup timeline, which records the unit),
    some workgroups took a unit other than their own index (the dynamic path ran), the output
    is bitwise that of the same launch over a workspace that was never initialised (static
    units), three calls in a row give the same bits, and each call leaves the word initialised
    with its count back at 0."""
    import paged_kv_cache_402_amd as pk
    from paged_kv_cache_402_amd._lib import lib as plib
    rng = np.random.default_rng(7300)
    if shape == "gqa_short":
        lens = [int(x) for x in rng.integers(1, 700, size=700)]
        case = gen.make_case("sch1", rng, lens, 32, 8, 128, 16, "bf16", values=False)
        part, pack = 256, 0
    elif shape == "mha_mixed":
        lens = [int(x) for x in rng.integers(1, 1500, size=90)]
        case = gen.make_case("sch2", rng, lens, 40, 40, 128, 32, "f16", values=False)
        part, pack = 512, 0
    elif shape == "packed":
        lens = [int(x) for x in rng.integers(1, 300, size=900)]
        case = gen.make_case("sch3", rng, lens, 16, 8, 128, 16, "bf16", values=False)
        part, pack = 256, 32
    else:
        lens = [int(x) for x in rng.integers(2, 900, size=400)]
        case = gen.make_case("sch4", rng, lens, 32, 8, 64, 16, "bf16", values=False)
        part, pack = 256, 0
    dt = case.dtype
    B, Hq, D, Hkv = len(lens), case.num_q_heads, case.head_dim, case.num_kv_heads
    W, bs = case.block_tables.shape[1], case.block_size
    shape4 = (case.num_blocks, Hkv, bs, D)
    k = gen.device_normal(shape4, dt, 7301, "cuda")
    v = gen.device_normal(shape4, dt, 7302, "cuda")
    q = gen.device_normal((B, Hq, D), dt, 7303, "cuda")
    tables, lns = i32(case.block_tables), i32(case.seq_lens)
    if pack:
        items, rows = pk.decode_work_list_packed(case.seq_lens, W, bs, part, pack)
    else:
        items = pk.decode_work_list(case.seq_lens, W, bs, part)
        rows = items.shape[0]
    work = i32(items)
    units = rows * Hkv
    need = pk.decode_workspace_bytes(B, Hq, W, bs, D, part)
    assert need > 0

    def run(ws, timeline=None):
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        if timeline is not None:
            pk.check(plib.pkv_debug_timeline(timeline.data_ptr(), units), "debug_timeline")
        try:
            if shape == "append_step":
                k_new = gen.device_normal((B, Hkv, D), dt, 7304, "cuda")
                v_new = gen.device_normal((B, Hkv, D), dt, 7305, "cuda")
                kk, vv = k.clone(), v.clone()
                pk.paged_attention_decode_append(out, q, k_new, v_new, kk, vv, tables, lns,
                                                 case.scale, partition_size=part, workspace=ws,
                                                 work_list=(work, rows) if pack else work)
            else:
                pk.paged_attention_decode(out, q, k, v, tables, lns, case.scale,
                                          partition_size=part, workspace=ws,
                                          work_list=(work, rows) if pack else work)
            torch.cuda.synchronize()
        finally:
            pk.check(plib.pkv_debug_timeline(None, 0), "debug_timeline")
        return out

    ws_static = torch.zeros(need, dtype=torch.uint8, device="cuda")     # never initialised
    want = run(ws_static)
    # each late workgroup's add found no cookie and kept its static unit: the count grew, the
    # high half stayed without the cookie
    assert _sched_word(ws_static) >> 32 == 0 and _sched_word(ws_static) > 0
    ws = pk.decode_workspace_init(torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    cookie = _sched_word(ws)
    assert cookie >> 32 != 0 and cookie & 0xFFFFFFFF == 0
    tl = torch.zeros(8 * units, dtype=torch.int32, device="cuda")
    for rep in range(3):
        tl.zero_()
        got = run(ws, tl)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), rep
        assert _sched_word(ws) == cookie, rep
        rec = tl.cpu().numpy().view(np.uint32).reshape(-1, 8)
        # every workgroup of these lists has work (and the first lane of a packed row holds a
        # real item), so every one recorded its unit: each unit exactly once
        assert (rec[:, 1] != 0).all(), rep
        taken = np.sort(rec[:, 4])
        assert np.array_equal(taken, np.arange(units)), rep
        assert (rec[:, 4] != np.arange(units)).any()        # the scheduling word was used
    assert np.isfinite(want.cpu().numpy()).all()


@pytest.mark.parametrize("kind", ["plain", "copy_on_write", "fork_groups", "matrix_core_g8",
                                  "short"])
def test_ticketed_items_match_the_launch(kind):
    """pkv_decode_ticketed_items against the launch itself. Over a workspace that was never
    initialised every late workgroup still adds one to the scheduling word (and keeps its
    static unit), so after one launch the word holds how many units were ticketed; the query,
    in items, is that count over the KV heads rounded up. A list of no more units than fit on
    the device at once tickets nothing: the query says 0 and the word stays 0."""
    import paged_kv_cache_402_amd as pk
    rng = np.random.default_rng(7400)
    Hkv, D, bs, dt = 8, 128, 16, "bf16"
    G = 8 if kind == "matrix_core_g8" else 4
    nseq = 40 if kind == "short" else 700
    lens = [int(x) for x in rng.integers(2, 700, size=nseq)]
    case = gen.make_case("tix", rng, lens, G * Hkv, Hkv, D, bs, dt, values=False)
    B, Hq, W = nseq, G * Hkv, case.block_tables.shape[1]
    part = 512 if kind == "matrix_core_g8" else 256
    shape4 = (case.num_blocks, Hkv, bs, D)
    k = gen.device_normal(shape4, dt, 7401, "cuda")
    v = gen.device_normal(shape4, dt, 7402, "cuda")
    q = gen.device_normal((B, Hq, D), dt, 7403, "cuda")
    k_new = gen.device_normal((B, Hkv, D), dt, 7404, "cuda")
    v_new = gen.device_normal((B, Hkv, D), dt, 7405, "cuda")
    tables, lns = i32(case.block_tables), i32(case.seq_lens)
    items = pk.decode_work_list(case.seq_lens, W, bs, part)
    work = i32(items)
    need = pk.decode_workspace_bytes(B, Hq, W, bs, D, part)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")        # never initialised
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    cow = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lkind, gsize = "plain", 1
    if kind == "copy_on_write":
        lkind = "copy_on_write"
        pk.paged_attention_partitions_step(out, q, k_new, v_new, cow, k, v, tables, lns,
                                           case.scale, partition_size=part, workspace=ws,
                                           work_list=work)
    elif kind == "fork_groups":
        lkind, gsize = "fork_groups", 1
        groups = torch.arange(B, dtype=torch.int32, device="cuda").view(B, 1)
        pk.paged_attention_partitions_step_groups(out, q, k_new, v_new, cow, k, v, tables, lns,
                                                  case.scale, groups, work,
                                                  partition_size=part, workspace=ws)
    else:
        pk.paged_attention_partitions(out, q, k, v, tables, lns, case.scale,
                                      partition_size=part, workspace=ws, work_list=work)
    torch.cuda.synchronize()
    count = _sched_word(ws) & 0xFFFFFFFF
    assert _sched_word(ws) >> 32 == 0
    got = pk.decode_ticketed_items(torch.bfloat16, D, Hq, Hkv, bs, part, items.shape[0], lkind,
                                   gsize)
    if kind == "short":
        assert items.shape[0] * Hkv < 1024 and count == 0 and got == 0
    else:
        assert count > 0
        assert got == -(-count // Hkv), (count, got)


def test_private_tail_list_is_bitwise_the_default_list():
    """The GQA 8B batch-256 workload with a 512-token shared prefix, at its 2048-token
    partitions, as the benchmark launches it (initialised workspace, late units by ticket):
    the reordered list moves the 12 partition-0 items (which read the prefix) out of the
    ticketed tail, and its outputs are bitwise those of the default list."""
    import paged_kv_cache_402_amd as pk
    case = gen.llama3_8b_gqa_prefix_case(values=False)
    q, k, v = _device_values(case, 4020)
    B, Hq, D = q.shape
    W, bs, Hkv, dt = case.block_tables.shape[1], case.block_size, case.num_kv_heads, case.dtype
    part = pk.default_partition(B, Hq, Hkv, D, bs, W)
    assert part == 2048
    items = pk.decode_work_list(case.seq_lens, W, bs, part)
    tail = pk.decode_ticketed_items(torch.bfloat16, D, Hq, Hkv, bs, part, items.shape[0])
    assert tail > 0
    moved_items, moved = pk.decode_work_list_private_tail(items, case.block_tables,
                                                          case.seq_lens, bs, case.num_blocks,
                                                          part, tail)
    assert moved > 0 and ((moved_items[-tail:] & 0xFFFF) >= 1).all()
    tables, lns = i32(case.block_tables), i32(case.seq_lens)
    need = pk.decode_workspace_bytes(B, Hq, W, bs, D, part)
    outs = []
    for lst in (items, moved_items):
        ws = pk.decode_workspace_init(torch.empty(need, dtype=torch.uint8, device="cuda"))
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        pk.paged_attention_partitions(out, q, k, v, tables, lns, case.scale, partition_size=part,
                                      workspace=ws, work_list=i32(lst))
        pk.paged_attention_reduce(out, lns, bs, W, ws, partition_size=part)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).clone())
    assert torch.equal(outs[0], outs[1])
    assert np.isfinite(outs[0].view(torch.bfloat16).float().cpu().numpy()).all()
