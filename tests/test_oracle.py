"""Pins of the fp64 oracle against facts fixed outside the oracle itself (CPU only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理"

Pins used: the worked block-table example printed on P3 §2.2.3 (tests/golden), closed forms
of softmax attention, brute force at 50 significant digits with mpmath, torch's
scaled_dot_product_attention in float64 on the CPU (independent library code), and the
invariances the pages state (placement does not matter, shared blocks equal private copies).
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

from oracle import cache_ops, paged_attention as pa
from oracle.storage import to_f64
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_table_worked_example.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------
# storage decoding
# ------------------------------------------------------------------------------------------

def test_bf16_bit_patterns_decode_exactly():
    pats = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F,
                     0x3C00], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133,
            (2.0 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -7]
    got = to_f64(pats, "bf16")
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)
    assert np.isnan(to_f64(np.array([0x7FC0], dtype=np.uint16), "bf16")[0])


def test_f16_f32_decode_exactly():
    assert to_f64(np.array([0x3C00, 0xC000, 0x0001], dtype=np.uint16).view(np.float16),
                  "f16").tolist() == [1.0, -2.0, 2.0 ** -24]
    x = np.array([1.5, -2.0 ** -149, 3.4e38], dtype=np.float32)
    assert to_f64(x, "f32").tolist() == [float(v) for v in x]


def test_generator_rounds_bf16_to_nearest_even():
    # 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -9], dtype=np.float32)
    got = to_f64(gen.round_to_storage(x, "bf16"), "bf16").tolist()
    assert got == [1.0, 1.0 + 2.0 ** -6, -1.0]


# ------------------------------------------------------------------------------------------
# the worked block-table example (P3 §2.2.3)
# ------------------------------------------------------------------------------------------

def _slot_id_pool(num_blocks, bs):
    """A pool whose single element per token row is that row's slot id (exact in float32)."""
    c = np.zeros((num_blocks, 1, bs, 1), dtype=np.float32)
    for blk in range(num_blocks):
        for off in range(bs):
            c[blk, 0, off, 0] = blk * bs + off
    return c


def test_worked_example_gather_order():
    g = golden()
    bs, L = g["printed"]["block_size"], g["printed"]["seq_len"]
    table = g["printed"]["physical_blocks"] + [-1]
    pool = _slot_id_pool(16, bs)
    rows = pa.gather_tokens(pool, table, L, 0)
    assert rows.shape == (L, 1)
    assert rows[:, 0].astype(int).tolist() == g["derived_by_hand"]["slots_of_tokens_0_to_34"]
    # logical block ranges printed on the page
    for j, (lo, hi) in enumerate(g["printed"]["logical_blocks_token_ranges"]):
        phys = g["printed"]["physical_blocks"][j]
        assert rows[lo:hi + 1, 0].astype(int).tolist() == [phys * bs + t % bs
                                                          for t in range(lo, hi + 1)]
    assert pa.num_logical_blocks(L, bs) == len(g["printed"]["physical_blocks"])


def test_worked_example_cache_write_slot_147():
    g = golden()
    bs = g["printed"]["block_size"]
    kc = np.zeros((16, 2, bs, 4), dtype=np.float32)
    vc = np.zeros_like(kc)
    k_new = np.arange(8, dtype=np.float32).reshape(1, 2, 4) + 1
    v_new = -k_new
    slot = g["derived_by_hand"]["slot_of_token_35"]
    k2, v2 = cache_ops.reshape_and_cache(k_new, v_new, kc, vc, [slot])
    assert (k2[9, :, 3, :] == k_new[0]).all() and (v2[9, :, 3, :] == v_new[0]).all()
    changed = np.argwhere((k2 != kc).any(axis=(1, 3)))
    assert changed.tolist() == [[9, 3]]
    # the token now reads back as logical position 35 of the table [7, 3, 9]
    rows = pa.gather_tokens(k2, [7, 3, 9], 36, 1)
    assert (rows[35] == k_new[0, 1]).all()


def test_cache_write_skips_negative_slots_and_rejects_out_of_pool():
    kc = np.zeros((2, 1, 4, 2), dtype=np.float32)
    k2, _ = cache_ops.reshape_and_cache(np.ones((2, 1, 2), np.float32),
                                        np.ones((2, 1, 2), np.float32), kc, kc, [-1, 5])
    assert k2[1, 0, 1].tolist() == [1.0, 1.0] and k2.sum() == 2.0
    with pytest.raises(IndexError):
        cache_ops.reshape_and_cache(np.ones((1, 1, 2), np.float32),
                                    np.ones((1, 1, 2), np.float32), kc, kc, [8])


def test_copy_blocks_reads_pre_call_state_and_touches_only_dst():
    rng = np.random.default_rng(1)
    kc = rng.standard_normal((6, 2, 4, 8)).astype(np.float32)
    vc = rng.standard_normal((6, 2, 4, 8)).astype(np.float32)
    k2, v2 = cache_ops.copy_blocks(kc, vc, [[1, 4], [2, 5]])
    assert (k2[4] == kc[1]).all() and (v2[5] == vc[2]).all()
    for blk in (0, 1, 2, 3):
        assert (k2[blk] == kc[blk]).all() and (v2[blk] == vc[blk]).all()


def test_gather_rejects_entries_outside_pool():
    pool = np.zeros((4, 1, 4, 1), np.float32)
    with pytest.raises(IndexError):
        pa.gather_tokens(pool, [1, 4], 6, 0)
    with pytest.raises(IndexError):
        pa.gather_tokens(pool, [-1], 1, 0)


# ------------------------------------------------------------------------------------------
# attention math: brute force, library routine, closed forms
# ------------------------------------------------------------------------------------------

def _brute_force_mp(qf, kcf, vcf, table, L, scale, group):
    """Pure-Python loops at 50 significant digits; walks the table token by token."""
    mpmath.mp.dps = 50
    Hq, d = qf.shape
    bs = kcf.shape[2]
    out = np.zeros((Hq, d))
    for h in range(Hq):
        kv = h // group
        scores = []
        for t in range(L):
            blk, off = table[t // bs], t % bs
            s = mpmath.mpf(0)
            for e in range(d):
                s += mpmath.mpf(float(qf[h, e])) * mpmath.mpf(float(kcf[blk, kv, off, e]))
            scores.append(mpmath.mpf(scale) * s)
        m = max(scores)
        w = [mpmath.exp(s - m) for s in scores]
        z = sum(w)
        for e in range(d):
            acc = mpmath.mpf(0)
            for t in range(L):
                blk, off = table[t // bs], t % bs
                acc += w[t] * mpmath.mpf(float(vcf[blk, kv, off, e]))
            out[h, e] = float(acc / z)
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_brute_force_50_digits(dtype):
    rng = np.random.default_rng(7)
    lens = [1, 3, 4, 5, 9]
    case = gen.make_case("bf", rng, lens, 4, 2, 5, 4, dtype, scale=0.7)
    out = pa.decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.seq_lens, case.scale, dtype)
    qf = to_f64(case.q, dtype)
    kcf, vcf = to_f64(case.k_cache, dtype), to_f64(case.v_cache, dtype)
    for b, L in enumerate(lens):
        ref = _brute_force_mp(qf[b], kcf, vcf, case.block_tables[b].tolist(), L,
                              float(np.float32(0.7)), 2)
        assert np.max(np.abs(out[b] - ref)) < 1e-13


def _scatter(keys, bs, phys_ids, num_blocks):
    """Test-side placement of contiguous [L][Hkv][d] rows into blocks phys_ids (no oracle code)."""
    L, Hkv, d = keys.shape
    pool = np.full((num_blocks, Hkv, bs, d), np.nan, dtype=keys.dtype)
    for t in range(L):
        pool[phys_ids[t // bs], :, t % bs, :] = keys[t]
    return pool


def test_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    Hq, Hkv, d, bs = 8, 2, 32, 16
    for L in (1, 16, 17, 100):
        keys = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        vals = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        q = rng.standard_normal((1, Hq, d)).astype(np.float32)
        nb = -(-L // bs)
        ids = rng.permutation(3 * nb)[:nb]
        kc, vc = _scatter(keys, bs, ids, 3 * nb), _scatter(vals, bs, ids, 3 * nb)
        table = np.full((1, nb + 2), -1, np.int32)
        table[0, :nb] = ids
        out = pa.decode_attention(q, kc, vc, table, np.array([L]), 0.3, "f32")[0]
        tq = torch.from_numpy(q.astype(np.float64)).reshape(1, Hq, 1, d)
        tk = torch.from_numpy(keys.astype(np.float64)).permute(1, 0, 2).repeat_interleave(
            Hq // Hkv, dim=0).unsqueeze(0)
        tv = torch.from_numpy(vals.astype(np.float64)).permute(1, 0, 2).repeat_interleave(
            Hq // Hkv, dim=0).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.contiguous(), tv.contiguous(), scale=float(np.float32(0.3)))
        assert np.max(np.abs(out - ref.reshape(Hq, d).numpy())) < 1e-12


def _one_seq_case(rng, L, Hq=2, Hkv=2, d=8, bs=4, dtype="f32"):
    return gen.make_case("one", rng, [L], Hq, Hkv, d, bs, dtype)


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(3)
    c = _one_seq_case(rng, 1)
    out = pa.decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, 1.0, "f32")
    blk = c.block_tables[0, 0]
    for h in range(2):
        assert (out[0, h] == c.v_cache[blk, h, 0].astype(np.float64)).all()


def test_zero_scale_and_constant_keys_give_mean_value():
    rng = np.random.default_rng(4)
    c = _one_seq_case(rng, 23)
    vmean = [to_f64(pa.gather_tokens(c.v_cache, c.block_tables[0], 23, h), "f32").mean(0)
             for h in range(2)]
    out = pa.decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, 0.0, "f32")
    for h in range(2):
        assert np.max(np.abs(out[0, h] - vmean[h])) < 1e-15
    kconst = np.array(c.k_cache)
    for j in range(6):
        blk = c.block_tables[0, j]
        kconst[blk] = 0.5
    out2 = pa.decode_attention(c.q, kconst, c.v_cache, c.block_tables, c.seq_lens, 1.0, "f32")
    for h in range(2):
        assert np.max(np.abs(out2[0, h] - vmean[h])) < 1e-15


def test_dominant_token_selects_its_value_row():
    rng = np.random.default_rng(5)
    c = _one_seq_case(rng, 30)
    L, bs = 30, 4
    q = np.zeros_like(c.q)
    q[0, :, 0] = 1.0
    kc = np.array(c.k_cache)
    for t in range(L):
        kc[c.block_tables[0, t // bs], :, t % bs, 0] = 0.0
    hot = 17
    kc[c.block_tables[0, hot // bs], :, hot % bs, 0] = 1.0
    out = pa.decode_attention(q, kc, c.v_cache, c.block_tables, c.seq_lens, 1000.0, "f32")
    want = c.v_cache[c.block_tables[0, hot // bs], :, hot % bs].astype(np.float64)
    assert np.max(np.abs(out[0] - want)) < 1e-300 + 1e-12


def test_zero_length_sequence_gives_zero_row():
    rng = np.random.default_rng(6)
    c = gen.make_case("z", rng, [0, 5], 2, 1, 8, 4, "f32")
    out = pa.decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, 1.0, "f32")
    assert (out[0] == 0).all() and np.isfinite(out[1]).all()


def test_token_permutation_invariance():
    """Softmax attention is a function of the set of (k, v) pairs: permuting tokens together
    leaves the output unchanged up to rounding."""
    rng = np.random.default_rng(8)
    L, Hkv, d = 40, 2, 16
    keys = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    vals = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((4, d)).astype(np.float32)
    perm = rng.permutation(L)
    a = pa.contiguous_attention(q, keys, vals, 0.25, "f32")
    b = pa.contiguous_attention(q, keys[perm], vals[perm], 0.25, "f32")
    assert np.max(np.abs(a - b)) < 1e-14


# ------------------------------------------------------------------------------------------
# invariances the pages state
# ------------------------------------------------------------------------------------------

def test_paged_equals_contiguous_for_any_block_permutation():
    """P1 §4.2: the sequence is logically contiguous whatever physical blocks hold it. The
    oracle's result must be bit-identical across placements and equal the contiguous form."""
    rng = np.random.default_rng(9)
    L, Hq, Hkv, d, bs = 35, 4, 2, 16, 16
    keys = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    vals = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    ref = pa.contiguous_attention(q[0], keys, vals, 0.125, "f32")
    outs = []
    for trial in range(3):
        ids = rng.permutation(32)[:3]
        if trial == 0:
            ids = np.array([7, 3, 9])
        kc, vc = _scatter(keys, bs, ids, 32), _scatter(vals, bs, ids, 32)
        table = np.full((1, 4), -1, np.int32)
        table[0, :3] = ids
        outs.append(pa.decode_attention(q, kc, vc, table, np.array([L]), 0.125, "f32")[0])
    for o in outs:
        assert np.array_equal(o, outs[0])
    assert np.array_equal(outs[0], ref)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(10)
    c = gen.make_case("g", rng, [13, 40], 4, 2, 8, 4, "f32")
    kc_rep = np.repeat(c.k_cache, 2, axis=1)
    vc_rep = np.repeat(c.v_cache, 2, axis=1)
    a = pa.decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, 0.5, "f32")
    b = pa.decode_attention(c.q, kc_rep, vc_rep, c.block_tables, c.seq_lens, 0.5, "f32")
    assert np.array_equal(a, b)


def test_shared_prefix_blocks_equal_private_copies():
    """P3 §2.2.3 (key point) and P1 §6.1: tables of several sequences may point at one set of
    prefix blocks; the KV is stored once and each sequence sees the same result as with a
    private copy."""
    rng = np.random.default_rng(12)
    bs, Hkv, d = 8, 2, 16
    nb_pool = 40
    kc = rng.standard_normal((nb_pool, Hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb_pool, Hkv, bs, d)).astype(np.float32)
    prefix = [5, 17, 2]
    shared = np.array([prefix + [30, 31], prefix + [33, -1]], np.int32)
    kc2, vc2 = np.array(kc), np.array(vc)
    for src, dst in zip(prefix, [20, 21, 22]):   # a private copy of the prefix for seq 1
        kc2[dst], vc2[dst] = kc[src], vc[src]
    private = np.array([prefix + [30, 31], [20, 21, 22, 33, -1]], np.int32)
    lens = np.array([38, 30])
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    a = pa.decode_attention(q, kc, vc, shared, lens, 0.25, "f32")
    b = pa.decode_attention(q, kc2, vc2, private, lens, 0.25, "f32")
    assert np.array_equal(a, b)
    # equal queries truncated to the prefix see identical outputs
    q2 = np.repeat(q[:1], 2, axis=0)
    c = pa.decode_attention(q2, kc, vc, shared, np.array([24, 24]), 0.25, "f32")
    assert np.array_equal(c[0], c[1])


def test_unused_slots_are_never_read():
    """Slots past seq_len and blocks past the table's used length hold NaN in the generated
    pools; any read of them would turn the output into NaN."""
    case = gen.tiny_case()
    out = pa.decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.seq_lens, case.scale, "f32")
    assert np.isfinite(out).all()


# ------------------------------------------------------------------------------------------
# planted mistakes: the pins above must catch plausible oracle bugs (CPU only)
# ------------------------------------------------------------------------------------------

def test_pins_catch_planted_mistakes(monkeypatch):
    g = golden()
    pool = _slot_id_pool(16, 16)
    real = pa.gather_tokens

    def reversed_table(cache, table_row, seq_len, kv_head):
        nb = pa.num_logical_blocks(seq_len, cache.shape[2])
        return real(cache, list(table_row[:nb])[::-1], seq_len, kv_head)

    rows = reversed_table(pool, [7, 3, 9], 35, 0)
    assert rows[:, 0].astype(int).tolist() != g["derived_by_hand"]["slots_of_tokens_0_to_34"]

    # a wrong head map (h % Hkv instead of h // group) breaks GQA == repeated MHA
    rng = np.random.default_rng(10)
    c = gen.make_case("g", rng, [13, 40], 4, 2, 8, 4, "f32")

    def wrong_map(q, k_cache, v_cache, tables, lens, scale, dtype):
        qf = to_f64(q, dtype)
        out = np.zeros(qf.shape)
        for b in range(qf.shape[0]):
            for h in range(qf.shape[1]):
                kv = h % k_cache.shape[1]
                kk = to_f64(pa.gather_tokens(k_cache, tables[b], int(lens[b]), kv), dtype)
                vv = to_f64(pa.gather_tokens(v_cache, tables[b], int(lens[b]), kv), dtype)
                out[b, h] = pa.attend_one(qf[b, h], kk, vv, scale)
        return out

    a = wrong_map(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, 0.5, "f32")
    b = wrong_map(c.q, np.repeat(c.k_cache, 2, 1), np.repeat(c.v_cache, 2, 1), c.block_tables,
                  c.seq_lens, 0.5, "f32")
    assert not np.array_equal(a, b)

    # dropping the max subtraction's partner (normalising by the wrong sum) breaks brute force
    def wrong_attend(q, keys, values, scale):
        s = scale * (keys @ q)
        p = np.exp(s - s.max())
        return (p @ values) / len(p)

    monkeypatch.setattr(pa, "attend_one", wrong_attend)
    rng = np.random.default_rng(7)
    case = gen.make_case("bf", rng, [5], 2, 1, 4, 4, "f32", scale=0.7)
    out = pa.decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.seq_lens, case.scale, "f32")
    ref = _brute_force_mp(to_f64(case.q, "f32")[0], to_f64(case.k_cache, "f32"),
                          to_f64(case.v_cache, "f32"), case.block_tables[0].tolist(), 5,
                          float(np.float32(0.7)), 2)
    assert np.max(np.abs(out[0] - ref)) > 1e-6


def test_pins_catch_more_planted_mistakes(monkeypatch):
    """A dropped scale and an off-by-one gather, planted in the oracle on the CPU, must each
    fail a pin: the 50-digit brute force and the worked block-table example."""
    rng = np.random.default_rng(11)
    case = gen.make_case("bf2", rng, [6], 2, 1, 4, 4, "f32", scale=0.7)
    ref = _brute_force_mp(to_f64(case.q, "f32")[0], to_f64(case.k_cache, "f32"),
                          to_f64(case.v_cache, "f32"), case.block_tables[0].tolist(), 6,
                          float(np.float32(0.7)), 2)
    real_attend = pa.attend_one

    def no_scale(q, keys, values, scale):
        return real_attend(q, keys, values, 1.0)

    monkeypatch.setattr(pa, "attend_one", no_scale)
    out = pa.decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                              case.seq_lens, case.scale, "f32")
    assert np.max(np.abs(out[0] - ref)) > 1e-6
    monkeypatch.setattr(pa, "attend_one", real_attend)

    g = golden()
    pool = _slot_id_pool(16, 16)
    real_gather = pa.gather_tokens

    def shifted(cache, table_row, seq_len, kv_head):
        # off by one token: row t read from position t + 1
        rows = real_gather(cache, table_row, seq_len + 1, kv_head)
        return rows[1:]

    rows = shifted(pool, [7, 3, 9], 35, 0)
    assert rows[:, 0].astype(int).tolist() != g["derived_by_hand"]["slots_of_tokens_0_to_34"]
