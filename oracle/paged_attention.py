"""fp64 oracle of decode attention over a paged KV cache (test infrastructure only).

What the method computes (P1 §4.2; P3 §2.2.3): each sequence's cached keys and values sit in
fixed-size physical blocks; the sequence's block table maps logical block j to a physical
block, and attention sees the tokens as one logically contiguous sequence. Growth appends a
block without moving data, so the result is exactly ordinary attention over the contiguous
sequence. This module therefore (1) gathers the sequence's tokens through its table into a
contiguous array and (2) applies textbook single-query softmax attention in float64.

Readings where the pages are silent (each listed in the design doc):
  - attention formula: out = sum_t softmax_t(scale * q.k_t) v_t over all L cached tokens of the
    sequence (decode attends to every cached token; no mask, bias, window or cap);
  - grouped heads: query head h reads KV head h // (Hq / Hkv);
  - scale: caller-given, used as the binary32 value the kernel receives;
  - a sequence of length 0 yields a zero output row;
  - table entries past ceil(L / block_size) and slots past L in the last block are never read.
"""
import numpy as np

from .storage import to_f64, scale_as_used


def num_logical_blocks(seq_len: int, block_size: int) -> int:
    """Blocks a sequence of `seq_len` tokens occupies: token t lives in logical block
    t // block_size at offset t % block_size (P3 §2.2.3: 35 tokens of block size 16 span
    logical blocks 0, 1 and 2)."""
    return (int(seq_len) + int(block_size) - 1) // int(block_size)


def gather_tokens(cache: np.ndarray, table_row, seq_len: int, kv_head: int) -> np.ndarray:
    """Logically contiguous [seq_len][d] rows of one KV head, read through the block table.

    cache: [num_blocks][Hkv][block_size][d] (any storage dtype; returned unconverted).
    Row t comes from physical block table_row[t // bs], offset t % bs (P1 §4.2; P3 §2.2.3).
    """
    num_blocks, _, bs, d = cache.shape
    nb = num_logical_blocks(seq_len, bs)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    if nb and not ((phys >= 0).all() and (phys < num_blocks).all()):
        raise IndexError("block table entry outside the pool")
    tiles = cache[phys, kv_head]                  # [nb][bs][d], logical order
    return tiles.reshape(nb * bs, d)[:seq_len]


def attend_one(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Textbook softmax attention of one float64 query row over float64 key/value rows."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    s = scale * (keys @ q)
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


def decode_attention(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype,
                     seqs=None) -> np.ndarray:
    """out[b][h] for every (or the listed) sequence b and query head h, in float64.

    q: storage [B][Hq][d]; k_cache, v_cache: storage [NB][Hkv][bs][d];
    block_tables: int [B][W]; seq_lens: int [B]; dtype in {"f32", "f16", "bf16"}.
    Returns [B][Hq][d] float64 (rows of sequences not listed in `seqs` stay zero).
    """
    qf = to_f64(q, dtype)
    B, Hq, d = qf.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    sc = scale_as_used(scale)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        for kv in range(Hkv):
            keys = to_f64(gather_tokens(k_cache, block_tables[b], L, kv), dtype)
            vals = to_f64(gather_tokens(v_cache, block_tables[b], L, kv), dtype)
            for h in range(kv * group, (kv + 1) * group):
                out[b, h] = attend_one(qf[b, h], keys, vals, sc)
    return out


def contiguous_attention(q, keys, values, scale, dtype) -> np.ndarray:
    """The prior, unpaged formulation: q [Hq][d], keys/values [L][Hkv][d] stored contiguously.
    Used to check that paging changes nothing (P1 §4.2)."""
    qf = to_f64(q, dtype)
    kf = to_f64(keys, dtype)
    vf = to_f64(values, dtype)
    Hq = qf.shape[0]
    Hkv = kf.shape[1]
    group = Hq // Hkv
    sc = scale_as_used(scale)
    return np.stack([attend_one(qf[h], kf[:, h // group], vf[:, h // group], sc)
                     for h in range(Hq)])
