"""Python handle on the C++ host block manager of libpagedkv.so (marshalling only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理"

The manager owns a fixed pool of blocks, one block table per sequence and a refcount per
block (P1 §4.1-§4.3; P2 §3.1; P3 §2.2.2-§2.2.3); fork and prefix sharing make tables share
blocks and a write into a shared block asks for a copy first (P1 §6; P2 §2.2).
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import lib, check, PKV_ENOBLOCKS, PagedKVError

STAT_KEYS = ("used", "free", "shared", "cow_copies", "alloc_failures", "num_seqs",
             "prefix_hits", "prefix_lookups")
PREFIX_KEYS = ("cached_blocks", "cached_unheld", "hits", "lookups")


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        h = lib.pkv_bm_create(num_blocks, block_size,
                              _p(order, ctypes.c_int32) if order is not None else None)
        if not h:
            check(-1, "pkv_bm_create")
        self._h = ctypes.c_void_p(h)
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None):
            lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # -- raw status-returning calls (negative codes are returned, not raised) -------------
    def add_seq_status(self, seq: int, num_tokens: int) -> int:
        return lib.pkv_bm_add_seq(self._h, seq, num_tokens)

    def fork_status(self, parent: int, child: int) -> int:
        return lib.pkv_bm_fork(self._h, parent, child)

    def share_prefix_status(self, src: int, dst: int, num_blocks: int) -> int:
        return lib.pkv_bm_share_prefix(self._h, src, dst, num_blocks)

    def extend_status(self, seq: int, num_tokens: int):
        """(status, cow_src, cow_dst) of appending num_tokens tokens at once."""
        cs, cd = ctypes.c_int32(-1), ctypes.c_int32(-1)
        st = lib.pkv_bm_extend(self._h, seq, num_tokens, ctypes.byref(cs), ctypes.byref(cd))
        if st < 0:
            return st, -1, -1
        return st, cs.value, cd.value

    def free_seq_status(self, seq: int) -> int:
        return lib.pkv_bm_free_seq(self._h, seq)

    def append_slot_status(self, seq: int):
        """(status, slot, cow_src, cow_dst); status 0 in place / fresh block, 1 copy first."""
        slot, cs, cd = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
        st = lib.pkv_bm_append_slot(self._h, seq, ctypes.byref(slot), ctypes.byref(cs),
                                    ctypes.byref(cd))
        if st < 0:
            return st, -1, -1, -1
        return st, slot.value, cs.value, cd.value

    # -- raising conveniences --------------------------------------------------------------
    def add_seq(self, seq: int, num_tokens: int):
        check(self.add_seq_status(seq, num_tokens), "add_seq")

    def fork(self, parent: int, child: int):
        check(self.fork_status(parent, child), "fork")

    def share_prefix(self, src: int, dst: int, num_blocks: int):
        check(self.share_prefix_status(src, dst, num_blocks), "share_prefix")

    def free_seq(self, seq: int):
        check(self.free_seq_status(seq), "free_seq")

    def extend(self, seq: int, num_tokens: int):
        """Appends num_tokens tokens; returns the (src, dst) copy needed first, or None."""
        st, cs, cd = self.extend_status(seq, num_tokens)
        check(st, "extend")
        return (cs, cd) if st == 1 else None

    def append_slot(self, seq: int):
        st, slot, cs, cd = self.append_slot_status(seq)
        check(st, "append_slot")
        return slot, (cs, cd) if st == 1 else None

    def append_slots(self, seqs):
        """One token for each listed sequence, atomically. Returns (slots int32 [n],
        cow_pairs int32 [k][2])."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        slots = np.empty(n, dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        ncow = ctypes.c_int(0)
        check(lib.pkv_bm_append_slots(self._h, _p(s, ctypes.c_int64), n, _p(slots, ctypes.c_int32),
                                      _p(pairs, ctypes.c_int32), ctypes.byref(ncow)),
              "append_slots")
        return slots, pairs[:ncow.value].copy()

    def append_step(self, seqs):
        """append_slots plus, per listed sequence, the block its last block was copied from
        (-1 if none): the cow_src argument of paged_attention_decode_step. Returns (slots,
        cow_pairs, cow_src int32 [n])."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        cow_src = np.empty(max(n, 1), dtype=np.int32)
        ncow = ctypes.c_int(0)
        check(lib.pkv_bm_append_step(self._h, _p(s, ctypes.c_int64), n, _p(slots, ctypes.c_int32),
                                     _p(pairs, ctypes.c_int32), ctypes.byref(ncow),
                                     _p(cow_src, ctypes.c_int32)), "append_step")
        return slots[:n], pairs[:ncow.value].copy(), cow_src[:n]

    def table(self, seq: int):
        """(physical block ids, length in tokens)."""
        ntok = ctypes.c_int(0)
        n = check(lib.pkv_bm_table(self._h, seq, None, 0, ctypes.byref(ntok)), "table")
        out = np.empty(max(n, 1), dtype=np.int32)
        check(lib.pkv_bm_table(self._h, seq, _p(out, ctypes.c_int32), n, None), "table")
        return out[:n].tolist(), ntok.value

    def slots(self, seq: int, start: int, count: int) -> np.ndarray:
        out = np.empty(max(count, 1), dtype=np.int32)
        check(lib.pkv_bm_slots(self._h, seq, start, count, _p(out, ctypes.c_int32)), "slots")
        return out[:count]

    def build_tables(self, seqs, width: int):
        """Padded int32 [n][width] tables (-1 past the end) and int32 [n] lengths."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        tables = np.empty((max(n, 1), width), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        check(lib.pkv_bm_build_tables(self._h, _p(s, ctypes.c_int64), n,
                                      _p(tables, ctypes.c_int32), width,
                                      _p(lens, ctypes.c_int32)), "build_tables")
        return tables[:n], lens[:n]

    def add_seq_cached_status(self, seq: int, token_ids):
        """(status, cached tokens) of adding a prompt through the prefix cache."""
        t = np.ascontiguousarray(token_ids, dtype=np.int32)
        n = ctypes.c_int(0)
        st = lib.pkv_bm_add_seq_cached(self._h, seq, _p(t, ctypes.c_int32) if t.size else None,
                                       int(t.size), ctypes.byref(n))
        return st, (n.value if st >= 0 else 0)

    def add_seq_cached(self, seq: int, token_ids) -> int:
        """Adds a prompt, reusing cached blocks of its leading full blocks (P1 §7.4; P3
        §2.2.8); returns how many leading tokens were already cached."""
        st, n = self.add_seq_cached_status(seq, token_ids)
        check(st, "add_seq_cached")
        return n

    def prefix_stats(self) -> dict:
        out = np.zeros(4, dtype=np.int64)
        check(lib.pkv_bm_prefix_stats(self._h, _p(out, ctypes.c_int64)), "prefix_stats")
        return {k: int(out[i]) for i, k in enumerate(PREFIX_KEYS)}

    def refcount(self, block: int) -> int:
        return check(lib.pkv_bm_refcount(self._h, block), "refcount")

    def stats(self) -> dict:
        out = np.zeros(8, dtype=np.int64)
        check(lib.pkv_bm_stats(self._h, _p(out, ctypes.c_int64)), "stats")
        return {k: int(out[i]) for i, k in enumerate(STAT_KEYS)}


__all__ = ["BlockManager", "PagedKVError", "PKV_ENOBLOCKS"]
