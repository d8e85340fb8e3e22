"""Reference model of the host block manager (oracle; test infrastructure only).

Follows the pages' description of paged KV memory:
  - a fixed pool of equal-size blocks; any free block serves any request (P1 §4.1);
  - one block table per sequence, logical block -> physical block (P1 §4.2; P3 §2.2.3);
  - growth on demand: a new block only when the last one is full (P1 §4.3; P3 §2.2.3);
  - release to the free pool when a sequence finishes or is preempted (P3 §2.2.2);
  - several tables may list the same physical blocks (P1 §6.1; P3 §2.2.3 key point);
  - a write into a shared block copies that one block first; the original stays as it is
    for its other users (P1 §6.2; P2 §2.2 for forked branches).

Readings where the pages are silent or garbled (listed in the design doc):
  - the pool never grows; an allocation that cannot be met fails with ENOBLOCKS, changes no
    state and counts one allocation failure (the pages' pseudo-code grows the pool instead);
  - "shared" means refcount > 1; the last holder (refcount 1) writes in place;
  - which free block is handed out is not fixed by the pages (any is correct); the model is a
    LIFO stack whose initial order is caller-given, so two implementations can be compared id
    for id; a freed sequence's blocks are pushed last-logical-block first, so its first logical
    block is the next one handed out;
  - the page's worked example says the 36th token fills block 2 of a 35-token sequence; the
    arithmetic (token t in logical block t // 16) puts that token at offset 3 of block 2 and
    opens a new block at token index 48. The model follows the arithmetic.
"""

import copy

OK = 0
EINVAL = -1
ENOBLOCKS = -3
ENOSEQ = -5


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("bad pool")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))        # stack: pop() hands out order[0] first
        self.rc = [0] * num_blocks
        self.seqs = {}                           # seq -> [blocks, num_tokens]
        self.cow_copies = 0
        self.alloc_failures = 0
        # prefix cache (P1 §7.4; P3 §2.2.8): key -> block for full prompt blocks; a key is
        # (previous block, its hand-out count, the block's tokens), so it names the exact
        # token prefix; unheld cached blocks wait in release order and are reused last
        self.cache = {}
        self.block_key = {}
        self.released = []                       # cached blocks no sequence holds, oldest first
        self.handouts = [0] * num_blocks
        self.prefix_hits = 0
        self.prefix_lookups = 0
        self.prefix_tokens = {}                  # block -> the full token prefix it ends

    # -- all-or-nothing support for multi-step operations ------------------------------------
    def snapshot(self):
        keep = self.alloc_failures
        state = copy.deepcopy({k: v for k, v in self.__dict__.items() if k != "alloc_failures"})
        return state, keep

    def restore(self, snap):
        state, _ = snap
        failures = self.alloc_failures
        self.__dict__.update(copy.deepcopy(state))
        self.alloc_failures = failures

    # -- block hand-out and release -------------------------------------------------------------
    def _available(self):
        return len(self.free) + len(self.released)

    def _take(self):
        if self.free:
            b = self.free.pop()
        else:                                    # oldest released cached block leaves the cache
            b = self.released.pop(0)
            del self.cache[self.block_key.pop(b)]
            self.prefix_tokens.pop(b, None)
        self.rc[b] = 1
        self.handouts[b] += 1
        return b

    def _hold(self, b):
        if self.rc[b] == 0 and b in self.released:
            self.released.remove(b)
        self.rc[b] += 1

    def _release(self, b):
        self.rc[b] -= 1
        if self.rc[b] == 0:
            if b in self.block_key:
                self.released.append(b)
            else:
                self.free.append(b)

    def _need(self, n):
        return (n + self.block_size - 1) // self.block_size

    def add_seq(self, seq, num_tokens):
        if seq in self.seqs or num_tokens < 0:
            return EINVAL
        need = self._need(num_tokens)
        if need > self._available():
            self.alloc_failures += 1
            return ENOBLOCKS
        blocks = [self._take() for _ in range(need)]
        self.seqs[seq] = [blocks, num_tokens]
        return OK

    def _key(self, parent, tokens):
        return (parent, self.handouts[parent] if parent >= 0 else 0, tuple(int(t) for t in tokens))

    def add_seq_cached(self, seq, token_ids):
        """Returns (status, cached tokens): leading full blocks whose exact token prefix is
        cached are reused, the rest are fresh and the fresh full blocks get registered."""
        tokens = [int(t) for t in token_ids]
        if seq in self.seqs:
            return EINVAL, 0
        bs = self.block_size
        nfull = len(tokens) // bs
        hits, parent = [], -1
        for j in range(nfull):
            b = self.cache.get(self._key(parent, tokens[j * bs:(j + 1) * bs]))
            if b is None:
                break
            hits.append(b)
            parent = b
        need = self._need(len(tokens)) - len(hits)
        unheld_hits = sum(1 for b in hits if self.rc[b] == 0)
        if need > self._available() - unheld_hits:
            self.alloc_failures += 1
            return ENOBLOCKS, 0
        for b in hits:
            self._hold(b)
        blocks = list(hits)
        for j in range(len(hits), self._need(len(tokens))):
            b = self._take()
            blocks.append(b)
            if j < nfull:
                key = self._key(parent, tokens[j * bs:(j + 1) * bs])
                self.cache[key] = b
                self.block_key[b] = key
                self.prefix_tokens[b] = tuple(tokens[:(j + 1) * bs])
                parent = b
        self.seqs[seq] = [blocks, len(tokens)]
        self.prefix_hits += len(hits)
        self.prefix_lookups += nfull
        return OK, len(hits) * bs

    def fork(self, parent, child):
        if parent not in self.seqs:
            return ENOSEQ
        if child in self.seqs:
            return EINVAL
        blocks, n = self.seqs[parent]
        for b in blocks:
            self._hold(b)
        self.seqs[child] = [list(blocks), n]
        return OK

    def share_prefix(self, src, dst, nblocks):
        if src not in self.seqs:
            return ENOSEQ
        if dst in self.seqs or nblocks < 0:
            return EINVAL
        blocks, n = self.seqs[src]
        if nblocks * self.block_size > n:
            return EINVAL
        for b in blocks[:nblocks]:
            self._hold(b)
        self.seqs[dst] = [list(blocks[:nblocks]), nblocks * self.block_size]
        return OK

    def append_slot(self, seq):
        """Returns (status, slot, cow_src, cow_dst); status 0 = written in place or into a fresh
        block, 1 = the shared last block was copied first (cow_src -> cow_dst)."""
        if seq not in self.seqs:
            return ENOSEQ, -1, -1, -1
        blocks, n = self.seqs[seq]
        off = n % self.block_size
        status, cs, cd = OK, -1, -1
        if off == 0:
            if self._available() == 0:
                self.alloc_failures += 1
                return ENOBLOCKS, -1, -1, -1
            blk = self._take()
            blocks.append(blk)
        else:
            last = blocks[-1]
            if self.rc[last] > 1:
                if self._available() == 0:
                    self.alloc_failures += 1
                    return ENOBLOCKS, -1, -1, -1
                blk = self._take()
                self.rc[last] -= 1
                blocks[-1] = blk
                self.cow_copies += 1
                status, cs, cd = 1, last, blk
            else:
                blk = last
        self.seqs[seq][1] = n + 1
        return status, blk * self.block_size + off, cs, cd

    def extend(self, seq, num_tokens):
        """num_tokens appends in a row, all or nothing. Returns (status, cow_src, cow_dst) of
        the first append (the only one that can copy)."""
        if seq not in self.seqs:
            return ENOSEQ, -1, -1
        if num_tokens < 0:
            return EINVAL, -1, -1
        snap = self.snapshot()
        first = (OK, -1, -1)
        for i in range(num_tokens):
            st, _, cs, cd = self.append_slot(seq)
            if st < 0:
                self.restore(snap)
                return st, -1, -1
            if i == 0:
                first = (st, cs, cd)
        return first

    def free_seq(self, seq):
        if seq not in self.seqs:
            return ENOSEQ
        blocks, _ = self.seqs.pop(seq)
        for b in reversed(blocks):
            self._release(b)
        return OK

    def table(self, seq):
        blocks, n = self.seqs[seq]
        return list(blocks), n

    def slots(self, seq, start, count):
        """Slot of each token position in [start, start + count)."""
        blocks, n = self.seqs[seq]
        if start < 0 or count < 0 or start + count > n:
            raise IndexError("positions outside the sequence")
        bs = self.block_size
        return [blocks[t // bs] * bs + t % bs for t in range(start, start + count)]

    def refcount(self, block):
        return self.rc[block]

    def stats(self):
        used = sum(1 for r in self.rc if r > 0)
        shared = sum(1 for r in self.rc if r > 1)
        return {"used": used, "free": self._available(), "shared": shared,
                "cow_copies": self.cow_copies, "alloc_failures": self.alloc_failures,
                "num_seqs": len(self.seqs), "prefix_hits": self.prefix_hits,
                "prefix_lookups": self.prefix_lookups}

    def prefix_stats(self):
        return {"cached_blocks": len(self.cache), "cached_unheld": len(self.released),
                "hits": self.prefix_hits, "lookups": self.prefix_lookups}
