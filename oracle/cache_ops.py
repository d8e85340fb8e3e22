"""Reference cache write and block copy (oracle; test infrastructure only). Bit-exact by
construction: numpy assignment of same-dtype arrays copies bit patterns unchanged.

Cache write (P1 §4.3; P3 §2.2.2-§2.2.3): a new token's K and V go to the slot the block
manager chose; slot s names physical block s // block_size, offset s % block_size. A negative
slot means "skip this token" (a reading: the pages do not define padding).

Block copy (P1 §6.2; P2 §2.2): copy-on-write duplicates exactly the one block being written,
for every KV head, K and V alike; all copies read the pre-call state.
"""
import numpy as np


def reshape_and_cache(k_new, v_new, k_cache, v_cache, slot_mapping):
    """Returns new (k_cache, v_cache) with token t's [Hkv][d] rows stored at slot_mapping[t]."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    bs = k_cache.shape[2]
    nslots = k_cache.shape[0] * bs
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        if s >= nslots:
            raise IndexError("slot outside the pool")
        kc[s // bs, :, s % bs, :] = k_new[t]
        vc[s // bs, :, s % bs, :] = v_new[t]
    return kc, vc


def copy_blocks(k_cache, v_cache, src_dst_pairs):
    """Returns new (k_cache, v_cache) where block dst holds the pre-call contents of block src
    for each (src, dst) pair."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for src, dst in np.asarray(src_dst_pairs).reshape(-1, 2).tolist():
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
    return kc, vc
