"""Python face of the device operations: argument marshalling only.

Each function reads shapes from torch tensors, checks dtypes/devices/contiguity, and calls the
C ABI with raw device pointers on torch's current HIP stream. All computation happens in the
HIP kernels of libpagedkv.so; nothing here computes on the host or falls back to torch ops.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import lib, check

KV_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
DEFAULT_PARTITION = 512


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a device (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _i32(t: torch.Tensor, name: str):
    _dev(t, name)
    if t.dtype != torch.int32:
        raise ValueError("%s must be int32" % name)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _kv_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in KV_DTYPES:
        raise ValueError("%s must be float32, float16 or bfloat16" % name)
    return KV_DTYPES[t.dtype]


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, max_blocks_per_seq: int,
                           block_size: int, head_dim: int,
                           partition_size: int = DEFAULT_PARTITION) -> int:
    return int(lib.pkv_decode_workspace_bytes(num_seqs, num_q_heads, max_blocks_per_seq,
                                              block_size, head_dim, partition_size))


def decode_workspace_init(workspace):
    """Initialises the workspace's scheduling word (pkv_decode_workspace_init): work-list
    launches then hand the units of late-starting workgroups out in list order."""
    _dev(workspace, "workspace")
    check(lib.pkv_decode_workspace_init(workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(workspace)), "decode_workspace_init")
    return workspace


def default_partition(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      block_size: int, max_blocks_per_seq: int) -> int:
    """The partition size pkv_decode_default_partition picks for these shapes (a multiple of
    256 tokens up to 2048)."""
    return check(lib.pkv_decode_default_partition(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  block_size, max_blocks_per_seq),
                 "default_partition")


def _resolve_partition(partition_size, B, Hq, Hkv, D, bs, W, work_list, shared_prefix=None):
    if partition_size is not None:
        return partition_size
    if work_list is not None or shared_prefix is not None:
        raise ValueError("pass the partition_size the work list was built with")
    return default_partition(B, Hq, Hkv, D, bs, W)


KV_STREAM, KV_CACHED = 0, 1   # PKV_KV_STREAM, PKV_KV_CACHED


def decode_kv_policy(block_tables, seq_lens, block_size: int, num_blocks: int,
                     work_list=None, partition_size: int = 0) -> int:
    """Cache policy for the KV reads of one decode launch (pkv_decode_kv_policy) from host
    tables [B][W] and lengths [B], over the partitions of the host `work_list` (the whole
    list, packed or not, built with `partition_size`) or over every token: KV_CACHED when at
    least half of its block reads repeat a block (forked sequences, a long common prefix),
    else KV_STREAM."""
    tab = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if tab.ndim != 2 or lens.shape != (tab.shape[0],):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    wl, n = None, 0
    if work_list is not None:
        items = np.ascontiguousarray(np.asarray(work_list, dtype=np.int32).reshape(-1))
        wl, n = items.ctypes.data_as(P_i32), items.shape[0]
    return check(lib.pkv_decode_kv_policy(tab.ctypes.data_as(P_i32), lens.ctypes.data_as(P_i32),
                                          tab.shape[0], tab.shape[1], block_size, num_blocks,
                                          wl, n, int(partition_size)),
                 "decode_kv_policy")


def decode_work_list(seq_lens, max_blocks_per_seq: int, block_size: int,
                     partition_size: int = DEFAULT_PARTITION) -> np.ndarray:
    """Host work list of the per-partition pass (pkv_decode_work_list) from host lengths:
    int32 items (sequence << 16 | partition), full partitions first, then the last partial
    partitions longest first. Upload it and pass it as work_list=."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    lp = lens.ctypes.data_as(P_i32)
    n = check(lib.pkv_decode_work_list(lp, lens.shape[0], max_blocks_per_seq, block_size,
                                       partition_size, None, 0), "decode_work_list")
    items = np.empty(n, dtype=np.int32)
    check(lib.pkv_decode_work_list(lp, lens.shape[0], max_blocks_per_seq, block_size,
                                   partition_size, items.ctypes.data_as(P_i32), n),
          "decode_work_list")
    return items


LAUNCH_KINDS = {"plain": 0, "copy_on_write": 1, "fork_groups": 2}


def decode_ticketed_items(kv_dtype: torch.dtype, head_dim: int, num_q_heads: int,
                          num_kv_heads: int, block_size: int, partition_size: int,
                          list_len: int, kind: str = "plain", group_size: int = 1) -> int:
    """Items at the end of a work list of list_len items that a launch with an initialised
    workspace hands out by ticket on the current device (pkv_decode_ticketed_items). kind:
    "plain" (the _list, _append, _shared and plain calls), "copy_on_write" (the _step calls)
    or "fork_groups" (the fork-group step, with its group_size)."""
    if kv_dtype not in KV_DTYPES:
        raise ValueError("kv_dtype must be float32, float16 or bfloat16")
    if kind not in LAUNCH_KINDS:
        raise ValueError("kind must be one of %s" % ", ".join(LAUNCH_KINDS))
    return check(lib.pkv_decode_ticketed_items(KV_DTYPES[kv_dtype], head_dim, num_q_heads,
                                               num_kv_heads, block_size, partition_size,
                                               int(list_len), LAUNCH_KINDS[kind],
                                               int(group_size)),
                 "decode_ticketed_items")


def decode_work_list_private_tail(work_list, block_tables, seq_lens, block_size: int,
                                  num_blocks: int, partition_size: int, tail_items: int):
    """A host work list (pkv_decode_work_list) reordered so that its last tail_items items
    (from decode_ticketed_items) read no block another item reads, where it has private items
    to spare (pkv_decode_work_list_private_tail). Returns (list, shared items moved out of the
    tail); the input is not modified."""
    tab = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if tab.ndim != 2 or lens.shape != (tab.shape[0],):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    items = np.array(np.asarray(work_list, dtype=np.int32).reshape(-1), copy=True)
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    moved = check(lib.pkv_decode_work_list_private_tail(
        tab.ctypes.data_as(P_i32), lens.ctypes.data_as(P_i32), tab.shape[0], tab.shape[1],
        block_size, num_blocks, partition_size, int(tail_items), items.ctypes.data_as(P_i32),
        items.shape[0]), "decode_work_list_private_tail")
    return items, moved


def decode_work_list_packed(seq_lens, max_blocks_per_seq: int, block_size: int,
                            partition_size: int = DEFAULT_PARTITION, pack_tokens: int = 64):
    """Host work list with the partitions of at most pack_tokens tokens packed four to a
    workgroup (pkv_decode_work_list_packed). Returns (list int32, rows): upload the list and
    pass work_list=(tensor, rows)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    lp = lens.ctypes.data_as(P_i32)
    rows = ctypes.c_int(0)
    n = check(lib.pkv_decode_work_list_packed(lp, lens.shape[0], max_blocks_per_seq, block_size,
                                              partition_size, pack_tokens, None, 0,
                                              ctypes.byref(rows)), "decode_work_list_packed")
    items = np.empty(n, dtype=np.int32)
    check(lib.pkv_decode_work_list_packed(lp, lens.shape[0], max_blocks_per_seq, block_size,
                                          partition_size, pack_tokens,
                                          items.ctypes.data_as(P_i32), n, ctypes.byref(rows)),
          "decode_work_list_packed")
    return items, rows.value


def plan_shared_prefix(block_tables, seq_lens, block_size: int,
                       partition_size: int = DEFAULT_PARTITION, min_members: int = 2):
    """Host planner of the shared-prefix decode (pkv_decode_plan_shared_prefix) from host
    tables [B][W] and lengths [B]. Returns (members int32 [n], prefix_partitions, work list
    int32 without the members' shared partitions); n = prefix_partitions = 0 when no group of
    at least min_members sequences shares a first partition."""
    tab = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B, W = tab.shape
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    members = np.zeros(max(1, B), dtype=np.int32)
    nm, pp = ctypes.c_int(0), ctypes.c_int(0)
    args = (tab.ctypes.data_as(P_i32), lens.ctypes.data_as(P_i32), B, W, block_size,
            partition_size, min_members, members.ctypes.data_as(P_i32), ctypes.byref(nm),
            ctypes.byref(pp))
    n = check(lib.pkv_decode_plan_shared_prefix(*args, None, 0), "plan_shared_prefix")
    items = np.empty(n, dtype=np.int32)
    check(lib.pkv_decode_plan_shared_prefix(*args, items.ctypes.data_as(P_i32), n),
          "plan_shared_prefix")
    return members[:nm.value].copy(), pp.value, items


def _work(work_list):
    """A device list, or (device list, rows) for a packed list: pointer and row count."""
    if work_list is None:
        return None, 0
    rows = None
    if isinstance(work_list, tuple):
        work_list, rows = work_list
    _i32(work_list, "work_list")
    if work_list.dim() != 1:
        raise ValueError("work_list must be 1-D")
    if rows is None:
        rows = work_list.shape[0]
    elif not 0 <= int(rows) <= work_list.shape[0]:
        raise ValueError("work_list rows %d outside [0, %d]" % (rows, work_list.shape[0]))
    return work_list.data_ptr(), int(rows)


def _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens):
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    _i32(block_tables, "block_tables")
    _i32(seq_lens, "seq_lens")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected q [B][Hq][D] and caches [NB][Hkv][bs][D] of equal shape")
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    if D2 != D or out.shape != q.shape:
        raise ValueError("head_dim mismatch between q, out and the caches")
    kdt = _kv_dtype(k_cache, "k_cache")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("q, k_cache and v_cache must share a dtype")
    if out.dtype not in (k_cache.dtype, torch.float32):
        raise ValueError("out must have the cache dtype or float32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables [B][W] and seq_lens [B] expected")
    return B, Hq, D, NB, Hkv, bs, kdt, KV_DTYPES[out.dtype], block_tables.shape[1]


def _workspace(q, B, Hq, W, bs, D, partition_size, workspace):
    need = decode_workspace_bytes(B, Hq, W, bs, D, partition_size)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = decode_workspace_init(torch.empty(need, dtype=torch.uint8, device=q.device))
    _dev(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale,
                           partition_size=None, workspace=None, work_list=None,
                           shared_prefix=None, kv_policy: int = 0):
    """out[b][h] = softmax(scale * q[b][h] . K_b) V_b over the seq_lens[b] tokens that sequence
    b's block table locates in the paged caches. With work_list (device int32 from
    decode_work_list, or (device list, rows) from decode_work_list_packed) the per-partition
    pass runs over that list. With shared_prefix =
    (members device int32, prefix_partitions) and the matching work_list (both from
    plan_shared_prefix) the members' shared partitions run in the shared-prefix pass.
    partition_size None picks default_partition's (then no work list may be given).
    kv_policy: KV_STREAM (non-temporal KV reads) or KV_CACHED (default cache policy), as
    decode_kv_policy picks it for the batch; speed only, the output is the same.
    Returns `out`."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    partition_size = _resolve_partition(partition_size, B, Hq, Hkv, D, bs, W, work_list,
                                        shared_prefix)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wsp = ws.data_ptr() if ws is not None else None
    if shared_prefix is not None:
        if work_list is None:
            raise ValueError("shared_prefix needs the work list plan_shared_prefix returns")
        mem, pp = shared_prefix
        _i32(mem, "members")
        wl, wn = _work(work_list)
        check(lib.pkv_paged_attention_decode_shared(
            out.data_ptr(), odt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kdt,
            block_tables.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale),
            partition_size, mem.data_ptr(), mem.shape[0], int(pp), wl, wn, wsp, wsb, int(kv_policy), _stream(q)),
            "paged_attention_decode_shared")
    elif work_list is None:
        check(lib.pkv_paged_attention_decode(
            out.data_ptr(), odt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kdt,
            block_tables.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale),
            partition_size, wsp, wsb, int(kv_policy), _stream(q)), "paged_attention_decode")
    else:
        wl, wn = _work(work_list)
        check(lib.pkv_paged_attention_decode_list(
            out.data_ptr(), odt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kdt,
            block_tables.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale),
            partition_size, wl, wn, wsp, wsb, int(kv_policy), _stream(q)), "paged_attention_decode_list")
    return out


def paged_attention_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, scale,
                               partition_size: int = DEFAULT_PARTITION, workspace=None,
                               work_list=None, kv_policy: int = 0):
    """First pass of paged_attention_decode only (per-partition attention). Returns the
    workspace that paged_attention_reduce needs (None if no sequence spans two partitions)."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wsp = ws.data_ptr() if ws is not None else None
    if work_list is None:
        check(lib.pkv_paged_attention_partitions(
            out.data_ptr(), odt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kdt,
            block_tables.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale),
            partition_size, wsp, wsb, int(kv_policy), _stream(q)), "paged_attention_partitions")
    else:
        wl, wn = _work(work_list)
        check(lib.pkv_paged_attention_partitions_list(
            out.data_ptr(), odt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kdt,
            block_tables.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale),
            partition_size, wl, wn, wsp, wsb, int(kv_policy), _stream(q)), "paged_attention_partitions_list")
    return ws


def _append_args(k_new, v_new, k_cache, B):
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, n)
        if t.dtype != k_cache.dtype or t.shape != (B, k_cache.shape[1], k_cache.shape[3]):
            raise ValueError("%s must be [B][Hkv][D] of the cache dtype" % n)


def paged_attention_decode_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens,
                                  scale, partition_size=None, workspace=None, work_list=None,
                                  kv_policy: int = 0):
    """Stores every sequence's newest token (k_new / v_new, [B][Hkv][D], token seq_lens[b] - 1)
    into the caches at the slot its block table gives and decodes, in one pass plus the merge:
    the same caches and bitwise the same output as reshape_and_cache then
    paged_attention_decode. Returns `out`."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    partition_size = _resolve_partition(partition_size, B, Hq, Hkv, D, bs, W, work_list)
    _append_args(k_new, v_new, k_cache, B)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wl, wn = _work(work_list)
    check(lib.pkv_paged_attention_decode_append(
        out.data_ptr(), odt, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), kdt, block_tables.data_ptr(),
        seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale), partition_size, wl, wn,
        ws.data_ptr() if ws is not None else None, wsb, int(kv_policy), _stream(q)),
        "paged_attention_decode_append")
    return out


def paged_attention_partitions_append(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                      seq_lens, scale, partition_size: int = DEFAULT_PARTITION,
                                      workspace=None, work_list=None, kv_policy: int = 0):
    """First pass of paged_attention_decode_append only. Returns the workspace for
    paged_attention_reduce."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    _append_args(k_new, v_new, k_cache, B)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wl, wn = _work(work_list)
    check(lib.pkv_paged_attention_partitions_append(
        out.data_ptr(), odt, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), kdt, block_tables.data_ptr(),
        seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale), partition_size, wl, wn,
        ws.data_ptr() if ws is not None else None, wsb, int(kv_policy), _stream(q)),
        "paged_attention_partitions_append")
    return ws


def _cow_arg(cow_src, B):
    _i32(cow_src, "cow_src")
    if tuple(cow_src.shape) != (B,):
        raise ValueError("cow_src must be int32 [num_seqs]")
    return cow_src.data_ptr()


def paged_attention_decode_step(out, q, k_new, v_new, cow_src, k_cache, v_cache, block_tables,
                                seq_lens, scale, partition_size=None, workspace=None,
                                work_list=None, kv_policy: int = 0):
    """One decode step in one pass plus the merge: each sequence's copy-on-write of its last
    block (cow_src int32 [B]: the source block, or -1), the cache write of its newest token
    (k_new / v_new) and the attention; bitwise copy_blocks, then reshape_and_cache, then
    paged_attention_decode, in the output and every row a sequence holds (a copied block's rows
    past the new token are left as they were). Returns `out`."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    partition_size = _resolve_partition(partition_size, B, Hq, Hkv, D, bs, W, work_list)
    _append_args(k_new, v_new, k_cache, B)
    cs = _cow_arg(cow_src, B)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wl, wn = _work(work_list)
    check(lib.pkv_paged_attention_decode_step(
        out.data_ptr(), odt, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), cs,
        k_cache.data_ptr(), v_cache.data_ptr(), kdt, block_tables.data_ptr(),
        seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale), partition_size, wl, wn,
        ws.data_ptr() if ws is not None else None, wsb, int(kv_policy), _stream(q)),
        "paged_attention_decode_step")
    return out


def paged_attention_partitions_step(out, q, k_new, v_new, cow_src, k_cache, v_cache,
                                    block_tables, seq_lens, scale,
                                    partition_size: int = DEFAULT_PARTITION, workspace=None,
                                    work_list=None, kv_policy: int = 0):
    """First pass of paged_attention_decode_step only. Returns the workspace for
    paged_attention_reduce."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    _append_args(k_new, v_new, k_cache, B)
    cs = _cow_arg(cow_src, B)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wl, wn = _work(work_list)
    check(lib.pkv_paged_attention_partitions_step(
        out.data_ptr(), odt, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), cs,
        k_cache.data_ptr(), v_cache.data_ptr(), kdt, block_tables.data_ptr(),
        seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale), partition_size, wl, wn,
        ws.data_ptr() if ws is not None else None, wsb, int(kv_policy), _stream(q)),
        "paged_attention_partitions_step")
    return ws


def plan_fork_groups(block_tables, seq_lens, cow_src, block_size: int, num_blocks: int,
                     group_size: int):
    """Host planner of the fork-group step (pkv_decode_plan_fork_groups) from host tables
    [B][W], lengths [B] and copy sources [B] (or None). Returns (groups int32 [n][group_size],
    -1 filling short groups; group_lens int32 [n])."""
    tab = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if tab.ndim != 2 or lens.shape != (tab.shape[0],):
        raise ValueError("block_tables must be [B][W] and seq_lens [B]")
    B, W = tab.shape
    P_i32 = ctypes.POINTER(ctypes.c_int32)
    cs = None
    if cow_src is not None:
        cs = np.ascontiguousarray(np.asarray(cow_src, dtype=np.int32))
        if cs.shape != (B,):
            raise ValueError("cow_src must be [B]")
    args = (tab.ctypes.data_as(P_i32), lens.ctypes.data_as(P_i32),
            cs.ctypes.data_as(P_i32) if cs is not None else None, B, W, block_size,
            num_blocks, group_size)
    n = check(lib.pkv_decode_plan_fork_groups(*args, None, None, 0), "decode_plan_fork_groups")
    groups = np.empty((max(n, 1), group_size), dtype=np.int32)
    glens = np.empty(max(n, 1), dtype=np.int32)
    check(lib.pkv_decode_plan_fork_groups(*args, groups.ctypes.data_as(P_i32),
                                          glens.ctypes.data_as(P_i32), n),
          "decode_plan_fork_groups")
    return groups[:n], glens[:n]


def _groups_arg(groups):
    _i32(groups, "groups")
    if groups.dim() != 2:
        raise ValueError("groups must be int32 [num_groups][group_size]")
    return groups.data_ptr(), groups.shape[0], groups.shape[1]


def paged_attention_decode_step_groups(out, q, k_new, v_new, cow_src, k_cache, v_cache,
                                       block_tables, seq_lens, scale, groups, work_list,
                                       partition_size=None, workspace=None, kv_policy: int = 0):
    """paged_attention_decode_step over fork groups (groups: device int32
    [num_groups][group_size] from plan_fork_groups; work_list: a list over the groups'
    lengths, plain or (list, rows) packed; cow_src: int32 [B] or None). Returns `out`."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    partition_size = _resolve_partition(partition_size, B, Hq, Hkv, D, bs, W, work_list)
    _append_args(k_new, v_new, k_cache, B)
    cs = _cow_arg(cow_src, B) if cow_src is not None else None
    gp, ng, gs = _groups_arg(groups)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wl, wn = _work(work_list)
    check(lib.pkv_paged_attention_decode_step_groups(
        out.data_ptr(), odt, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), cs,
        k_cache.data_ptr(), v_cache.data_ptr(), kdt, block_tables.data_ptr(),
        seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale), partition_size, gp, ng, gs,
        wl, wn, ws.data_ptr() if ws is not None else None, wsb, int(kv_policy), _stream(q)),
        "paged_attention_decode_step_groups")
    return out


def paged_attention_partitions_step_groups(out, q, k_new, v_new, cow_src, k_cache, v_cache,
                                           block_tables, seq_lens, scale, groups, work_list,
                                           partition_size: int = DEFAULT_PARTITION,
                                           workspace=None, kv_policy: int = 0):
    """First pass of paged_attention_decode_step_groups only. Returns the workspace for
    paged_attention_reduce."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    _append_args(k_new, v_new, k_cache, B)
    cs = _cow_arg(cow_src, B) if cow_src is not None else None
    gp, ng, gs = _groups_arg(groups)
    ws, wsb = _workspace(q, B, Hq, W, bs, D, partition_size, workspace)
    wl, wn = _work(work_list)
    check(lib.pkv_paged_attention_partitions_step_groups(
        out.data_ptr(), odt, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), cs,
        k_cache.data_ptr(), v_cache.data_ptr(), kdt, block_tables.data_ptr(),
        seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale), partition_size, gp, ng, gs,
        wl, wn, ws.data_ptr() if ws is not None else None, wsb, int(kv_policy), _stream(q)),
        "paged_attention_partitions_step_groups")
    return ws


def paged_attention_prefix(out, q, k_cache, v_cache, block_tables, seq_lens, scale, members,
                           prefix_partitions: int, workspace,
                           partition_size: int = DEFAULT_PARTITION):
    """The shared-prefix pass alone: writes the members' partials of the shared partitions
    into `workspace` (as sized by decode_workspace_bytes), and the output row of any member
    that fits one partition into `out`."""
    B, Hq, D, NB, Hkv, bs, kdt, odt, W = _decode_args(out, q, k_cache, v_cache, block_tables,
                                                      seq_lens)
    _dev(workspace, "workspace")
    _i32(members, "members")
    check(lib.pkv_paged_attention_prefix(
        out.data_ptr(), odt, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kdt,
        block_tables.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, bs, NB, W, float(scale),
        partition_size, members.data_ptr(), members.shape[0], int(prefix_partitions),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q)),
        "paged_attention_prefix")


def paged_attention_reduce(out, seq_lens, block_size, max_blocks_per_seq, workspace,
                           partition_size: int = DEFAULT_PARTITION):
    """Second pass of paged_attention_decode only: merges the partitions' partials into out."""
    _dev(out, "out")
    _i32(seq_lens, "seq_lens")
    B, Hq, D = out.shape
    odt = _kv_dtype(out, "out")
    if workspace is None:
        wsp, wsb = None, 0
    else:
        _dev(workspace, "workspace")
        wsp, wsb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib.pkv_paged_attention_reduce(out.data_ptr(), odt, seq_lens.data_ptr(), B, Hq, D,
                                         block_size, max_blocks_per_seq, partition_size, wsp,
                                         wsb, _stream(out)), "paged_attention_reduce")
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping):
    """Stores token t's K/V rows ([Hkv][D] each) at slot slot_mapping[t] of the caches
    (bit copy; negative slots are skipped)."""
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    _i32(slot_mapping, "slot_mapping")
    if k.dim() != 3 or k.shape != v.shape or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("expected k, v [T][Hkv][D] and caches [NB][Hkv][bs][D]")
    T, Hkv, D = k.shape
    NB, Hkv2, bs, D2 = k_cache.shape
    if (Hkv, D) != (Hkv2, D2) or slot_mapping.shape != (T,):
        raise ValueError("k/v rows do not match the cache layout or slot_mapping length")
    dt = _kv_dtype(k_cache, "k_cache")
    if not (k.dtype == v.dtype == v_cache.dtype == k_cache.dtype):
        raise ValueError("k, v and the caches must share a dtype")
    check(lib.pkv_reshape_and_cache(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(),
                                    v_cache.data_ptr(), dt, slot_mapping.data_ptr(), T, Hkv, D,
                                    bs, NB, _stream(k)), "reshape_and_cache")


def copy_blocks(k_cache, v_cache, src_dst_pairs):
    """For each (src, dst) row of the int32 [n][2] tensor, block dst of both caches becomes a
    bit copy of block src."""
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache")
    _i32(src_dst_pairs, "src_dst_pairs")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.dim() != 4:
        raise ValueError("caches must share shape [NB][Hkv][bs][D] and dtype")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [n][2]")
    NB, Hkv, bs, D = k_cache.shape
    check(lib.pkv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(),
                              _kv_dtype(k_cache, "k_cache"), src_dst_pairs.data_ptr(),
                              src_dst_pairs.shape[0], Hkv, D, bs, NB, _stream(k_cache)),
          "copy_blocks")


def read_probe(buf, tile_bytes: int, tile_ids, tiles_per_group: int, sink,
               nontemporal: bool = False, sentinel: int = 0x9E3779B9):
    """Measurement only: reads the tile_bytes tiles of the byte buffer `buf` named by the
    device int32 `tile_ids`, tiles_per_group of them per 256-lane workgroup (pkv_read_probe),
    with the default or the non-temporal cache policy. `sink` is a device int32/uint32 tensor
    of at least one element."""
    _dev(buf, "buf")
    _i32(tile_ids, "tile_ids")
    _dev(sink, "sink")
    check(lib.pkv_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), int(tile_bytes),
                             tile_ids.data_ptr(), tile_ids.numel(), int(tiles_per_group),
                             1 if nontemporal else 0, int(sentinel) & 0xFFFFFFFF,
                             sink.data_ptr(), _stream(buf)),
          "read_probe")
