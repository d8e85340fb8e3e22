#!/usr/bin/env python3
"""Benchmark of one decode step of paged attention on one MI355X.

A step is one pass of the whole device path for one batch and one attention layer:
copy-on-write block copies (when the workload has any), the cache write of each sequence's new
token, the per-partition decode kernel and the partition merge. The block manager runs on the
host at set-up (its per-step cost is timed separately and reported as host_manager_us_per_step).

Default workload: 256 sequences, 32 query / 8 KV heads, head_dim 128, block 16, bf16, a
512-token prefix shared by every sequence (32 physical blocks, refcount 256) and a private
suffix of uniform length on [64, 3584]. Inputs are synthetic (seeded) and resident in HBM
before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line: value = KV-read GB/s over the distinct KV bytes the step must read
(a shared block counts once), plus decode tokens/s, the roofline of the decode kernel (bytes
per launch over its HIP-event duration) and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV-read GB/s (% of HBM peak) and decode tokens/s"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
BENCH_WORKLOADS = ("llama3_8b_gqa_prefix", "llama2_7b_mha", "long_context_splitk",
                   "llama13b_longtail", "llama13b_fork_long", "llama3_8b_long_shared_prefix",
                   "llama3_8b_short_batch",
                   "tiny")


# Packed work lists pay off on batches of short, latency-bound partitions (measured on one
# MI355X, cold steps): the long-tail mix 57.4 -> 53.1 us at 256 tokens (512: 62.9 us); the
# short batch 124.7 -> 82.8 us at 48.
DEFAULT_PACK = {"llama13b_longtail": 256, "llama3_8b_short_batch": 48}
# parallel-sampling workloads (a fork per prompt, then one appended token per branch): their
# generators in workloads/gen.py
# grid of the workloads whose measured best is not the plain list (cold steps, one MI355X):
# the branches of long forked prompts 293.9 -> 195.8 us in fork groups; a 4096-token document
# shared by 256 sequences 413 -> 118.5 us with the shared-prefix pass
DEFAULT_GRID = {"llama13b_fork_long": "forks", "llama3_8b_long_shared_prefix": "shared"}
# partition size of the (workload, grid) pairs whose measured best is not the library's default:
# the long-prompt fork groups, 1680 workgroups at 2048 tokens (1.6 resident rounds, a long
# drain), 192.9 -> 182.8 us at 1024 (1536: 184.3 us)
DEFAULT_PARTITION = {("llama13b_fork_long", "forks"): 1024}
FORKED = {"llama13b_longtail": "llama13b_longtail_case",
          "llama13b_fork_long": "llama13b_fork_long_case"}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama3_8b_gqa_prefix", choices=BENCH_WORKLOADS)
    p.add_argument("--partition", type=int, default=0,
                   help="tokens per context partition (0: the workload's measured best, %s, else "
                        "the library's default for the shapes)"
                        % ", ".join("%s with --grid %s %d" % (w, g, v)
                                    for (w, g), v in DEFAULT_PARTITION.items()))
    p.add_argument("--grid", choices=("shared", "list", "full", "forks"), default=None,
                   help="shared: partitions that a group of sequences shares run once for the "
                        "whole group on the matrix cores, the rest over a work list; list: "
                        "every partition over the host work list (one workgroup per partition "
                        "that holds tokens); full: the full partition x sequence grid; forks: "
                        "the branches of each fork in one workgroup's rows, their shared tokens "
                        "read once (workloads with a fused copy-on-write step). Default: "
                        "the workload's measured best, %s, else list"
                        % ", ".join("%s %s" % kv for kv in DEFAULT_GRID.items()))
    p.add_argument("--append", choices=("fused", "separate"), default="fused",
                   help="fused: the decode pass stores the new tokens' K/V itself; separate: "
                        "reshape_and_cache runs first as its own launch")
    p.add_argument("--pack", type=int, default=-1,
                   help="with --grid list: partitions of at most this many tokens run four to a "
                        "workgroup, one wave each (0: none; -1: the workload's measured best, "
                        "%s, else 0)" % ", ".join("%s %d" % kv for kv in DEFAULT_PACK.items()))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain block copy of known size (HBM counter calibration)")
    p.add_argument("--read-probe", action="store_true",
                   help="only measure plain HBM reads (pkv_read_probe): a 2 GiB stream, random "
                        "tiles of 4-64 KiB from a 2.5 GiB pool, and the GQA 8B workload's "
                        "pattern with a block's 8 heads read by 8 workgroups or by one")
    p.add_argument("--timeline", action="store_true",
                   help="after the timed steps, run 3 more with the per-workgroup timeline of the "
                        "decode partition kernel switched on (pkv_debug_timeline) and report "
                        "ramp-up, occupancy, tail and per-workgroup fixed cost")
    p.add_argument("--no-sched", action="store_true",
                   help="leave the workspace's scheduling word uninitialised: every workgroup of "
                        "a work-list launch keeps its static unit (for comparison)")
    p.add_argument("--keep-tail", action="store_true",
                   help="leave the work list's ticketed tail as built, shared items included "
                        "(default: pkv_decode_work_list_private_tail moves them out; for "
                        "comparison)")
    p.add_argument("--kv-policy", choices=("auto", "stream", "cached"), default="auto",
                   help="cache policy of the decode kernel's KV reads; auto: "
                        "pkv_decode_kv_policy on the workload's tables")
    p.add_argument("--no-read-probe", action="store_true",
                   help="leave the short read probe (achievable_GBps) out of the headline run")
    p.add_argument("--warm", action="store_true",
                   help="time back-to-back steps by wall clock, leaving the previous step's "
                        "KV in L2 and the 256 MB memory-side cache (default: read a 1 GiB "
                        "buffer before every step and time the step alone with HIP events)")
    p.add_argument("--serve", action="store_true",
                   help="only run the continuous-batching loop on synthetic request traffic "
                        "(scheduler + cache writes + decode every step) and, on the same "
                        "traffic, static batching")
    p.add_argument("--serve-steps", type=int, default=400)
    p.add_argument("--prefix-cache", action="store_true",
                   help="only count how many requests sharing system prompts a pool admits "
                        "with and without the prefix cache (host block manager, no GPU)")
    p.add_argument("--fork-tree", action="store_true",
                   help="only count the blocks branch trees hold (host block manager, no GPU)")
    return p.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------------
# workload set-up through the block manager
# ---------------------------------------------------------------------------------------------

def private_tail(pk, st, items, tables, lens, part, kind, group_size=1):
    """The work list with the units its launch hands out by ticket (the last half machine-full)
    made of items that read no block another item reads (pkv_decode_work_list_private_tail):
    a ticketed unit may run on another XCD than its KV head's, where a shared prefix is not in
    L2."""
    case = st["case"]
    tail = pk.decode_ticketed_items(st["k"].dtype, case.head_dim, case.num_q_heads,
                                    case.num_kv_heads, case.block_size, part, items.shape[0],
                                    kind, group_size)
    out, moved = pk.decode_work_list_private_tail(items, tables, lens, case.block_size,
                                                  case.num_blocks, part, tail)
    log("ticketed tail: %d items, %d shared items moved out of it" % (tail, moved))
    return out, moved


def build_forked_state(pk, gen, torch, dev, maker):
    """Parallel sampling step: every prompt is forked into its branches, then each branch
    appends one token; branches whose last prompt block is partial copy it first (the manager
    emits the copy-on-write pairs). The timed step replays that step: copy_blocks of the same
    pairs, cache write of the same slots, decode over the same tables."""
    fc = maker(values=False)
    bs, nb = fc.block_size, fc.num_blocks
    bm = pk.BlockManager(nb, bs, fc.free_order)
    for g, L in enumerate(fc.decode_lens.tolist()):
        parent = g * fc.branches
        bm.add_seq(parent, L - 1)
        for br in range(1, fc.branches):
            bm.fork(parent, parent + br)
    B = fc.num_seqs
    slots, pairs, cow_src = bm.append_step(range(B))
    tables, seq_lens = bm.build_tables(range(B), fc.table_width)
    case = gen.PagedDecodeCase(fc.name, fc.dtype, fc.num_q_heads, fc.num_kv_heads, fc.head_dim, bs,
                               nb, seq_lens, tables, fc.scale,
                               meta={"cow_pairs": int(pairs.shape[0]), "branches": fc.branches})
    return case, bm, slots, pairs, cow_src


def build_state(name, pk, gen, torch, dev):
    if name in FORKED:
        case, bm, slots, pairs, cow_src = build_forked_state(pk, gen, torch, dev,
                                                             getattr(gen, FORKED[name]))
        B = case.num_seqs
        shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
        seed = 402100
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
        return {
            "case": case, "bm": bm,
            "k": gen.device_normal(shape, case.dtype, seed, dev),
            "v": gen.device_normal(shape, case.dtype, seed + 1, dev),
            "q": gen.device_normal((B, case.num_q_heads, case.head_dim), case.dtype, seed + 2, dev),
            "k_new": gen.device_normal((B, case.num_kv_heads, case.head_dim), case.dtype, seed + 3, dev),
            "v_new": gen.device_normal((B, case.num_kv_heads, case.head_dim), case.dtype, seed + 4, dev),
            "tables": torch.from_numpy(case.block_tables).to(dev),
            "lens": torch.from_numpy(case.seq_lens).to(dev),
            "slots": torch.from_numpy(slots).to(dev),
            "pairs": torch.from_numpy(np.ascontiguousarray(pairs.reshape(-1, 2))).to(dev)
            if pairs.shape[0] else None,
            "cow_src": torch.from_numpy(cow_src).to(dev),
            "cow_src_host": cow_src, "slots_host": slots,
            "out": torch.empty((B, case.num_q_heads, case.head_dim), dtype=tdt, device=dev),
        }
    maker = gen.WORKLOADS[name]
    case = maker(values=False)
    B, bs, W = case.num_seqs, case.block_size, case.table_width
    lens = case.seq_lens.astype(np.int64)
    # free order that makes the manager hand out exactly the generated placement
    order, seen = [], set()
    for b in range(B):
        for j in range(-(-int(lens[b]) // bs)):
            x = int(case.block_tables[b, j])
            if x not in seen:
                seen.add(x)
                order.append(x)
    order += [x for x in range(case.num_blocks) if x not in seen]
    bm = pk.BlockManager(case.num_blocks, bs, np.array(order, np.int32))
    prefix_tokens = case.meta.get("prefix_tokens", 0)
    if prefix_tokens:
        owner = -1
        bm.add_seq(owner, prefix_tokens)
        for b in range(B):
            bm.share_prefix(owner, b, prefix_tokens // bs)
            bm.extend(b, int(lens[b]) - prefix_tokens)
        bm.free_seq(owner)
    else:
        for b in range(B):
            bm.add_seq(b, int(lens[b]))
    tables, seq_lens = bm.build_tables(range(B), W)
    assert np.array_equal(tables, case.block_tables) and np.array_equal(seq_lens, case.seq_lens)
    # the token written this step is the last one each sequence attends to
    slots = np.array([bm.slots(b, int(lens[b]) - 1, 1)[0] for b in range(B)], np.int32)
    shape = (case.num_blocks, case.num_kv_heads, bs, case.head_dim)
    seed = 402100
    st = {
        "case": case, "bm": bm,
        "k": gen.device_normal(shape, case.dtype, seed, dev),
        "v": gen.device_normal(shape, case.dtype, seed + 1, dev),
        "q": gen.device_normal((B, case.num_q_heads, case.head_dim), case.dtype, seed + 2, dev),
        "k_new": gen.device_normal((B, case.num_kv_heads, case.head_dim), case.dtype, seed + 3, dev),
        "v_new": gen.device_normal((B, case.num_kv_heads, case.head_dim), case.dtype, seed + 4, dev),
        "tables": torch.from_numpy(tables).to(dev),
        "lens": torch.from_numpy(seq_lens).to(dev),
        "slots": torch.from_numpy(slots).to(dev),
        "pairs": None,
    }
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
    st["out"] = torch.empty((B, case.num_q_heads, case.head_dim), dtype=tdt, device=dev)
    return st


def host_manager_cost(pk, case, iters=20):
    """Host microseconds per decode step of the block manager: one append per sequence plus the
    padded table export, on a private manager holding the same lengths."""
    B, bs = case.num_seqs, case.block_size
    lens = case.seq_lens.astype(np.int64)
    width = case.table_width + iters // bs + 2
    need = int((-(-lens // bs)).sum())
    bm = pk.BlockManager(max(case.num_blocks, need) + B * (iters // bs + 2), bs)
    prefix = case.meta.get("prefix_tokens", 0)
    if prefix:
        bm.add_seq(-1, prefix)
    for b in range(B):
        if prefix:
            bm.share_prefix(-1, b, prefix // bs)
            bm.extend(b, int(lens[b]) - prefix)
        else:
            bm.add_seq(b, int(lens[b]))
    ids = np.arange(B, dtype=np.int64)
    t0 = time.perf_counter()
    for _ in range(iters):
        bm.append_slots(ids)
        bm.build_tables(ids, width)
    return (time.perf_counter() - t0) / iters * 1e6


# ---------------------------------------------------------------------------------------------
# algorithmic bytes
# ---------------------------------------------------------------------------------------------

def shared_bytes(case, part, members, pp):
    """Algorithmic bytes that move from the per-partition kernel to the shared-prefix pass:
    the shared partitions' KV (read once per KV head), the members' q (read again), the
    shared partitions' table entries, and the partials of the shared partitions."""
    eb = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    n = int(len(members))
    kv = case.kv_bytes_per_token() * pp * part
    tables = 4 * n * pp * (part // case.block_size)
    partials = n * pp * case.num_q_heads * (case.head_dim + 2) * 4
    q = n * case.num_q_heads * case.head_dim * eb
    return {"kv": kv, "tables": tables, "partials": partials, "q": q,
            "prefix_kernel": kv + 4 * pp * (part // case.block_size) + 4 * n + q + partials}


def byte_model(case, part):
    eb = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    B, Hq, D, bs = case.num_seqs, case.num_q_heads, case.head_dim, case.block_size
    lens = case.seq_lens.astype(np.int64)
    kv_tok = case.kv_bytes_per_token()
    unique = kv_tok * case.unique_slots()
    logical = kv_tok * int(lens.sum())
    nparts = np.maximum(1, -(-lens // part))
    multi = nparts > 1
    tables = 4 * int((-(-lens // bs)).sum())
    q = B * Hq * D * eb
    partial_rows = int((nparts * multi).sum()) * Hq
    partials = partial_rows * (D + 2) * 4
    out_single = int((~multi).sum()) * Hq * D * eb
    out_all = B * Hq * D * eb
    decode_kernel = unique + q + tables + 4 * B + partials + out_single
    reduce_kernel = partials + out_all - out_single
    cache_write = 2 * 2 * B * case.num_kv_heads * D * eb    # read new rows, write slots
    return {"kv_unique": unique, "kv_logical": logical, "decode_kernel": decode_kernel,
            "reduce_kernel": reduce_kernel, "cache_write": cache_write,
            "partitions": int(nparts.sum()), "multi_partition_seqs": int(multi.sum())}


# ---------------------------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# ---------------------------------------------------------------------------------------------

def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (platform.processor() is often just the
    architecture)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(st, target_s, gen):
    from oracle import paged_attention as opa
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl absent: numpy's default is one BLAS pool
        blas_threads = os.cpu_count() or 1
    import torch
    case = st["case"]
    dt, bs = case.dtype, case.block_size
    kv_tok = case.kv_bytes_per_token()

    def host(t):
        t = t.cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()

    spent, done, seen, passes_bytes = 0.0, 0, {}, 0
    for b in (i % case.num_seqs for i in range(10 ** 9)):
        if b == 0 and done:                  # a pass over the batch is one step's work
            passes_bytes += kv_tok * sum(seen.values())
            seen = {}
        L = int(case.seq_lens[b])
        nb = -(-L // bs)
        ids = case.block_tables[b, :nb]
        idx = torch.from_numpy(ids.astype(np.int64)).to(st["k"].device)
        ksub, vsub = host(st["k"][idx]), host(st["v"][idx])
        q = host(st["q"][b:b + 1])
        table = np.arange(nb, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        opa.decode_attention(q, ksub, vsub, table, np.array([L], np.int32), case.scale, dt)
        spent += time.perf_counter() - t0
        done += 1
        for j, blk in enumerate(ids.tolist()):
            seen[blk] = max(seen.get(blk, 0), min(bs, L - j * bs))
        if spent >= target_s:
            break
    uniq_bytes = passes_bytes + kv_tok * sum(seen.values())
    return {"value": round(uniq_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": "fp64 numpy oracle, %d sequence decodes (all %d query heads) cycling over "
                      "the %d sequences in order until %.1f s; GB/s over each pass's distinct KV "
                      "bytes (a pass over the batch is one step), summed; host %s, %d "
                      "logical CPUs" % (done, case.num_q_heads, case.num_seqs, spent,
                                        cpu_model(), len(os.sched_getaffinity(0))),
            "cpu_model": cpu_model(), "logical_cpus": len(os.sched_getaffinity(0)),
            "seconds": round(spent, 3), "tokens_per_s": round(done / spent, 3)}


# ---------------------------------------------------------------------------------------------

# ---------------------------------------------------------------------------------------------
# measured HBM traffic of the decode kernel (from rocprofv3 counter runs kept under profiles/)
# ---------------------------------------------------------------------------------------------

KERNEL_SOURCES = ("paged_kv_cache_402_amd/csrc/decode.hip",
                  "paged_kv_cache_402_amd/csrc/decode_kernel.h",
                  "paged_kv_cache_402_amd/csrc/decode_step.hip",
                  "paged_kv_cache_402_amd/csrc/decode_groups.hip",
                  "paged_kv_cache_402_amd/csrc/common.h",
                  "paged_kv_cache_402_amd/csrc/launch.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# the launch settings that a traffic profile must share with the run it is reported for
TRAFFIC_LAUNCH_KEYS = ("partition_size", "grid", "pack_tokens", "append", "copy_on_write",
                       "kv_policy", "late_units", "ticketed_tail_shared_items_moved")


def traffic_launch_key(config):
    return ",".join("%s=%s" % (k, config.get(k)) for k in TRAFFIC_LAUNCH_KEYS)


def measured_traffic(workload_name, config):
    """HBM bytes per launch of the decode kernel from profiles/hbm_traffic_<workload>*.txt:
    FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the same counter reads for a
    copy of known size. Only a profile of the same launch settings counts (its launch_key);
    None when there is none, or when the kernel sources changed since it was taken."""
    key = traffic_launch_key(config)
    prefix = "hbm_traffic_%s" % workload_name
    pdir = os.path.join(ROOT, "profiles")
    for fname in sorted(os.listdir(pdir)):
        if not (fname.startswith(prefix) and fname.endswith(".txt")):
            continue
        kv = {}
        with open(os.path.join(pdir, fname)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("workload") != workload_name or kv.get("launch_key") != key:
            continue
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        try:
            return int(float(kv["traffic_bytes_per_launch"]))
        except (KeyError, ValueError):
            return None
    return None


def copy_probe(pk, torch, dev):
    """A plain copy of known size through copy_blocks: 4096 blocks of 64 KiB per cache, read
    once and written once (512 MiB each way), repeated 5 times."""
    nb, H, bs, D = 8192, 8, 16, 128
    k = torch.zeros((nb, H, bs, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(0, 4096), torch.arange(4096, 8192)], 1).to(torch.int32).to(dev)
    for _ in range(5):
        pk.copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    per = 2 * 4096 * H * bs * D * 2
    print(json.dumps({"copy_probe": True, "bytes_read_per_launch": per,
                      "bytes_written_per_launch": per, "launches": 5}), flush=True)


PROBE_POOL_BYTES = 5 << 29          # 2.5 GiB: the GQA 8B pool's size, beyond the 256 MB MALL
PROBE_READ_BYTES = 1820 << 20       # about the GQA 8B decode kernel's bytes per launch


def probe_patterns(full):
    """(name, tile_bytes, tile ids, tiles per workgroup, what it stands for). Seeded."""
    rng = np.random.default_rng(402700)
    pats = [("stream_2GiB", 64 << 10, np.arange((2 << 30) >> 16), 16,
             "one 2 GiB contiguous read, 1 MiB per workgroup")]

    def rand_tiles(tb, tpw):
        n = PROBE_READ_BYTES // tb
        ids = rng.choice(PROBE_POOL_BYTES // tb, n, replace=False)
        return ("random_%dKiB" % (tb >> 10), tb, ids, tpw,
                "%d distinct random %d KiB tiles of a 2.5 GiB pool, 1 MiB per workgroup"
                % (n, tb >> 10))
    pats.append(rand_tiles(4 << 10, 256))
    if not full:
        return pats
    for tb in (8 << 10, 16 << 10, 64 << 10):
        pats.append(rand_tiles(tb, (1 << 20) // tb))
    # the GQA 8B workload's pattern: blocks of 8 KV heads x 4 KiB (32 KiB, one cache), a
    # workgroup per (256-block item, KV head) with the heads of one item consecutive (so the
    # 8 XCDs take one head each), against one workgroup reading 32 whole blocks
    nblk = PROBE_READ_BYTES // (32 << 10) // 256 * 256
    blocks = rng.choice(PROBE_POOL_BYTES // (32 << 10), nblk, replace=False)
    items = blocks.reshape(-1, 256)
    split = (items[:, None, :] * 8 + np.arange(8)[None, :, None]).reshape(-1)
    pats.append(("gqa_heads_split_4KiB", 4 << 10, split, 256,
                 "%d random 32 KiB blocks; workgroup (item of 256 blocks, head h) reads head "
                 "h's 4 KiB of each; consecutive workgroups differ in head" % nblk))
    pats.append(("gqa_heads_grouped_32KiB", 32 << 10, blocks, 32,
                 "the same %d blocks; one workgroup reads 32 whole blocks" % nblk))
    # the same 4 KiB tiles as random_4KiB, a quarter of them, each group of 256 read by four
    # consecutive workgroups: the reuse of blocks that forked sequences share
    quarter = pats[1][2][: len(pats[1][2]) // 4 // 256 * 256].reshape(-1, 256)
    pats.append(("shared4_4KiB", 4 << 10, np.repeat(quarter, 4, axis=0).reshape(-1), 256,
                 "%d of the random 4 KiB tiles, each item of 256 read by 4 consecutive "
                 "workgroups (bytes counts every read)" % quarter.size))
    pats.append(("random_4KiB_one_per_group", 4 << 10,
                 rng.choice(PROBE_POOL_BYTES >> 12, PROBE_READ_BYTES >> 12, replace=False), 1,
                 "the same bytes as random_4KiB, one tile (4 KiB) per workgroup"))
    return pats


PROBE_POLICIES = (("default", False), ("nontemporal", True))


def read_probe(pk, torch, dev, full, reps=10):
    """Plain-read bandwidth of each pattern under each load cache policy (the default one, and
    the non-temporal one of the attention kernels' KV-row loads): 2 warm-up launches, then
    `reps` launches, each after a 1 GiB read of other data (cold L2 and memory-side cache, as
    the decode timing); HIP events on the launch stream around each; GB/s = bytes read /
    median launch time."""
    buf = torch.ones(PROBE_POOL_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    evict = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    evict_sum = torch.zeros((), dtype=torch.float32, device=dev)
    res = []
    for name, tb, ids, tpw, what in probe_patterns(full):
        d_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev)
        for policy, nt in PROBE_POLICIES:
            for _ in range(2):
                pk.read_probe(buf, tb, d_ids, tpw, sink, nontemporal=nt)
            ts = []
            for _ in range(reps):
                torch.sum(evict, dim=0, out=evict_sum)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                pk.read_probe(buf, tb, d_ids, tpw, sink, nontemporal=nt)
                e1.record()
                ts.append((e0, e1))
            torch.cuda.synchronize()
            ms = np.array([a.elapsed_time(b) for a, b in ts])
            nbytes = int(len(ids)) * tb
            res.append({"pattern": name, "policy": policy, "bytes": nbytes, "tile_bytes": tb,
                        "workgroups": -(-len(ids) // tpw),
                        "median_ms": round(float(np.median(ms)), 5),
                        "GBps": round(nbytes / (float(np.median(ms)) * 1e-3) / 1e9, 1),
                        "GBps_p10_p90": [round(nbytes / (float(np.percentile(ms, q)) * 1e-3)
                                               / 1e9, 1) for q in (90, 10)],
                        "what": what})
            log("read probe %s, %s policy: %.1f GB/s" % (name, policy, res[-1]["GBps"]))
    del buf, evict
    return res


def probe_rate(probe, pattern, policy):
    for r in probe:
        if r["pattern"] == pattern and r["policy"] == policy:
            return r["GBps"]
    raise KeyError((pattern, policy))


def timeline_summary(tl, items, num_kv_heads, part, lens, kv_row_bytes):
    """Per-workgroup records {start, end, HW_ID, XCC_ID} (100 MHz clock) of one launch over
    a work list -> occupancy, ramp-up, tail and fixed cost per workgroup."""
    rec = tl.reshape(-1, 8).astype(np.int64)
    ok = rec[:, 1] != 0
    wg = np.nonzero(ok)[0]
    unit = rec[ok, 4]
    t0 = rec[ok, 0].min()
    start = (rec[ok, 0] - t0) / 100.0          # us
    end = (rec[ok, 1] - t0) / 100.0
    span = float(end.max())
    # tokens of each workgroup's partition
    it = items[unit // num_kv_heads].astype(np.int64) & 0xFFFFFFFF
    b, p = it >> 16, it & 0xFFFF
    n = np.minimum(lens[b].astype(np.int64) - p * part, part)
    grid = np.arange(0.0, span, 0.25)
    active = np.array([int(((start <= t) & (end > t)).sum()) for t in grid])
    peak = int(active.max())
    ramp = float(grid[np.argmax(active >= 0.95 * peak)])
    tail_from = float(grid[len(active) - 1 - np.argmax(active[::-1] >= 0.9 * peak)])
    dur = end - start
    # duration = fixed + per-token: least squares over all workgroups
    A = np.stack([np.ones_like(n, dtype=np.float64), n.astype(np.float64)], 1)
    coef = np.linalg.lstsq(A, dur, rcond=None)[0]
    xcc = rec[ok, 3] & 0xF
    first_k = float(np.sort(start)[min(len(start) - 1, peak - 1)])
    head = unit % num_kv_heads
    # phases of wave 0 (start -> end of K pass -> end of V pass -> end), by partition length
    tk = (rec[ok, 5] - rec[ok, 0]) / 100.0
    tv = (rec[ok, 6] - rec[ok, 5]) / 100.0
    te = (rec[ok, 1] - rec[ok, 6]) / 100.0
    phases = {}
    for lo, hi in ((0, 32), (32, 128), (128, 512), (512, 1024), (1024, 4096)):
        sel = (n >= lo) & (n < hi) & (rec[ok, 5] != 0) & (rec[ok, 6] != 0)
        if sel.any():
            phases["%d-%d" % (lo, hi - 1)] = {
                "workgroups": int(sel.sum()),
                "to_k_end_us": round(float(np.median(tk[sel])), 2),
                "k_end_to_v_end_us": round(float(np.median(tv[sel])), 2),
                "v_end_to_end_us": round(float(np.median(te[sel])), 2)}
    # bandwidth estimate: each workgroup's KV bytes (K and V rows of its tokens, one head)
    # spread evenly over its lifetime, summed per 5 us window
    kv_bytes = 2 * n.astype(np.float64) * kv_row_bytes
    win = 5.0
    edges = np.arange(0.0, span + win, win)
    bw = np.zeros(len(edges) - 1)
    for s0, e0, by in zip(start, end, kv_bytes):
        if e0 <= s0:
            continue
        lo = np.clip(edges[:-1], s0, e0)
        hi = np.clip(edges[1:], s0, e0)
        bw += by * (hi - lo) / (e0 - s0)
    bw_tbps = bw / (win * 1e-6) / 1e12
    mean_bw = float(kv_bytes.sum() / (span * 1e-6) / 1e12)
    return {"workgroups": int(ok.sum()), "span_us": round(span, 2), "peak_active": peak,
            "xcd_is_id_mod_8": round(float(((wg % 8) == xcc).mean()), 4),
            "last_end_per_head_us": [round(float(end[head == h].max()), 2)
                                     for h in range(min(num_kv_heads, 8))],
            "mean_active": round(float(active.mean()), 1),
            "ramp_to_95pct_us": round(ramp, 2),
            "first_%d_started_by_us" % peak: round(first_k, 2),
            "tail_below_90pct_us": round(span - tail_from, 2),
            "fixed_us_per_workgroup": round(float(coef[0]), 2),
            "us_per_1k_tokens": round(float(coef[1]) * 1000, 2),
            "mean_duration_us": round(float(dur.mean()), 2),
            "last_end_per_xcd_us": [round(float(end[xcc == x].max()), 2) if (xcc == x).any()
                                    else None for x in range(8)],
            "phases_median_by_tokens": phases,
            "kv_TBps_mean": round(mean_bw, 3),
            "kv_TBps_per_5us": [round(float(x), 2) for x in bw_tbps]}


def serve_loop(pk, torch, dev, steps, static=False, warm_steps=None):
    """Continuous batching on synthetic traffic with the GQA 8B layer shape (32 query / 8 KV
    heads, head_dim 128, block 16, bf16): Poisson arrivals of 2.5 requests per step, prompts
    uniform on [64, 1024] tokens, outputs geometric with mean 128 (at most 512), a pool of
    10240 blocks (163840 tokens), at most 256 running requests and 16384 tokens per step.
    Every step runs the C++ scheduler, writes the admitted prompts' and the new tokens' K/V
    (reshape_and_cache), then decodes the batch (work list + merge), and synchronises, as a
    server does before sampling. static=True admits a new batch only when the previous one
    has finished (static batching, P1 §8.2). Returns per-step records of the timed steps."""
    from workloads import traces
    NB, bs, Hq, Hkv, D, W = 10240, 16, 32, 8, 128, 96
    max_seqs, budget = 256, 16384
    part = pk.default_partition(max_seqs, Hq, Hkv, D, bs, W)
    rng = np.random.default_rng(402900)
    reqs = traces.request_stream(rng, 4000, 2.5, (64, 1024), 128, 512)
    bm = pk.BlockManager(NB, bs)
    sched = pk.Scheduler(bm, max_seqs, budget, 16)
    k = torch.zeros((NB, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    g = torch.Generator(device=dev)
    g.manual_seed(402901)
    kv_new = torch.randn((budget, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((max_seqs, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((max_seqs, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(pk.decode_workspace_bytes(max_seqs, Hq, W, bs, D, part), dtype=torch.uint8,
                     device=dev)
    pin = lambda n: torch.empty(n, dtype=torch.int32, pin_memory=True)
    h_slots, h_tab, h_lens = pin(budget), pin(max_seqs * W), pin(max_seqs)
    h_work = pin(max_seqs * (W * bs // part + 1))
    d_slots = torch.empty(budget, dtype=torch.int32, device=dev)
    d_tab = torch.empty(max_seqs * W, dtype=torch.int32, device=dev)
    d_lens = torch.empty(max_seqs, dtype=torch.int32, device=dev)
    d_work = torch.empty_like(h_work, device=dev)
    pending = sorted(reqs, key=lambda r: r.arrival)
    held = []                        # static batching: arrived, not yet handed to the scheduler
    warm_steps = steps // 2 if warm_steps is None else warm_steps
    recs = []
    for step in range(warm_steps + steps):
        t0 = time.perf_counter()
        while pending and pending[0].arrival <= step:
            held.append(pending.pop(0))
        st = sched.stats()
        if not static or (st["running"] == 0 and st["waiting"] == 0):
            take = held if not static else held[:max_seqs]
            for r in take:
                sched.add_request(r.req_id, r.prompt_len, r.output_len)
            held = held[len(take):]
        s = sched.step()
        n, T = s.batch.shape[0], s.slots.shape[0]
        if T:
            h_slots[:T] = torch.from_numpy(s.slots)
            d_slots[:T].copy_(h_slots[:T], non_blocking=True)
            pk.reshape_and_cache(kv_new[:T], kv_new[:T], k, v, d_slots[:T])
        if n:
            tab, lens = bm.build_tables(s.batch, W)
            items = pk.decode_work_list(lens, W, bs, part)
            h_tab[:n * W] = torch.from_numpy(tab.reshape(-1))
            h_lens[:n] = torch.from_numpy(lens)
            h_work[:items.shape[0]] = torch.from_numpy(items)
            d_tab[:n * W].copy_(h_tab[:n * W], non_blocking=True)
            d_lens[:n].copy_(h_lens[:n], non_blocking=True)
            d_work[:items.shape[0]].copy_(h_work[:items.shape[0]], non_blocking=True)
            pk.paged_attention_decode(out[:n], q[:n], k, v, d_tab[:n * W].view(n, W), d_lens[:n],
                                      0.0884, partition_size=part, workspace=ws,
                                      work_list=d_work[:items.shape[0]],
                                      kv_policy=pk.decode_kv_policy(tab, lens, bs, NB))
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if step >= warm_steps:
            recs.append({"s": dt, "batch": n, "slots": T, "used": bm.stats()["used"],
                         "preempted": len(s.preempted), "finished": len(s.finished),
                         "kv_tokens": int(lens.sum()) if n else 0})
    return recs, NB


def serve_report(pk, torch, dev, steps):
    out = {"serve": True, "workload": "gqa8b_layer_poisson2.5_prompt64-1024_out128",
           "num_blocks": 10240, "block_size": 16, "max_num_seqs": 256}
    for mode in ("continuous", "static"):
        recs, NB = serve_loop(pk, torch, dev, steps, static=(mode == "static"))
        t = sum(r["s"] for r in recs)
        tok = sum(r["batch"] for r in recs)
        kv = sum(r["kv_tokens"] for r in recs) * 2 * 8 * 128 * 2
        out[mode] = {"steps": len(recs), "seconds": round(t, 4),
                     "decode_tokens_per_s": round(tok / t, 1),
                     "ms_per_step": round(1e3 * t / len(recs), 4),
                     "mean_batch": round(tok / len(recs), 1),
                     "pool_utilisation": round(float(np.mean([r["used"] for r in recs])) / NB, 4),
                     "prompt_tokens_per_step": round(float(np.mean([r["slots"] - r["batch"]
                                                                    for r in recs])), 1),
                     "preempted": sum(r["preempted"] for r in recs),
                     "finished": sum(r["finished"] for r in recs),
                     "logical_kv_GBps": round(kv / t / 1e9, 1)}
        log("%s: %s" % (mode, out[mode]))
    print(json.dumps(out), flush=True)


def prefix_cache_admission(pk, num_blocks, bs, system_lens, rng, cached, max_requests=100000):
    """Admits requests (a system prompt drawn uniformly from `system_lens`' prompts, then a
    private user part of U[16, 512] random token ids) into a fixed pool until one does not
    fit. Returns (requests admitted, prompt tokens, tokens found in the cache)."""
    prompts = [rng.integers(0, 32000, n).astype(np.int32) for n in system_lens]
    bm = pk.BlockManager(num_blocks, bs)
    admitted = tokens = hit_tokens = 0
    while admitted < max_requests:
        sysp = prompts[int(rng.integers(0, len(prompts)))]
        user = rng.integers(0, 32000, int(rng.integers(16, 513))).astype(np.int32)
        toks = np.concatenate([sysp, user])
        if cached:
            st, hit = bm.add_seq_cached_status(admitted, toks)
        else:
            st, hit = bm.add_seq_status(admitted, int(toks.shape[0])), 0
        if st < 0:
            break
        admitted += 1
        tokens += int(toks.shape[0])
        hit_tokens += hit
    bm.close()
    return admitted, tokens, hit_tokens


def prefix_cache_report(pk):
    """P3 §2.2.8 / §2.2.11: requests that share a system prompt reuse its cached blocks, so a
    pool of 10240 blocks of 16 tokens admits more of them. Seeded; host only."""
    rows = []
    for k in (1, 4, 16):
        for sys_len in (256, 512, 1024, 2048):
            res = {}
            for cached in (False, True):
                rng = np.random.default_rng(403000 + k * 10000 + sys_len)
                res[cached] = prefix_cache_admission(pk, 10240, 16, [sys_len] * k, rng, cached)
            a0, a1 = res[False][0], res[True][0]
            rows.append({"system_prompts": k, "system_tokens": sys_len, "admitted_private": a0,
                         "admitted_cached": a1, "capacity_gain": round(a1 / a0 - 1, 4),
                         "prompt_tokens_cached": round(res[True][2] / res[True][1], 4)})
    print(json.dumps({"prefix_cache": True, "num_blocks": 10240, "block_size": 16,
                      "user_tokens": "U[16, 512]", "rows": rows}), flush=True)


def fork_tree_report(pk):
    """Blocks held by branch trees on the block manager against private copies per branch
    (every branch holding ceil(tokens / block_size) blocks of its own). Prompts of
    Geometric(1/200) tokens clipped to [1, 2048] (the long-tail length mix), block size 16;
    parallel sampling: n branches of 128 tokens; beam search: `width` beams for 128 steps.
    saving = 1 - sum over steps of blocks held / sum of private blocks, over the steps where
    more than one branch is alive; peak = the largest per-step count of each."""
    from workloads import traces
    rng = np.random.default_rng(402500)
    prompts = np.clip(rng.geometric(1 / 200, size=32), 1, 2048)
    bs = 16
    rows = []
    settings = [("parallel_sampling", n) for n in (2, 4, 8)] + [("beam_search", w)
                                                                  for w in (2, 4, 8)]
    for kind, n in settings:
        held = private = peak_h = peak_p = steps = 0
        t_host = 0.0
        for i, P in enumerate(prompts.tolist()):
            trng = np.random.default_rng(402600 + i)
            if kind == "parallel_sampling":
                tr = traces.parallel_sampling_trace(trng, P, n, 128)
            else:
                tr = traces.beam_search_trace(trng, P, n, 128)
            need = 4 * n * (-(-(P + 130) // bs)) + 8
            bm = pk.BlockManager(need, bs)
            bm.add_seq(tr.root, P)
            live = {tr.root}
            ntok = {tr.root: P}
            for st in tr.steps:
                t0 = time.perf_counter()
                for s in st.frees:
                    bm.free_seq(s)
                for par, c in st.forks:
                    bm.fork(par, c)
                if st.appends:
                    bm.append_slots(st.appends)
                t_host += time.perf_counter() - t0
                live -= set(st.frees)
                for par, c in st.forks:
                    live.add(c)
                    ntok[c] = ntok[par]
                for s in st.appends:
                    ntok[s] += 1
                if len(live) > 1:
                    h = bm.stats()["used"]
                    pv = sum(-(-ntok[s] // bs) for s in live)
                    held, private, steps = held + h, private + pv, steps + 1
                    peak_h, peak_p = max(peak_h, h), max(peak_p, pv)
            bm.close()
        rows.append({"tree": kind, "branches": n, "prompts": len(prompts),
                     "saving": round(1 - held / private, 4),
                     "saving_at_peak": round(1 - peak_h / peak_p, 4),
                     "mean_blocks_held": round(held / steps, 1),
                     "mean_blocks_private": round(private / steps, 1),
                     "host_us_per_step": round(t_host / max(1, steps) * 1e6, 2)})
    print(json.dumps({"fork_tree": True, "block_size": bs,
                      "prompt_mean": round(float(prompts.mean()), 1), "rows": rows}), flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), flush=True)
        sys.exit(2)
    if args.fork_tree or args.prefix_cache:
        import paged_kv_cache_402_amd as pk
        if args.fork_tree:
            fork_tree_report(pk)
        if args.prefix_cache:
            prefix_cache_report(pk)
        return
    import torch
    import paged_kv_cache_402_amd as pk
    from workloads import gen
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(pk, torch, dev)
        return
    if args.read_probe:
        print(json.dumps({"read_probe": read_probe(pk, torch, dev, full=True),
                          "peak_GBps": HBM_PEAK_GBPS}), flush=True)
        return
    if args.serve:
        serve_report(pk, torch, dev, args.serve_steps)
        return

    if args.pack < 0:
        args.pack = DEFAULT_PACK.get(args.workload, 0)
    if args.grid is None:
        args.grid = DEFAULT_GRID.get(args.workload, "list")
    log("setting up %s" % args.workload)
    st = build_state(args.workload, pk, gen, torch, dev)
    case = st["case"]
    part = (args.partition or DEFAULT_PARTITION.get((args.workload, args.grid))
            or pk.default_partition(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                    case.head_dim, case.block_size, case.table_width))
    bytes_ = byte_model(case, part)
    work, members, pp, items = None, None, 0, None
    groups = None
    # the ticketed tail made private (late units are ticketed only over an initialised
    # workspace; the list and fork grids keep this partition)
    reorder_tail = (pk.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.table_width,
                                              case.block_size, case.head_dim, part) > 0
                    and not args.no_sched and not args.keep_tail)
    moved = 0
    kind = "copy_on_write" if st["pairs"] is not None and args.append == "fused" else "plain"
    if args.grid == "forks":
        if "cow_src_host" not in st or args.append != "fused":
            raise SystemExit("--grid forks needs a forked workload (%s) and the "
                             % ", ".join(FORKED) +
                             "fused append")
        # as many branches per group as the rows of a workgroup allow (8 query rows at most)
        gsize = max(1, min(case.meta.get("branches", 1),
                           8 // (case.num_q_heads // case.num_kv_heads)))
        groups_h, glens = pk.plan_fork_groups(case.block_tables, case.seq_lens,
                                              st["cow_src_host"], case.block_size,
                                              case.num_blocks, gsize)
        groups = torch.from_numpy(np.ascontiguousarray(groups_h)).to(dev)
        if args.pack > 0:
            items, rows = pk.decode_work_list_packed(glens, case.table_width, case.block_size,
                                                     part, args.pack)
            work = (torch.from_numpy(items).to(dev), rows)
        else:
            items = pk.decode_work_list(glens, case.table_width, case.block_size, part)
            if reorder_tail:
                items, moved = private_tail(pk, st, items, case.block_tables[groups_h[:, 0]],
                                            glens, part, "fork_groups", gsize)
            work = torch.from_numpy(items).to(dev)
        # table entries: each group's shared ones once, plus every member's entry of its new
        # token's block; the group rows, the list and the groups' lengths
        bs_ = case.block_size
        per_seq_tables = 4 * int((-(-case.seq_lens.astype(np.int64) // bs_)).sum())
        group_tables = 4 * int((-(-glens.astype(np.int64) // bs_)).sum()) + 4 * case.num_seqs
        bytes_["decode_kernel"] += (group_tables - per_seq_tables + 4 * int(items.shape[0])
                                    + 4 * groups_h.size - 4 * (case.num_seqs - groups_h.shape[0]))
        log("fork groups: %d of up to %d sequences, work list %d entries"
            % (groups_h.shape[0], gsize, items.shape[0]))
    elif args.grid == "list" and args.pack > 0:
        items, rows = pk.decode_work_list_packed(case.seq_lens, case.table_width,
                                                 case.block_size, part, args.pack)
        work = (torch.from_numpy(items).to(dev), rows)
        bytes_["decode_kernel"] += 4 * int(items.shape[0])     # rows and packed items
        log("work list: %d rows, %d entries" % (rows, items.shape[0]))
    elif args.grid == "list":
        items = pk.decode_work_list(case.seq_lens, case.table_width, case.block_size, part)
        if reorder_tail:
            items, moved = private_tail(pk, st, items, case.block_tables, case.seq_lens, part,
                                        kind)
        work = torch.from_numpy(items).to(dev)
        bytes_["decode_kernel"] += 4 * int(items.shape[0])     # one item read per launch
    elif args.grid == "shared":
        mem, pp, items = pk.plan_shared_prefix(case.block_tables, case.seq_lens, case.block_size,
                                               part)
        # the shared pass launches (KV heads x row chunks x shared partitions) workgroups: with
        # no partition asked for, halve the partition while that gives under two per compute
        # unit (512)
        while not args.partition and part > 256 and pp > 0:
            chunks = -(-mem.shape[0] // (64 // (case.num_q_heads // case.num_kv_heads)))
            if case.num_kv_heads * chunks * pp >= 512:
                break
            part //= 2
            bytes_ = byte_model(case, part)
            mem, pp, items = pk.plan_shared_prefix(case.block_tables, case.seq_lens,
                                                   case.block_size, part)
        work = torch.from_numpy(items).to(dev)
        members = torch.from_numpy(mem).to(dev)
        sb = shared_bytes(case, part, mem, pp)
        bytes_["decode_kernel"] += 4 * int(items.shape[0]) - sb["kv"] - sb["tables"] - sb["partials"]
        bytes_["prefix_kernel"] = sb["prefix_kernel"]
        log("shared prefix: %d members, %d partitions" % (mem.shape[0], pp))
    # cache policy of the per-partition pass's KV reads, from the tables and the partitions
    # that pass reads (pkv_decode_kv_policy; the shared-prefix list leaves the shared
    # partitions to the prefix pass)
    policy = {"stream": pk.KV_STREAM, "cached": pk.KV_CACHED}.get(args.kv_policy)
    if policy is None and groups is not None:
        # the list names groups: their first members' tables and the groups' lengths
        policy = pk.decode_kv_policy(case.block_tables[groups_h[:, 0]], glens, case.block_size,
                                     case.num_blocks, work_list=items, partition_size=part)
    elif policy is None:
        policy = pk.decode_kv_policy(case.block_tables, case.seq_lens, case.block_size,
                                     case.num_blocks, work_list=items, partition_size=part)
    log("KV read policy: %s" % ("cached" if policy == pk.KV_CACHED else "stream"))
    # no workspace: no sequence spans two partitions and the merge pass has nothing to do
    ws_bytes = pk.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.table_width,
                                         case.block_size, case.head_dim, part)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    if ws_bytes and not args.no_sched:
        pk.decode_workspace_init(ws)     # list launches hand out late units from its header
    elif ws_bytes:
        ws.zero_()                       # no scheduling cookie: static units only
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    # the step's stages in launch order; one event before the first and one after each stage
    # that runs, so a stage's time is the span between its neighbouring events
    # (with --grid shared the new token always lies in a sequence's own partitions, which the
    # fused per-partition pass covers; the shared-prefix pass never reads it)
    fused = args.append == "fused"
    # with the cache write fused, the copies of copy-on-write blocks are fused too
    fused_cow = fused and st["pairs"] is not None
    if fused:
        # the new rows are stored by the decode pass: 2 * B * Hkv * d * eb more bytes written
        bytes_["decode_kernel"] += bytes_["cache_write"] // 2
    if fused_cow:
        # the copies: a copying sequence reads its last block's rows before the new token from
        # the source block (which its siblings list too) and writes them into its copy. The
        # copy's rows are then written, never read: they leave the distinct bytes read and
        # enter the bytes written, so the kernel's total stays as counted
        copied = st["cow_src_host"] >= 0
        copy_rows = int((st["slots_host"][copied] % case.block_size).sum())
        bytes_["kv_unique"] -= copy_rows * case.kv_bytes_per_token()
    stages = (["copy_blocks"] if st["pairs"] is not None and not fused_cow else []) + \
        ([] if fused else ["reshape_and_cache"]) + \
        (["shared_prefix"] if members is not None and pp > 0 else []) + \
        ["decode_partitions"] + (["partition_reduce"] if ws_bytes > 0 else [])

    def run_stage(name):
        if name == "copy_blocks":
            pk.copy_blocks(st["k"], st["v"], st["pairs"])
        elif name == "reshape_and_cache":
            pk.reshape_and_cache(st["k_new"], st["v_new"], st["k"], st["v"], st["slots"])
        elif name == "shared_prefix":
            pk.paged_attention_prefix(st["out"], st["q"], st["k"], st["v"], st["tables"], st["lens"],
                                      case.scale, members, pp, ws, partition_size=part)
        elif name == "decode_partitions" and groups is not None:
            pk.paged_attention_partitions_step_groups(st["out"], st["q"], st["k_new"], st["v_new"],
                                                      st["cow_src"], st["k"], st["v"],
                                                      st["tables"], st["lens"], case.scale,
                                                      groups, work, partition_size=part,
                                                      workspace=ws, kv_policy=policy)
        elif name == "decode_partitions" and fused_cow:
            pk.paged_attention_partitions_step(st["out"], st["q"], st["k_new"], st["v_new"],
                                               st["cow_src"], st["k"], st["v"], st["tables"],
                                               st["lens"], case.scale, partition_size=part,
                                               workspace=ws, work_list=work, kv_policy=policy)
        elif name == "decode_partitions" and fused:
            pk.paged_attention_partitions_append(st["out"], st["q"], st["k_new"], st["v_new"],
                                                 st["k"], st["v"], st["tables"], st["lens"],
                                                 case.scale, partition_size=part, workspace=ws,
                                                 work_list=work, kv_policy=policy)
        elif name == "decode_partitions":
            # paged_attention_decode's two launches, called apart so each has its own events
            pk.paged_attention_partitions(st["out"], st["q"], st["k"], st["v"], st["tables"],
                                          st["lens"], case.scale, partition_size=part,
                                          workspace=ws, work_list=work, kv_policy=policy)
        else:
            pk.paged_attention_reduce(st["out"], st["lens"], case.block_size, case.table_width,
                                      ws, partition_size=part)

    def step(evs=None):
        """One step; evs: None, or events recorded before the first stage and after the last
        (two events), or before the first and after every stage (len(stages) + 1)."""
        if evs is not None:
            evs[0].record()
        for j, name in enumerate(stages):
            run_stage(name)
            if evs is not None and len(evs) > 2:
                evs[j + 1].record()
        if evs is not None and len(evs) == 2:
            evs[1].record()

    def new_events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    # The read probe (achievable bandwidth) runs before the warm-up steps: it also keeps the GPU
    # busy long enough for its clocks to settle, which the few warm-up steps alone do not (run
    # after the timed steps, the probe left the first timed steps up to 8% slower than the rest).
    probe = None
    if not args.no_read_probe:
        log("read probe (achievable read bandwidth)")
        probe = read_probe(pk, torch, dev, full=False)
    log("warmup %d" % W)
    for _ in range(W):
        step()
    torch.cuda.synchronize()
    # Each layer of a model reads its own KV once per step, so between two reads of one
    # layer's KV the other layers' KV has passed through the caches. Reading (not writing:
    # dirty lines would be written back inside the timed step) 1 GiB of other data before
    # every step gives the step the same cold L2 and memory-side cache.
    evict = None if args.warm else torch.ones(1 << 28, dtype=torch.float32, device=dev)
    evict_sum = torch.zeros((), dtype=torch.float32, device=dev)

    def timed(nev):
        """K steps (each after the eviction read unless --warm); returns (events per step,
        wall ms per step)."""
        ev = [new_events(nev) for _ in range(K)]
        t0 = time.perf_counter()
        for i in range(K):
            if evict is not None:
                torch.sum(evict, dim=0, out=evict_sum)
            step(ev[i])
        torch.cuda.synchronize()
        return ev, (time.perf_counter() - t0) * 1e3 / K

    # The step: two events per step, around its whole launch sequence, so nothing is
    # recorded between its kernels. Cold: the step's own span (the eviction sits before it).
    log("timing %d steps%s" % (K, "" if args.warm else " (1 GiB read before each)"))
    ev, ms_wall = timed(2)
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    ms_step = ms_wall if args.warm else float(np.mean(step_ms))
    # The breakdown and the decode kernel's launch duration (roofline): K more steps, with an
    # event after every stage.
    log("timing %d steps with an event after every stage" % K)
    ev_st, _ = timed(len(stages) + 1)
    ms_step_staged = float(np.mean([e[0].elapsed_time(e[-1]) for e in ev_st]))
    per = {name: [e[j].elapsed_time(e[j + 1]) for e in ev_st] for j, name in enumerate(stages)}
    stage_ms = {name: round(float(np.mean(per[name])), 5) if name in per else None
                for name in ("decode_partitions", "partition_reduce", "copy_blocks",
                             "reshape_and_cache", "shared_prefix")}
    t_dec = per["decode_partitions"]
    dec_ms = float(np.mean(t_dec))
    gbps = bytes_["kv_unique"] / (ms_step * 1e-3) / 1e9
    kernel_bytes = bytes_["decode_kernel"]
    achieved = kernel_bytes / (dec_ms * 1e-3) / 1e9
    log("step %.4f ms (median %.4f; %.4f with an event after every stage), decode kernel "
        "%.4f ms (p10 %.4f, p90 %.4f); %s"
        % (ms_step, float(np.median(step_ms)), ms_step_staged, dec_ms,
           np.percentile(t_dec, 10), np.percentile(t_dec, 90),
           ", ".join("%s %.4f ms" % (k, v) for k, v in stage_ms.items()
                     if v is not None and k != "decode_partitions")))

    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(float(np.median(step_ms)), 5),
        "ms_per_step_p10_p90": [round(float(np.percentile(step_ms, 10)), 5),
                                round(float(np.percentile(step_ms, 90)), 5)],
        "ms_each_step": [round(float(x), 4) for x in step_ms],
        "timing": "wall clock over back-to-back steps (warm caches)" if args.warm else
                  ("HIP events around each step's launches (none between them), 1 GiB read "
                   "before each (cold L2 and memory-side cache); wall clock incl. the eviction "
                   "reads %.4f ms/step. kernel_ms and roofline come from %d more steps with "
                   "an event after every stage (step %.5f ms there)"
                   % (ms_wall, K, ms_step_staged)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q on the device; seeded lengths and placement)",
        "config": {"workload": case.name, "num_seqs": case.num_seqs,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": case.block_size,
                   "kv_dtype": case.dtype, "accumulate": "f32", "partition_size": part,
                   "grid": args.grid, "late_units": "static" if args.no_sched else "ticketed",
                   "ticketed_tail_shared_items_moved": moved,
                   "kv_policy": "cached" if policy == pk.KV_CACHED else "stream",
                   "pack_tokens": args.pack if args.grid in ("list", "forks") else 0,
                   "append": "fused" if fused else "separate",
                   "copy_on_write": ("fused" if fused_cow else "separate")
                   if st["pairs"] is not None else "none",
                   "prefix_tokens": case.meta.get("prefix_tokens", 0),
                   "mean_seq_len": round(float(case.seq_lens.mean()), 1),
                   "num_blocks": case.num_blocks, "parallelism": "single GPU",
                   **({"fork_groups": int(groups.shape[0]), "fork_group_size": int(groups.shape[1])}
                      if groups is not None else {}),
                   **({"named_partition_size": 512,
                       "partition_note": "the workload's definition names 512-token partitions; "
                                         "run with --partition 512 for that form (the default "
                                         "partition of the library's policy is faster)"}
                      if case.name == "long_context_splitk" and part != 512 else {})},
        "decode_tokens_per_s": round(case.num_seqs / (ms_step * 1e-3), 1),
        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "kv_unique_bytes": bytes_["kv_unique"],
        "kv_logical_bytes": bytes_["kv_logical"],
        "effective_logical_GBps": round(bytes_["kv_logical"] / (ms_step * 1e-3) / 1e9, 2),
        "kernel_ms": stage_ms,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None,
                     "kernel": "paged_decode_partition_kernel",
                     "scope": "the decode partition kernel alone, per launch; the whole "
                              "step's fraction is frac_of_hbm_peak",
                     "bytes_per_launch": kernel_bytes},
    }
    result["roofline"]["traffic"] = measured_traffic(case.name, result["config"])
    result["traffic_launch_key"] = traffic_launch_key(result["config"])
    if probe is not None:
        ach = probe_rate(probe, "stream_2GiB", "nontemporal")
        result["achievable_GBps"] = ach
        result["achievable_note"] = ("2 GiB streaming read with the KV loads' non-temporal "
                                     "cache policy, measured on this device (pkv_read_probe; "
                                     "%.1f GB/s with the default policy), beside the nominal "
                                     "%.0f GB/s peak"
                                     % (probe_rate(probe, "stream_2GiB", "default"),
                                        HBM_PEAK_GBPS))
        result["frac_of_achievable"] = round(gbps / ach, 4)
        result["read_probe"] = probe
    if args.timeline:
        if work is None or isinstance(work, tuple):
            raise SystemExit("--timeline needs the plain work list (--grid list, no --pack)")
        from paged_kv_cache_402_amd._lib import lib as _plib
        cap = case.num_kv_heads * int(work.shape[0])
        tl = torch.zeros(8 * cap, dtype=torch.int32, device=dev)
        summaries = []
        for _ in range(3):
            tl.zero_()
            if evict is not None:
                torch.sum(evict, dim=0, out=evict_sum)
            torch.cuda.synchronize()
            pk.check(_plib.pkv_debug_timeline(tl.data_ptr(), cap), "debug_timeline")
            step()
            torch.cuda.synchronize()
            pk.check(_plib.pkv_debug_timeline(None, 0), "debug_timeline")
            eb = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
            summaries.append(timeline_summary(tl.cpu().numpy().view(np.uint32), work.cpu().numpy(),
                                              case.num_kv_heads, part, case.seq_lens,
                                              case.head_dim * eb))
            log("timeline: %s" % summaries[-1])
        result_timeline = summaries
    else:
        result_timeline = None
    log("host manager cost")
    result["host_manager_us_per_step"] = round(host_manager_cost(pk, case), 1)
    if result_timeline is not None:
        result["timeline"] = result_timeline
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, about %.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(st, args.cpu_seconds, gen)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
