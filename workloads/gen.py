"""Seeded synthetic workloads for paged decode attention.

Pages cited (all three are web pages about vLLM's PagedAttention):
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)

What lives here: sequence lengths, block placement (which physical block ids a
table lists), free-list orders, and N(0,1) values rounded to a storage dtype.
What does not: any attention, softmax, slot arithmetic or cache-write logic.
Both sides of every parity test (the fp64 oracle and the HIP library) consume
the arrays made here and nothing else from each other.

Storage representation of a KV element on the host:
  "f32"  -> numpy float32
  "f16"  -> numpy float16
  "bf16" -> numpy uint16 holding the bfloat16 bit pattern
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# Seeds of the five named workloads: default_rng(402000 + index).
SEED_BASE = 402000


def storage_numpy_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 samples -> storage array (round to nearest, ties to even). Inputs are finite."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def nan_value(dtype: str):
    """A quiet NaN in storage form; used to poison slots that must never be read."""
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.uint16(0x7FC0)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) drawn in fp32, rounded to the storage dtype."""
    return round_to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


def blocks_needed(seq_len: int, block_size: int) -> int:
    return -(-int(seq_len) // int(block_size))


@dataclass
class PagedDecodeCase:
    """One decode batch over a paged pool. Arrays are host numpy in storage form."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray      # int32 [B][W], padded with -1
    scale: float                  # a float32-representable value
    q: np.ndarray | None = None   # storage [B][Hq][d]
    k_cache: np.ndarray | None = None  # storage [NB][Hkv][bs][d]
    v_cache: np.ndarray | None = None
    free_order: np.ndarray | None = None  # int32 [NB], order a block manager hands out ids
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def table_width(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes_per_token(self) -> int:
        """K and V bytes of one token over all KV heads of one layer."""
        return 2 * self.num_kv_heads * self.head_dim * elem_bytes(self.dtype)

    def unique_slots(self) -> int:
        """Distinct (physical block, offset) pairs that hold a token some sequence attends to."""
        seen = {}
        bs = self.block_size
        for b in range(self.num_seqs):
            L = int(self.seq_lens[b])
            nb = blocks_needed(L, bs)
            for j in range(nb):
                blk = int(self.block_tables[b, j])
                used = min(bs, L - j * bs)
                seen[blk] = max(seen.get(blk, 0), used)
        return int(sum(seen.values()))

    def logical_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())


def pad_tables(rows: list[list[int]], width: int) -> np.ndarray:
    t = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        if len(r) > width:
            raise ValueError("table row longer than width")
        t[i, : len(r)] = r
    return t


def used_blocks_in_order(tables: np.ndarray, seq_lens: np.ndarray, block_size: int) -> np.ndarray:
    """Distinct valid physical ids, in order of first appearance (seq-major, then logical)."""
    out, seen = [], set()
    for b in range(tables.shape[0]):
        for j in range(blocks_needed(int(seq_lens[b]), block_size)):
            blk = int(tables[b, j])
            if blk not in seen:
                seen.add(blk)
                out.append(blk)
    return np.asarray(out, dtype=np.int64)


def fill_pool(rng, num_blocks, num_kv_heads, block_size, head_dim, dtype, tables, seq_lens,
              poison=True, chunk_blocks=2048):
    """K and V pools: every block that a table uses gets N(0,1) values (drawn block by block in
    first-appearance order); unused blocks and the slots past seq_len in each sequence's last
    block hold NaN when `poison` (zero otherwise)."""
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    npdt = storage_numpy_dtype(dtype)
    fillv = nan_value(dtype) if poison else npdt(0)
    kc = np.full(shape, fillv, dtype=npdt)
    vc = np.full(shape, fillv, dtype=npdt)
    used = used_blocks_in_order(tables, seq_lens, block_size)
    for c0 in range(0, len(used), chunk_blocks):
        ids = used[c0:c0 + chunk_blocks]
        kc[ids] = normal(rng, (len(ids),) + shape[1:], dtype)
        vc[ids] = normal(rng, (len(ids),) + shape[1:], dtype)
    # poison (or zero) the unwritten tail of each sequence's private last block
    refs = {}
    for b in range(tables.shape[0]):
        for j in range(blocks_needed(int(seq_lens[b]), block_size)):
            refs[int(tables[b, j])] = refs.get(int(tables[b, j]), 0) + 1
    for b in range(tables.shape[0]):
        L = int(seq_lens[b])
        if L % block_size == 0:
            continue
        last = int(tables[b, blocks_needed(L, block_size) - 1])
        if refs[last] == 1:
            kc[last, :, L % block_size:, :] = fillv
            vc[last, :, L % block_size:, :] = fillv
    return kc, vc


def _tables_from_ids(ids: np.ndarray, lens: np.ndarray, block_size: int, width: int,
                     prefix: list[int] | None = None) -> np.ndarray:
    rows, pos = [], 0
    for L in lens:
        n = blocks_needed(int(L), block_size)
        rows.append(list(map(int, ids[pos:pos + n])))
        pos += n
    if prefix is not None:
        rows = [list(prefix) + r for r in rows]
    return pad_tables(rows, width)


def make_case(name, rng, seq_lens, num_q_heads, num_kv_heads, head_dim, block_size, dtype,
              num_blocks=None, pool_factor=1.25, width=None, scale=None, values=True, poison=True,
              fragmented=False):
    """A decode batch with private blocks drawn at random without replacement from a pool of
    ceil(pool_factor * need) blocks (or from a shuffled pool when `fragmented`)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = int(sum(blocks_needed(L, block_size) for L in seq_lens))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * need)))
    if fragmented:
        ids = rng.permutation(num_blocks)[:need]
    else:
        ids = rng.choice(num_blocks, need, replace=False)
    if width is None:
        width = max(1, max(blocks_needed(L, block_size) for L in seq_lens) if len(seq_lens) else 1)
    tables = _tables_from_ids(ids, seq_lens, block_size, width)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    case = PagedDecodeCase(name=name, dtype=dtype, num_q_heads=num_q_heads,
                           num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                           num_blocks=num_blocks, seq_lens=seq_lens, block_tables=tables,
                           scale=scale)
    if values:
        case.q = normal(rng, (len(seq_lens), num_q_heads, head_dim), dtype)
        case.k_cache, case.v_cache = fill_pool(rng, num_blocks, num_kv_heads, block_size, head_dim,
                                               dtype, tables, seq_lens, poison=poison)
    return case


# ---------------------------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------------------------

def tiny_case(pin_worked_example: bool = False, values: bool = True) -> PagedDecodeCase:
    """4 sequences of lengths {1, 15, 16, 35}, 4 query = 4 KV heads, head_dim 64, block 16, fp32,
    a pool of 32 blocks handed out in the order of a seeded permutation. With
    `pin_worked_example`, the 35-token sequence holds physical blocks 7, 3, 9 as in the worked
    block-table example (P3 §2.2.3) and the other sequences take ids from the rest."""
    rng = np.random.default_rng(SEED_BASE + 0)
    lens = np.array([1, 15, 16, 35], dtype=np.int32)
    nb_pool, bs = 32, 16
    perm = rng.permutation(nb_pool).astype(np.int32)
    if pin_worked_example:
        rest = [int(x) for x in perm if int(x) not in (7, 3, 9)]
        free_order = np.array(rest[:3] + [7, 3, 9] + rest[3:], dtype=np.int32)
    else:
        free_order = perm
    tables = _tables_from_ids(free_order, lens, bs, width=4)
    case = PagedDecodeCase(name="tiny_f32_d64_bs16", dtype="f32", num_q_heads=4, num_kv_heads=4,
                           head_dim=64, block_size=bs, num_blocks=nb_pool, seq_lens=lens,
                           block_tables=tables, scale=float(np.float32(1.0 / 8.0)),
                           free_order=free_order)
    if values:
        case.q = normal(rng, (4, 4, 64), "f32")
        case.k_cache, case.v_cache = fill_pool(rng, nb_pool, 4, bs, 64, "f32", tables, lens)
        # one new token per sequence for the cache-write step
        case.meta["k_new"] = normal(rng, (4, 4, 64), "f32")
        case.meta["v_new"] = normal(rng, (4, 4, 64), "f32")
        case.meta["q_next"] = normal(rng, (4, 4, 64), "f32")
    return case


def llama2_7b_mha_case(num_seqs: int = 64, values: bool = True, poison: bool = True,
                       max_len: int = 2048) -> PagedDecodeCase:
    """Batch 64, 32 heads MHA, head_dim 128, block 16, bf16; seq_lens uniform on [128, 2048];
    blocks drawn without replacement from a pool of 1.25x the total need."""
    rng = np.random.default_rng(SEED_BASE + 1)
    lens = rng.integers(128, max_len + 1, size=num_seqs).astype(np.int32)
    return make_case("llama2_7b_mha_b%d_bf16" % num_seqs, rng, lens, 32, 32, 128, 16, "bf16",
                     width=max_len // 16, values=values, poison=poison)


def llama3_8b_gqa_prefix_case(num_seqs: int = 256, values: bool = True, poison: bool = True,
                              prefix_tokens: int = 512, max_suffix: int = 3584) -> PagedDecodeCase:
    """Batch 256, 32 query / 8 KV heads, head_dim 128, block 16, bf16. Every sequence starts with
    the same 512-token system prefix (32 physical blocks listed by every table), then a private
    suffix of uniform length on [64, 3584]. Pool = 1.25x the total need."""
    rng = np.random.default_rng(SEED_BASE + 2)
    bs = 16
    suffix = rng.integers(64, max_suffix + 1, size=num_seqs).astype(np.int32)
    npre = prefix_tokens // bs
    need = npre + int(sum(blocks_needed(s, bs) for s in suffix))
    num_blocks = int(math.ceil(1.25 * need))
    ids = rng.choice(num_blocks, need, replace=False)
    prefix = list(map(int, ids[:npre]))
    width = (prefix_tokens + max_suffix + bs - 1) // bs
    tables = _tables_from_ids(ids[npre:], suffix, bs, width, prefix=prefix)
    lens = (suffix + prefix_tokens).astype(np.int32)
    case = PagedDecodeCase(name="llama3_8b_gqa_prefix_b%d_bf16" % num_seqs, dtype="bf16",
                           num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=bs,
                           num_blocks=num_blocks, seq_lens=lens, block_tables=tables,
                           scale=float(np.float32(1.0 / math.sqrt(128))),
                           meta={"prefix_blocks": prefix, "prefix_tokens": prefix_tokens})
    if values:
        case.q = normal(rng, (num_seqs, 32, 128), "bf16")
        case.k_cache, case.v_cache = fill_pool(rng, num_blocks, 8, bs, 128, "bf16", tables, lens,
                                               poison=poison)
    return case


@dataclass
class ForkedSamplingCase:
    """Parallel sampling: `groups` prompts, each decoded by `branches` sequences that share the
    prompt's blocks. Holds only inputs; the block manager decides tables, slots and copies."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    branches: int
    decode_lens: np.ndarray      # int32 [groups]; length passed to decode (prompt + 1 new token)
    prompt_k: list               # per group: storage [L-1][Hkv][d]
    prompt_v: list
    new_k: np.ndarray            # storage [groups*branches][Hkv][d]
    new_v: np.ndarray
    q: np.ndarray                # storage [groups*branches][Hq][d]
    free_order: np.ndarray       # int32 [NB]
    table_width: int
    scale: float

    @property
    def num_seqs(self) -> int:
        return int(self.decode_lens.shape[0]) * self.branches


def llama13b_longtail_case(groups: int = 32, branches: int = 4, values: bool = True,
                           mean_len: int = 200, max_len: int = 2048) -> ForkedSamplingCase:
    """Batch 128 = 32 prompts x 4 branches, 40 heads MHA, head_dim 128, block 32, fp16. Decode
    lengths are geometric with mean 200 on {1, 2, ...}, clipped to [1, 2048]. Each branch shares
    the prompt (the first L-1 tokens) and appends its own token at position L-1."""
    rng = np.random.default_rng(SEED_BASE + 3)
    bs, H, d = 32, 40, 128
    lens = np.clip(rng.geometric(1.0 / mean_len, size=groups), 1, max_len).astype(np.int32)
    # upper bound of blocks held after the step: prompt blocks + one private block per branch
    bound = int(sum(blocks_needed(int(L) - 1, bs) + branches for L in lens))
    num_blocks = int(math.ceil(1.25 * bound))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    pk, pv = [], []
    nk = nv = q = None
    if values:
        for L in lens:
            pk.append(normal(rng, (int(L) - 1, H, d), "f16"))
            pv.append(normal(rng, (int(L) - 1, H, d), "f16"))
        n = groups * branches
        nk = normal(rng, (n, H, d), "f16")
        nv = normal(rng, (n, H, d), "f16")
        q = normal(rng, (n, H, d), "f16")
    return ForkedSamplingCase(name="llama13b_longtail_%dx%d_f16" % (groups, branches), dtype="f16",
                              num_q_heads=H, num_kv_heads=H, head_dim=d, block_size=bs,
                              num_blocks=num_blocks, branches=branches, decode_lens=lens,
                              prompt_k=pk, prompt_v=pv, new_k=nk, new_v=nv, q=q,
                              free_order=free_order, table_width=max_len // bs,
                              scale=float(np.float32(1.0 / math.sqrt(d))))


def llama13b_fork_long_case(values: bool = True) -> ForkedSamplingCase:
    """The long-tail shape (32 prompts x 4 branches, 40 MHA heads, head_dim 128, block 32, fp16)
    over long prompts: decode lengths geometric with mean 2000, clipped to [1, 8192] (parallel
    sampling over a document-length prompt, where the shared prompt dominates the bytes)."""
    c = llama13b_longtail_case(values=values, mean_len=2000, max_len=8192)
    c.name = "llama13b_fork_long_32x4_f16"
    return c


def long_context_splitk_case(num_seqs: int = 16, values: bool = True, poison: bool = True,
                             min_len: int = 32768, max_len: int = 131072) -> PagedDecodeCase:
    """Batch 16, 64 query / 8 KV heads, head_dim 128, block 64, bf16; seq_lens uniform on
    [32768, 131072]; blocks taken from a shuffled pool of 1.25x the total need."""
    rng = np.random.default_rng(SEED_BASE + 4)
    lens = rng.integers(min_len, max_len + 1, size=num_seqs).astype(np.int32)
    return make_case("long_context_gqa_b%d_bf16" % num_seqs, rng, lens, 64, 8, 128, 64, "bf16",
                     width=max_len // 64, fragmented=True, values=values, poison=poison)


def llama3_8b_long_shared_prefix_case(num_seqs: int = 256, values: bool = True,
                                      poison: bool = True) -> PagedDecodeCase:
    """The GQA 8B shape with a long shared context (a 4096-token document every request
    reads, as in retrieval over one document: P1 §8.3) and short private suffixes, uniform on
    [64, 512]. Same seed and layout rules as llama3_8b_gqa_prefix_case."""
    case = llama3_8b_gqa_prefix_case(num_seqs, values, poison, prefix_tokens=4096,
                                     max_suffix=512)
    case.name = "llama3_8b_long_shared_prefix_b%d_bf16" % num_seqs
    return case


def llama3_8b_short_batch_case(num_seqs: int = 2048, values: bool = True, poison: bool = True,
                               max_len: int = 48) -> PagedDecodeCase:
    """The GQA 8B shape (32 query / 8 KV heads, head_dim 128, block 16, bf16) on a large batch
    of short sequences, lengths uniform on [1, 48]: the early decode steps of many requests
    with short prompts, where every partition is short and the launch is bound by latency.
    Private blocks from a pool of 1.25x the need."""
    rng = np.random.default_rng(SEED_BASE + 6)
    lens = rng.integers(1, max_len + 1, size=num_seqs).astype(np.int32)
    return make_case("llama3_8b_short_batch_b%d_bf16" % num_seqs, rng, lens, 32, 8, 128, 16,
                     "bf16", width=-(-max_len // 16), values=values, poison=poison)


WORKLOADS = {
    "tiny": tiny_case,
    "llama3_8b_short_batch": llama3_8b_short_batch_case,
    "llama3_8b_long_shared_prefix": llama3_8b_long_shared_prefix_case,
    "llama2_7b_mha": llama2_7b_mha_case,
    "llama3_8b_gqa_prefix": llama3_8b_gqa_prefix_case,
    "llama13b_longtail": llama13b_longtail_case,
    "long_context_splitk": long_context_splitk_case,
}


# ---------------------------------------------------------------------------------------------
# Device-side value synthesis (for full-size runs where numpy generation would dominate)
# ---------------------------------------------------------------------------------------------

def device_normal(shape, dtype: str, seed: int, device):
    """N(0,1) in fp32 from torch's seeded device generator, rounded to the storage dtype by
    torch's conversion (round to nearest even). Returns a torch tensor of the storage dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return x.to(tdt)
