/*
 * pagedkv.h — C ABI of libpagedkv.so: decode attention over a paged KV cache on MI355X
 * (gfx950), the cache-write and block-copy kernels it relies on, and a host block manager.
 *
 * Pages cited (all three describe vLLM's PagedAttention):
 *   P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
 *   P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
 *   P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)
 *
 * ------------------------------------------------------------------------------------------
 * Conventions shared by every call
 * ------------------------------------------------------------------------------------------
 *  - Every call returns an int status (PKV_OK or a negative PKV_E* code) and never throws.
 *    pkv_last_error() returns a thread-local message describing the last failure.
 *  - Device calls take device pointers owned by the caller, enqueue work on `stream`
 *    (a hipStream_t; NULL = the null stream) and never synchronise. Shapes, dtypes and
 *    alignment are checked on the host before any launch (PKV_EINVAL / PKV_EDTYPE); launch
 *    failures return PKV_EHIP.
 *  - The contents of device index arrays (table entries, seq_lens, slots, pairs) are not
 *    checked on the host (that would need a device->host copy). Every kernel bounds-checks
 *    them on the device instead and skips an out-of-range entry (a table entry outside
 *    [0, num_blocks), a slot outside [0, num_blocks*block_size), a pair outside the pool), so
 *    bad indices never address memory outside the caller's buffers. Results for such inputs
 *    are unspecified.
 *  - The library allocates no device memory. Split-K partials live in a caller-provided
 *    workspace of pkv_decode_workspace_bytes() bytes.
 *  - Data types: PKV_F32 (IEEE binary32), PKV_F16 (IEEE binary16), PKV_BF16 (bfloat16).
 *    All arithmetic is fp32; conversion to a 16-bit output rounds to nearest, ties to even.
 *
 * ------------------------------------------------------------------------------------------
 * KV pool layout (P1 §4.1; P2 §2.1; P3 §2.2.2: fixed-size blocks, 16 tokens by default)
 * ------------------------------------------------------------------------------------------
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim], row-major, separate
 *                      buffers of the same dtype. The tile of one (block, KV head) is
 *                      block_size*head_dim*elem_bytes contiguous bytes (4 KiB for block 16,
 *                      head_dim 128, bf16), so one token row is head_dim*elem_bytes contiguous
 *                      bytes that lanes read as 16-byte vectors.
 *   slot s           : physical block s / block_size, offset s % block_size (P3 §2.2.3).
 *   block_tables     : int32 [num_seqs][max_blocks_per_seq]; entry [b][j] is the physical
 *                      block holding tokens j*block_size .. (j+1)*block_size-1 of sequence b
 *                      (P1 §4.2; P3 §2.2.3). Entries at j >= ceil(seq_len/block_size) are
 *                      never read (padding, -1 by convention). Several rows may list the same
 *                      physical block (prefix sharing, P1 §6.1; P3 §2.2.3).
 *   seq_lens         : int32 [num_seqs]; tokens cached for each sequence, including the token
 *                      written by this step's pkv_reshape_and_cache. Values above
 *                      max_blocks_per_seq*block_size are clamped to it; negatives act as 0.
 * Limits: head_dim in {64, 128, 256}; block_size a power of two in [8, 256];
 *         num_q_heads / num_kv_heads in {1, 2, 4, 8}; num_blocks*block_size < 2^31;
 *         head_dim*elem_bytes a multiple of 128; 16-byte aligned q/out/caches.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,      /* bad shape, size, pointer or argument */
  PKV_EDTYPE = -2,      /* unsupported dtype combination */
  PKV_ENOBLOCKS = -3,   /* block manager: the fixed pool cannot meet the request */
  PKV_EHIP = -4,        /* a HIP launch or runtime call failed */
  PKV_ENOSEQ = -5,      /* block manager: unknown sequence id */
  PKV_EWORKSPACE = -6   /* workspace missing or smaller than pkv_decode_workspace_bytes() */
};

/* Library version (major*10000 + minor*100 + patch). */
int pkv_version(void);

/* Thread-local text of the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

/* ==========================================================================================
 * Device operations
 * ========================================================================================== */

/* Bytes of split-K workspace pkv_paged_attention_decode needs: a 256-byte header (its first
 * 8 bytes are the scheduling word below), then for every (sequence, query head, context
 * partition) one running max and one exponent sum (fp32 pairs, their area padded to a
 * multiple of 16 bytes), then one head_dim-long fp32 accumulator. partition_size defaults to
 * 512 when 0 is passed. Returns 0 on bad input or when no sequence can span two partitions. */
size_t pkv_decode_workspace_bytes(int num_seqs, int num_q_heads, int max_blocks_per_seq,
                                  int block_size, int head_dim, int partition_size);

/* Initialises a workspace's scheduling word (one tiny kernel on stream; no allocation, no
 * memset). Optional: the per-partition pass over a work list (the _list, _append, _step and
 * _shared entry points) then hands the work units of its last workgroups (half as many as
 * are resident at once) out in the list's order from that word, one atomic per workgroup, so
 * the last, short partitions go to whichever XCD has room instead of a fixed eighth of them to
 * each; the output is bitwise the same either way. Each call leaves the word initialised, so
 * once per workspace (for instance right after allocating it) is enough. A workspace that was
 * never initialised works too, with the fixed assignment. Calls sharing a workspace must not
 * overlap in time (already required by the partials). A workspace_bytes of 0 is a no-op. */
int pkv_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Cache policy of a decode launch's KV reads (a gfx950 matter; no page defines it). Every KV
 * row of a sequence is read once per launch, so by default the reads are non-temporal
 * (PKV_KV_STREAM: global_load ... nt), which reads HBM about 12% faster. Blocks that several
 * sequences of the batch list (P1 §6.1-6.2; P3 §2.2.8: forks of parallel sampling and beam
 * search, a common prompt prefix) are read again by other workgroups of the same launch;
 * where such repeats are most of the reads, the default policy (PKV_KV_CACHED) keeps those
 * lines in L2 for them and is faster. */
enum { PKV_KV_STREAM = 0, PKV_KV_CACHED = 1 };

/* The policy for one launch, from host copies of its block tables ([num_seqs]
 * [max_blocks_per_seq]) and seq_lens: PKV_KV_CACHED when at least half of the launch's block
 * reads repeat a block another read already names, i.e. reads >= 2 x distinct blocks; else
 * PKV_KV_STREAM. The reads are the in-pool table entries of the tokens the launch attends
 * (lengths clamped to the table): every token of every sequence with work_list NULL, else
 * those of the partitions (of partition_size tokens, a multiple of block_size) that the host
 * list's list_len entries name: a list from pkv_decode_work_list, all of a packed list from
 * pkv_decode_work_list_packed (its packed-row entries are skipped, the items they point at are
 * counted where they stand), or the list of pkv_decode_plan_shared_prefix, which leaves the
 * shared partitions to the shared-prefix pass. O(reads + num_blocks) on the host; negative on
 * bad arguments. */
int pkv_decode_kv_policy(const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                         int max_blocks_per_seq, int block_size, int num_blocks,
                         const int32_t* work_list, int list_len, int partition_size);

/* Decode attention over the paged cache (P1 §4.2; P2 §3.1; P3 §2.2.4: the kernel reads
 * KV block by block through the block table).
 *   out[b][h][:] = sum_t softmax_t(scale * q[b][h].k_t) v_t
 * over the seq_lens[b] cached tokens t of sequence b, where k_t and v_t are row t % block_size
 * of KV head h / (num_q_heads/num_kv_heads) in physical block block_tables[b][t / block_size].
 * A sequence of length 0 produces a zero row.
 *   out          : [num_seqs][num_q_heads][head_dim] of out_dtype (kv_dtype or PKV_F32)
 *   q            : [num_seqs][num_q_heads][head_dim] of kv_dtype
 *   scale        : softmax scale (usually 1/sqrt(head_dim))
 *   partition_size: tokens per context partition (split-K); a multiple of 32 and of
 *                  block_size in [32, 2048]; 0 selects 512. Sequences longer than one
 *                  partition are finished by a second, deterministic merge pass.
 *   workspace    : 16-byte aligned device buffer of at least pkv_decode_workspace_bytes()
 *                  bytes (else PKV_EWORKSPACE, or PKV_EINVAL if misaligned); may be NULL
 *                  only if workspace_bytes is 0 and no sequence can span two partitions
 *                  (max_blocks_per_seq*block_size <= partition_size). Calls that share a
 *                  workspace must not overlap in time (enqueue them on one stream).
 *   kv_policy    : cache policy of the KV reads (PKV_KV_STREAM or PKV_KV_CACHED, else
 *                  PKV_EINVAL); it changes speed only, never a bit of the output.
 *                  pkv_decode_kv_policy picks it from the block tables.
 * Two launches: per-partition attention, then (when some sequence spans two partitions) a
 * deterministic merge of the partitions' partials.
 * The output is a deterministic function of the inputs: it does not depend on where the
 * blocks sit in the pool, nor on which other sequences share them. */
int pkv_paged_attention_decode(void* out, int out_dtype, const void* q, const void* k_cache,
                               const void* v_cache, int kv_dtype, const int32_t* block_tables,
                               const int32_t* seq_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, float scale, int partition_size,
                               void* workspace, size_t workspace_bytes,
                               int kv_policy, void* stream);

/* pkv_paged_attention_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same two launches
 * and bitwise the same output, with the split-K partials in the library's own fixed scratch
 * area (64 MiB, a file-scope device array; each GPU the library runs on holds one until the
 * process ends) instead of a caller workspace. Nothing is allocated, by the library or
 * anyone: the area's address on the current device is looked up once (hipGetSymbolAddress)
 * at the first call on that device. Shapes whose partials need more than 64 MiB
 * (pkv_decode_workspace_bytes > 64 MiB) fail with PKV_EWORKSPACE and launch nothing. Every
 * call on one GPU uses the same area and nothing in it needs clearing (every partial the merge
 * reads is written first by the same call), so calls on one GPU must not overlap in time:
 * calls on different streams, or from different threads, without ordering between them
 * race. */
int pkv_paged_attention_decode_noalloc(void* out, int out_dtype, const void* q,
                                       const void* k_cache, const void* v_cache, int kv_dtype,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks,
                                       int max_blocks_per_seq, float scale, int partition_size,
                                       int kv_policy, void* stream);

/* The two launches of pkv_paged_attention_decode, exposed separately so a caller can time or
 * schedule them apart. Same arguments and results as the combined call:
 *   _partitions: one workgroup per (KV head, sequence, partition) attends over its partition;
 *                single-partition sequences get their final row in `out`, others leave
 *                (max, sum, accumulator) partials in the workspace.
 *   _reduce    : for sequences with more than one partition, merges the partials in
 *                partition order into `out`. */
int pkv_paged_attention_partitions(void* out, int out_dtype, const void* q, const void* k_cache,
                                   const void* v_cache, int kv_dtype,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int num_blocks, int max_blocks_per_seq,
                                   float scale, int partition_size, void* workspace,
                                   size_t workspace_bytes, int kv_policy, void* stream);
int pkv_paged_attention_reduce(void* out, int out_dtype, const int32_t* seq_lens, int num_seqs,
                               int num_q_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int partition_size,
                               const void* workspace, size_t workspace_bytes, void* stream);

/* A partition size for these shapes: the longest multiple of 256 tokens up to 2048 (and a
 * multiple of block_size) whose workgroup takes at most its share of a compute unit's LDS at
 * the occupancy the kernel's registers allow (40 KiB, four per compute unit, up to 4 query
 * heads per KV head; 53 KiB, three, at 8) and that still gives at least 1024 workgroups if
 * every sequence were as long as its table allows (256 otherwise). Longer partitions mean
 * fewer workgroups, less fixed cost per token and fewer partials to merge; the floor keeps
 * small batches spread over the machine. Negative on bad arguments. */
int pkv_decode_default_partition(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq);

/* Work list of the per-partition pass, built on the host from host seq_lens: one item per
 * (sequence b, context partition p) that holds tokens, item = (b << 16) | p as int32 bits
 * (a length-0 sequence has one item, p = 0, that writes its zero row). Lengths are clamped
 * to [0, max_blocks_per_seq * block_size] as the kernel clamps them. Order: the full
 * partitions in (sequence, partition) order, then every sequence's last, shorter partition,
 * longest first. num_seqs is at most 32767 (an item's top bit stays clear). With work_list
 * NULL returns the item count; otherwise writes the items (capacity >= count, else
 * PKV_EINVAL) and returns the count. Negative on bad arguments. */
int pkv_decode_work_list(const int32_t* seq_lens, int num_seqs, int max_blocks_per_seq,
                         int block_size, int partition_size, int32_t* work_list, int capacity);

/* The same list with its short partitions packed: items of at most pack_tokens tokens
 * (0 < pack_tokens <= partition_size / 4; 0 packs nothing) are taken four at a time by one
 * workgroup, one wave each, for the same KV head, instead of one workgroup each. A serving
 * mix of many short sequences then needs a quarter of the workgroups for them; each is latency
 * bound (a chain of dependent loads), so the launch shortens. Layout: *rows entries first,
 * each a plain item or a packed row 0x80000000 | idx naming the four items stored at
 * idx .. idx + 3 further on in the list (a last, partial group is padded with items naming
 * sequence 0xFFFF, which every launch skips). The short items are grouped in the plain list's
 * order (longest first); the rows run in decreasing order of the tokens one wave of the row
 * takes: a plain item's tokens / 4 rounded up, a packed row's longest item (ties in list
 * order, plain rows first), so the rows that take longest start first. Pass the whole list
 * and work_items = *rows to the _list and _append entry points. A packed wave computes its
 * partition alone, so those outputs equal the four-wave ones up to fp32 rounding order, not
 * bitwise. Returns the list length (with work_list NULL: a size query, *rows still set);
 * negative on bad arguments. */
int pkv_decode_work_list_packed(const int32_t* seq_lens, int num_seqs, int max_blocks_per_seq,
                                int block_size, int partition_size, int pack_tokens,
                                int32_t* work_list, int capacity, int* rows);

/* Kinds of per-partition launch, for pkv_decode_ticketed_items: the _list, _append, _shared
 * and plain entry points (PKV_LAUNCH_PLAIN), those with copy-on-write sources, the _step
 * entry points (PKV_LAUNCH_COPY_ON_WRITE), and the fork-group step (PKV_LAUNCH_FORK_GROUPS). */
enum { PKV_LAUNCH_PLAIN = 0, PKV_LAUNCH_COPY_ON_WRITE = 1, PKV_LAUNCH_FORK_GROUPS = 2 };

/* How many items at the end of a work list of list_len items a launch with an initialised
 * workspace (pkv_decode_workspace_init) hands out by ticket on the current device: the units
 * of its last workgroups, half as many as are resident at once (or those past the first
 * machine-full when there are fewer), rounded up to whole items (an item is num_kv_heads
 * units). The sizes and dtypes are the launch's; group_size is the
 * fork groups' size for PKV_LAUNCH_FORK_GROUPS and ignored otherwise. Queries the occupancy
 * of the kernel such a launch picks (no launch; PKV_EHIP without a usable device). Returns the
 * count (0: nothing is ticketed, as when the list holds no more units than fit at once),
 * negative on bad arguments. (A gfx950 scheduling matter; no page defines it.) */
int pkv_decode_ticketed_items(int kv_dtype, int head_dim, int num_q_heads, int num_kv_heads,
                              int block_size, int partition_size, int list_len, int launch_kind,
                              int group_size);

/* Reorders a host work list from pkv_decode_work_list (not a packed one) in place, so that the
 * items a launch hands out by ticket read no block that another item of the list reads too.
 * A ticketed unit runs on whichever XCD has room, where the blocks its sequence shares with
 * others (a common prompt prefix, P1 §6.1; P3 §2.2.8) are not in that XCD's L2, and are read
 * from HBM again; a unit that keeps its place keeps its KV head's XCD, where they are. An item
 * is shared when one of the in-pool blocks its tokens read (lengths clamped as the kernel
 * clamps them) is read by the list more than once. If any of the last tail_items items (from
 * pkv_decode_ticketed_items) is shared, the list's last tail_items private items move to its
 * end, keeping their order, and every other item keeps its order before them; the walk back
 * for private items stops at the first one over 5/4 of the longest item of the old tail, so the
 * end of the launch does not grow much longer (a long item placed last lengthens its drain by
 * more than the re-reads save); when no private item from before the tail qualifies, the list
 * stays as it is. Outputs are bitwise the same in any item order. Returns how many shared
 * items left the tail (0: the list is unchanged), negative on bad arguments
 * (items naming a sequence >= num_seqs or a packed row). O(reads + list_len) on the host. */
int pkv_decode_work_list_private_tail(const int32_t* block_tables, const int32_t* seq_lens,
                                      int num_seqs, int max_blocks_per_seq, int block_size,
                                      int num_blocks, int partition_size, int tail_items,
                                      int32_t* work_list, int list_len);

/* pkv_paged_attention_decode / _partitions with the per-partition pass launched over a work
 * list (device int32, from pkv_decode_work_list, or pkv_decode_work_list_packed with
 * work_items its rows) instead of the full (partition, sequence) grid: one workgroup per
 * (KV head, row), so no workgroup is spent on partitions past a sequence's end, and the short
 * last partitions run at the end of the launch. num_seqs is at most 32767. The list must hold
 * every partition of every sequence exactly once (the merge pass reads all of them); items
 * naming a sequence >= num_seqs or a partition past the sequence's end are skipped. Every
 * partition of a plain list computes exactly what it computes in the full-grid launch, so the
 * output is bitwise the same. */
int pkv_paged_attention_decode_list(void* out, int out_dtype, const void* q, const void* k_cache,
                                    const void* v_cache, int kv_dtype,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, int max_blocks_per_seq,
                                    float scale, int partition_size, const int32_t* work_list,
                                    int work_items, void* workspace, size_t workspace_bytes,
                                    int kv_policy, void* stream);
int pkv_paged_attention_partitions_list(void* out, int out_dtype, const void* q,
                                        const void* k_cache, const void* v_cache, int kv_dtype,
                                        const int32_t* block_tables, const int32_t* seq_lens,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, int num_blocks,
                                        int max_blocks_per_seq, float scale, int partition_size,
                                        const int32_t* work_list, int work_items, void* workspace,
                                        size_t workspace_bytes, int kv_policy, void* stream);

/* Decode with the cache write of the step's new tokens fused in (P1 §4.3; P3 §2.2.3: the
 * newest token's K/V are stored into the block the table gives, then attended to): k_new and
 * v_new ([num_seqs][num_kv_heads][head_dim] of kv_dtype, device) hold the K and V rows of
 * token seq_lens[b] - 1 of every sequence b with seq_lens[b] > 0. The per-partition pass
 * reads that token's rows from k_new / v_new and stores them into k_cache / v_cache at the
 * slot the block table gives (block table[b][(L-1)/block_size], offset (L-1)%block_size),
 * so the caches end as pkv_reshape_and_cache with those slots would leave them and the output
 * is bitwise that of pkv_reshape_and_cache followed by the unfused decode. The slot's block
 * must be held by sequence b alone (the block manager's append gives that); a table entry
 * outside the pool skips the store and the token. work_list may be NULL (work_items 0) for
 * the full grid, or a list from pkv_decode_work_list. */
int pkv_paged_attention_decode_append(void* out, int out_dtype, const void* q, const void* k_new,
                                      const void* v_new, void* k_cache, void* v_cache,
                                      int kv_dtype, const int32_t* block_tables,
                                      const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int num_blocks, int max_blocks_per_seq, float scale,
                                      int partition_size, const int32_t* work_list,
                                      int work_items, void* workspace, size_t workspace_bytes,
                                      int kv_policy, void* stream);
/* Its per-partition pass alone (the merge is pkv_paged_attention_reduce). */
int pkv_paged_attention_partitions_append(void* out, int out_dtype, const void* q,
                                          const void* k_new, const void* v_new, void* k_cache,
                                          void* v_cache, int kv_dtype,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_dim, int block_size, int num_blocks,
                                          int max_blocks_per_seq, float scale,
                                          int partition_size, const int32_t* work_list,
                                          int work_items, void* workspace,
                                          size_t workspace_bytes, int kv_policy, void* stream);

/* One decode step in one pass (P1 §6.2, §4.3; P2 §2.2): the copy-on-write of each sequence's
 * last block, the cache write of its new token and the attention. cow_src (device int32
 * [num_seqs]) names, for each sequence whose last block the block manager has just made a
 * private copy of (pkv_bm_append_slot returned 1), the block it copied from (cow_src of that
 * call; the table already lists the copy), and -1 for the others; entries outside the pool
 * are ignored. For such a sequence the pass reads the earlier tokens of that block from the
 * source, and the workgroup of each KV head stores every such row it reads into the
 * sequence's last block as it uses it, so the copy costs no loads of its own; the new token's
 * row comes from k_new / v_new. The output, and every cache row a sequence holds, are bitwise
 * those of pkv_copy_blocks, then pkv_reshape_and_cache, then the decode; the copied block's
 * rows past the new token (no token of the sequence is there yet; its next appends write them)
 * keep what they held, where pkv_copy_blocks would have copied the source's. Precondition
 * (what a fork gives): in this launch the source block is written only at that same
 * new-token row, by the sequence that kept it. Otherwise as
 * pkv_paged_attention_decode_append. */
int pkv_paged_attention_decode_step(void* out, int out_dtype, const void* q, const void* k_new,
                                    const void* v_new, const int32_t* cow_src, void* k_cache,
                                    void* v_cache, int kv_dtype, const int32_t* block_tables,
                                    const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int max_blocks_per_seq, float scale,
                                    int partition_size, const int32_t* work_list, int work_items,
                                    void* workspace, size_t workspace_bytes,
                                    int kv_policy, void* stream);
/* Its per-partition pass alone (the merge is pkv_paged_attention_reduce). */
int pkv_paged_attention_partitions_step(void* out, int out_dtype, const void* q,
                                        const void* k_new, const void* v_new,
                                        const int32_t* cow_src, void* k_cache, void* v_cache,
                                        int kv_dtype, const int32_t* block_tables,
                                        const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, int max_blocks_per_seq, float scale,
                                        int partition_size, const int32_t* work_list,
                                        int work_items, void* workspace, size_t workspace_bytes,
                                        int kv_policy, void* stream);

/* ------------------------------------------------------------------------------------------
 * Fork groups (P2 §2.2: the branches of a parallel-sampling fork share their prompt's blocks
 * until each writes its own token; P1 §6.2 copy-on-write). Right after a fork, every branch
 * attends to the same tokens before its own new one. A fork group lists such sequences: the
 * same length, the same table entries before the new token's block, and, for the earlier rows
 * of that block, the same block to read them from (the block the copies were made from, or
 * the block itself for the branch that kept it). The step then reads those tokens once per
 * group and KV head, for every member's query heads at once, instead of once per member.
 * ------------------------------------------------------------------------------------------ */

/* Host planner, from host copies of the tables, lengths and copy sources (cow_src may be NULL:
 * no copies): the runs of sequences with equal keys (length; table entries before the new
 * token's block; the block the new token's block reads its earlier rows from, which is
 * cow_src[b] when it names a pool block, else the table's entry, and none when the new token
 * opens its block), in increasing sequence order, cut into groups of at most group_size.
 * groups (capacity x group_size int32) receives them, -1 filling a short group, and
 * group_lens (capacity int32) their length; the groups are ordered by their first member. A
 * sequence of length 0 is a group of its own. With groups and group_lens NULL returns the
 * group count; otherwise writes them (capacity >= count, else PKV_EINVAL) and returns the
 * count. Negative on bad arguments. The work list over the groups is pkv_decode_work_list
 * (or _packed) of group_lens. */
int pkv_decode_plan_fork_groups(const int32_t* block_tables, const int32_t* seq_lens,
                                const int32_t* cow_src, int num_seqs, int max_blocks_per_seq,
                                int block_size, int num_blocks, int group_size, int32_t* groups,
                                int32_t* group_lens, int capacity);

/* pkv_paged_attention_decode_step over fork groups: groups (device int32
 * [num_groups][group_size], from pkv_decode_plan_fork_groups or a caller that knows its forks;
 * -1 marks an empty place) and a work list whose items name groups (pkv_decode_work_list or
 * _packed of the groups' lengths; required). group_size x (num_q_heads / num_kv_heads) must be
 * 1, 2, 4 or 8 (8 only up to head_dim 128). Each workgroup reads the group's shared tokens
 * through its first member's table, scores them against every member's query heads, adds
 * each member's own new token from k_new / v_new, stores each member's new K and V rows into
 * its own block, and stores the earlier rows of the new token's block into the copy of every
 * member whose cow_src names a source (cow_src may be NULL: no copies). Outputs, and every
 * cache row a sequence holds, are those of pkv_paged_attention_decode_step on the same
 * arguments: the cache rows bitwise, the outputs up to fp32 rounding order (the own token is
 * added after the shared ones). The per-partition pass writes nothing for sequences in no
 * group, but the merge that decode_step_groups runs afterwards covers every sequence longer
 * than one partition: list every such sequence in a group (the planner's groups hold every
 * sequence). num_seqs and num_groups are at most 32767. A group's workgroup does the
 * arithmetic of all its rows at the occupancy of a kernel with that many rows: it pays where
 * the shared tokens dominate the bytes (forks of prompts of thousands of tokens: 1.5x faster
 * measured), not for short prompts, whose per-sequence step is bound by load latency rather
 * than bytes (there it measured slower). kv_policy as for the other entry points; to pick it
 * with pkv_decode_kv_policy, pass the groups' first members' table rows, the groups' lengths
 * and the list over the groups (the reads the launch makes). */
int pkv_paged_attention_decode_step_groups(
    void* out, int out_dtype, const void* q, const void* k_new, const void* v_new,
    const int32_t* cow_src, void* k_cache, void* v_cache, int kv_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
    float scale, int partition_size, const int32_t* groups, int num_groups, int group_size,
    const int32_t* work_list, int work_items, void* workspace, size_t workspace_bytes,
    int kv_policy, void* stream);
/* Its per-partition pass alone (the merge is pkv_paged_attention_reduce). */
int pkv_paged_attention_partitions_step_groups(
    void* out, int out_dtype, const void* q, const void* k_new, const void* v_new,
    const int32_t* cow_src, void* k_cache, void* v_cache, int kv_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
    float scale, int partition_size, const int32_t* groups, int num_groups, int group_size,
    const int32_t* work_list, int work_items, void* workspace, size_t workspace_bytes,
    int kv_policy, void* stream);

/* ------------------------------------------------------------------------------------------
 * Shared-prefix decode (P1 §6.1; P3 §2.2.3, §2.2.8: sequences that start with the same
 * prompt list the same physical blocks). The leading partitions that a group of sequences
 * shares are attended once per (KV head, partition) for all the group's query rows, as
 * matrix-core products, instead of once per sequence; the sequences' own partitions run in
 * the per-partition pass over a work list that leaves the shared ones out, and the merge pass
 * combines both. The result equals pkv_paged_attention_decode's up to fp32 rounding (the
 * shared part sums in another order), not bit for bit.
 * ------------------------------------------------------------------------------------------ */

/* Host planner, from host copies of the tables and lengths (same layout as the decode
 * arguments). Candidates are the sequences longer than one partition; they are grouped by
 * the block ids of their first partition and the largest group is taken (ties: the group
 * holding the lowest sequence index), if it has at least max(2, min_members) sequences.
 * prefix_partitions = the number of leading partitions every member lists identically and
 * that leave every member at least one token after them. members (capacity num_seqs)
 * receives the group in increasing sequence order, *num_members its size (0 and
 * *prefix_partitions 0 when no group qualifies). work_list / capacity / return value as in
 * pkv_decode_work_list, without the members' shared partitions. */
int pkv_decode_plan_shared_prefix(const int32_t* block_tables, const int32_t* seq_lens,
                                  int num_seqs, int max_blocks_per_seq, int block_size,
                                  int partition_size, int min_members, int32_t* members,
                                  int* num_members, int* prefix_partitions, int32_t* work_list,
                                  int capacity);

/* All three passes: shared-prefix pass (if num_members and prefix_partitions are > 0), the
 * per-partition pass over work_list, the merge. members (device int32 [num_members]) and
 * prefix_partitions come from pkv_decode_plan_shared_prefix, or from a caller that knows
 * the sharing (the block manager's forks and shared prefixes): every member must list the
 * first member's block ids in its first prefix_partitions * partition_size / block_size
 * table entries, and work_list must hold every other partition of every sequence (those of
 * non-members, and the members' partitions past the shared ones) exactly once. Each member
 * attends only to its own seq_lens[b] tokens, so a member may end inside the shared
 * partitions (the planner never picks one); one that fits a single partition gets its output
 * row from the shared-prefix pass itself. Table entries outside the pool are left out with
 * their tokens, as in the per-partition pass. The shared-prefix pass needs fp16 or bf16 KV,
 * head_dim 128 and partition_size / block_size <= 256 (else PKV_EINVAL); the workspace is
 * the one pkv_decode_workspace_bytes sizes. Members naming a sequence outside the batch are
 * skipped. */
int pkv_paged_attention_decode_shared(void* out, int out_dtype, const void* q,
                                      const void* k_cache, const void* v_cache, int kv_dtype,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int num_seqs, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks,
                                      int max_blocks_per_seq, float scale, int partition_size,
                                      const int32_t* members, int num_members,
                                      int prefix_partitions, const int32_t* work_list,
                                      int work_items, void* workspace, size_t workspace_bytes,
                                      int kv_policy, void* stream);
/* The shared-prefix pass alone (for timing or scheduling apart): writes the members'
 * partials of the shared partitions into the workspace, and the output row (out, of
 * out_dtype: kv_dtype or PKV_F32) of any member that fits one partition. */
int pkv_paged_attention_prefix(void* out, int out_dtype, const void* q, const void* k_cache,
                               const void* v_cache, int kv_dtype, const int32_t* block_tables,
                               const int32_t* seq_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, float scale, int partition_size,
                               const int32_t* members, int num_members, int prefix_partitions,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Cache write (P1 §4.3; P3 §2.2.2-§2.2.3): token t's K and V rows ([num_kv_heads][head_dim],
 * contiguous, t-major) are copied bit for bit to slot slot_mapping[t] of k_cache / v_cache.
 * A negative slot skips the token. Slots must be distinct. */
int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                          int dtype, const int32_t* slot_mapping, int num_tokens,
                          int num_kv_heads, int head_dim, int block_size, int num_blocks,
                          void* stream);

/* Copy-on-write block copy (P1 §6.2; P2 §2.2): for each (src, dst) pair of the int32
 * [num_pairs][2] array, block dst of both caches (all KV heads, all slots) becomes a bit
 * copy of block src. dst values must be distinct and disjoint from every src. */
int pkv_copy_blocks(void* k_cache, void* v_cache, int dtype, const int32_t* src_dst_pairs,
                    int num_pairs, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, void* stream);

/* Read-bandwidth probe (measurement only; no page defines it). The pages give no kernel
 * figure, and decode is judged against HBM bandwidth: this call measures the read rate the
 * device actually reaches, in the decode kernel's access patterns, as the achievable ceiling
 * reported beside the nominal peak. One 256-lane workgroup per tiles_per_group (1..1024)
 * consecutive entries of tile_ids (device int32 [num_tiles]); entry i names the tile_bytes
 * (a power of two in [256, 1 MiB]) contiguous bytes at tile_ids[i] * tile_bytes of buf (device,
 * 16-byte aligned, buf_bytes long); ids outside the buffer are skipped. Every byte of every
 * listed tile is loaded once. flags: 0 for the default cache policy, PKV_PROBE_NONTEMPORAL for
 * the non-temporal loads that the attention kernels use for KV rows; other bits PKV_EINVAL.
 * sink (device uint32) is written only if a lane's fold of its loaded words equals sentinel.
 * Enqueued on stream; no synchronisation. */
enum { PKV_PROBE_NONTEMPORAL = 1 };
int pkv_read_probe(const void* buf, size_t buf_bytes, int tile_bytes, const int32_t* tile_ids,
                   int num_tiles, int tiles_per_group, int flags, uint32_t sentinel,
                   uint32_t* sink, void* stream);

/* Per-workgroup timeline of the per-partition decode pass (measurement only; no page defines
 * it). With capacity > 0, every later launch of the per-partition pass (any decode entry
 * point) writes, for each of its workgroups w < capacity, eight uint32 at buf + 8 w: start
 * and end time (s_memrealtime, a 100 MHz clock, low 32 bits), the HW_ID register (CU, SIMD
 * and shader-engine ids), the XCC_ID register (XCD), the work unit it took (work-list
 * launches: row * num_kv_heads + KV head; else w), the times its first wave finished its key
 * pass and its value pass, and the tokens of its partition, from the workgroup's first
 * lane. Workgroups that find no work (list entries past a sequence's end) write nothing, so
 * clear the buffer first. buf: device, 16-byte aligned, 32 * capacity bytes, owned by the
 * caller and kept alive until the timeline is switched off with capacity 0. Process-wide;
 * not for concurrent use with launches on other threads. */
int pkv_debug_timeline(void* buf, int capacity);

/* ==========================================================================================
 * Host block manager (P2 §3.1 manager sketch; P1 §4.1-§4.3, §6; P3 §2.2.2-§2.2.3)
 * A fixed pool of num_blocks blocks; a per-sequence block table; a refcount per block. Host
 * memory only, owned by the handle. Not thread-safe: one thread per handle at a time.
 * Failing calls change no state (PKV_ENOBLOCKS also counts one allocation failure).
 * ========================================================================================== */
typedef struct pkv_bm pkv_bm;

/* free_order: NULL (ids 0,1,2,... in that order) or a permutation of [0, num_blocks) giving
 * the order in which blocks are handed out. Freed blocks are handed out again last-freed
 * first; a freed sequence releases its last logical block first. Returns NULL on bad input. */
pkv_bm* pkv_bm_create(int num_blocks, int block_size, const int32_t* free_order);
void pkv_bm_destroy(pkv_bm* bm);

/* New sequence holding num_tokens tokens in ceil(num_tokens/block_size) fresh blocks. */
int pkv_bm_add_seq(pkv_bm* bm, int64_t seq, int num_tokens);

/* child gets parent's table and length; every listed block's refcount grows by one
 * (parallel sampling / beam branches share the parent's blocks, P2 §2.2). */
int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child);

/* New sequence dst whose table is the first num_prefix_blocks (full) blocks of src, shared
 * (P1 §6.1; P3 §2.2.3 key point). Its length is num_prefix_blocks*block_size. */
int pkv_bm_share_prefix(pkv_bm* bm, int64_t src, int64_t dst, int num_prefix_blocks);

/* Reserves the slot of the sequence's next token (its current length becomes the position).
 * Position % block_size == 0: a fresh block is appended (P3 §2.2.3). Otherwise the token
 * goes into the last block; if that block is shared (refcount > 1) it is first replaced by a
 * fresh private block whose contents the caller must copy from *cow_src to *cow_dst with
 * pkv_copy_blocks before writing (P1 §6.2). Returns 0 (no copy), 1 (copy needed) or <0. */
int pkv_bm_append_slot(pkv_bm* bm, int64_t seq, int32_t* slot, int32_t* cow_src,
                       int32_t* cow_dst);

/* pkv_bm_append_slot for n sequences in order, atomically: on failure every append of the
 * batch is undone. slots: int32[n]; cow_pairs: int32[n][2] receives the copies needed, in
 * order; *num_cow their count. */
int pkv_bm_append_slots(pkv_bm* bm, const int64_t* seqs, int n, int32_t* slots,
                        int32_t* cow_pairs, int* num_cow);

/* pkv_bm_append_slots that also fills cow_src (int32[n], may be NULL): for each listed
 * sequence, the block its last block was copied from by this append (the src of its
 * copy-on-write pair), or -1 when its token went into a private or fresh block. That array is
 * the cow_src argument of pkv_paged_attention_decode_step for the same batch order (P1 §6.2:
 * a write into a shared block copies exactly that block first). On failure nothing changes,
 * cow_src included. */
int pkv_bm_append_step(pkv_bm* bm, const int64_t* seqs, int n, int32_t* slots,
                       int32_t* cow_pairs, int* num_cow, int32_t* cow_src);

/* Appends num_tokens tokens to the sequence, as that many pkv_bm_append_slot calls in a row
 * (prefill of a new chunk), atomically: on failure nothing changes. At most the first token
 * can need a copy-on-write; *cow_src / *cow_dst (may be NULL) receive it, or -1. The slots
 * of the new tokens are available from pkv_bm_slots. Returns 0, 1 (copy needed) or <0. */
int pkv_bm_extend(pkv_bm* bm, int64_t seq, int num_tokens, int32_t* cow_src, int32_t* cow_dst);

/* Releases the sequence: every block's refcount drops by one; blocks reaching zero return
 * to the free pool (P3 §2.2.2). */
int pkv_bm_free_seq(pkv_bm* bm, int64_t seq);

/* Copies up to cap entries of the sequence's table to out; *num_tokens (if not NULL) gets
 * its length. Returns the number of blocks in the table, or <0. */
int pkv_bm_table(const pkv_bm* bm, int64_t seq, int32_t* out, int cap, int* num_tokens);

/* Slots of token positions [start, start+count) of the sequence (all < its length). */
int pkv_bm_slots(const pkv_bm* bm, int64_t seq, int start, int count, int32_t* out);

/* Padded int32 [n][width] block tables (-1 past each table's end) and int32 seq_lens[n] for
 * the listed sequences, ready for pkv_paged_attention_decode. Fails if a table is wider. */
int pkv_bm_build_tables(const pkv_bm* bm, const int64_t* seqs, int n, int32_t* tables,
                        int width, int32_t* seq_lens);

/* Refcount of one block (0 = free), or <0 for an id outside the pool. */
int pkv_bm_refcount(const pkv_bm* bm, int32_t block);

/* Counters for pool monitoring (P3 §2.2.13 asks for pool occupancy, allocation failures and
 * the prefix-cache hit rate): out[0] blocks held by sequences, [1] blocks available for
 * allocation (free, plus cached blocks no sequence holds), [2] shared blocks (refcount > 1),
 * [3] copy-on-write copies issued, [4] allocation failures, [5] live sequences, [6] prefix
 * cache hits (blocks reused by pkv_bm_add_seq_cached), [7] prefix cache lookups (full prompt
 * blocks looked up). */
int pkv_bm_stats(const pkv_bm* bm, int64_t out[8]);

/* ------------------------------------------------------------------------------------------
 * Prefix caching (P1 §7.4; P3 §2.2.8, §2.2.13): requests that start with the same tokens
 * (a shared system prompt) reuse the physical blocks that already hold those tokens' K/V.
 * Only full blocks of prompts added with pkv_bm_add_seq_cached are cached. A block is
 * registered under its key: the block before it (its id and how many times it has been
 * handed out, or none) and its block_size token ids, so a key names the whole token prefix
 * up to that block exactly; there are no hash collisions. Cached blocks that no sequence
 * holds any more stay cached and count as available; they are handed out again only when no
 * free block is left, the one released longest ago first, and then leave the cache.
 * ------------------------------------------------------------------------------------------ */

/* New sequence holding the num_tokens prompt tokens token_ids[0..num_tokens). Its leading
 * full blocks whose token prefix is cached are reused (refcount + 1); the rest are fresh
 * blocks, and the fresh full ones are registered. *num_cached_tokens (may be NULL) receives
 * how many leading tokens are already in the cache: the caller writes K/V only for the
 * tokens after them (slots from pkv_bm_slots). Fails atomically with PKV_ENOBLOCKS. */
int pkv_bm_add_seq_cached(pkv_bm* bm, int64_t seq, const int32_t* token_ids, int num_tokens,
                          int* num_cached_tokens);

/* out[0] registered blocks, [1] of them held by no sequence, [2] hits, [3] lookups. */
int pkv_bm_prefix_stats(const pkv_bm* bm, int64_t out[4]);

/* ------------------------------------------------------------------------------------------
 * Continuous batching (P1 §8.2; P3 §2.2.12): a host scheduler over a block manager. Each step
 * frees the requests that are done, admits waiting requests first come, first served (while
 * the batch has room, the step's token budget covers their prompt and the pool keeps
 * watermark_blocks free after taking prompt + 1 tokens; it stops at the first that does not
 * fit), then gives every running request one token slot in admission order. When the pool is
 * empty the most recently admitted running request is preempted (P3 §2.2.2, §2.2.5): its
 * blocks are freed, the tokens it produced join its prompt for recomputation, and it returns
 * to the front of the queue. Host memory only; one thread per handle; the scheduler owns the
 * sequences it creates in the manager (sequence id = request id).
 * ------------------------------------------------------------------------------------------ */
typedef struct pkv_sched pkv_sched;

/* Step results, in caller-owned arrays: batch, finished, admitted and preempted hold
 * max_num_seqs ids each, cow_pairs max_num_seqs rows of (src, dst); slots, slot_seq and
 * slot_pos hold max_step_tokens entries. slots lists the admitted prompts' tokens (request
 * order, positions 0..prompt-1) and then one token per batch entry; slot_seq / slot_pos name
 * the request and the token position each slot is for. */
typedef struct {
  int64_t* batch;
  int32_t* slots;
  int64_t* slot_seq;
  int32_t* slot_pos;
  int32_t* cow_pairs;
  int64_t* finished;
  int64_t* admitted;
  int64_t* preempted;
  int num_batch, num_slots, num_cow, num_finished, num_admitted, num_preempted;
} pkv_sched_step_out;

/* block_size must be the manager's (else NULL); max_step_tokens >= max_num_seqs. NULL on bad
 * input. */
pkv_sched* pkv_sched_create(pkv_bm* bm, int block_size, int max_num_seqs, int max_step_tokens,
                            int watermark_blocks);
void pkv_sched_destroy(pkv_sched* s);
/* Queues a request of prompt_tokens (>= 1) that produces output_tokens (>= 1). prompt +
 * output must fit max_step_tokens and the pool less the watermark (a preempted request comes
 * back as one prompt); request ids must be new. */
int pkv_sched_add_request(pkv_sched* s, int64_t req_id, int prompt_tokens, int output_tokens);
/* Advances one decode step and fills *out. */
int pkv_sched_step(pkv_sched* s, pkv_sched_step_out* out);
/* out[0] waiting, [1] running, [2] finished, [3] admitted, [4] preempted (totals), [5] steps,
 * [6] decode tokens, [7] prompt tokens written. */
int pkv_sched_stats(const pkv_sched* s, int64_t out[8]);

/* ------------------------------------------------------------------------------------------
 * KV-pool sizing (P3 §2.2.5, §2.2.7). The pool is fixed at start-up from a memory fraction;
 * this host-only helper turns the device memory, the weights and the model's KV shape into
 * the num_blocks to pass to pkv_bm_create and to allocate the caches with, and into how many
 * requests of a given context length fit at once. Integer arithmetic only.
 * ------------------------------------------------------------------------------------------ */

/* How utilization_ppm is applied. P3's worked figure (80 GB device, 40 GB of weights, 0.9 ->
 * about 36 GB of pool) takes the fraction of what the weights leave: REMAINDER. DEVICE takes
 * the fraction of the whole device as the process's cap, and the weights come out of it. */
enum { PKV_UTIL_OF_REMAINDER = 0, PKV_UTIL_OF_DEVICE = 1 };

/* device_bytes: memory of one GPU; weight_bytes: its weights; reserve_bytes: activations and
 * workspaces kept out of the pool; utilization_ppm: the memory fraction in parts per million,
 * in (0, 1000000]. One token's KV takes num_layers * 2 * num_kv_heads * head_dim * elem_bytes
 * bytes (elem_bytes 1, 2 or 4); every layer has its own K and V cache of num_blocks blocks.
 *   REMAINDER: pool = floor((device - weights - reserve) * ppm / 1e6)
 *   DEVICE:    pool = floor(device * ppm / 1e6) - weights - reserve
 * out[0] pool bytes, [1] KV bytes per token (all layers), [2] bytes per block (all layers),
 * [3] num_blocks = floor(pool / out[2]), [4] blocks per request = ceil(context_tokens /
 * block_size), [5] requests served at once = floor(out[3] / out[4]), [6] bytes of one layer's
 * K cache (= V cache) [num_blocks][num_kv_heads][block_size][head_dim], [7] requests served
 * at once if each reserved max_model_len tokens contiguously = floor(pool / (out[1] *
 * max_model_len)). PKV_EINVAL for out-of-range arguments or num_blocks * block_size >=
 * 2^31 (slot ids are int32); PKV_ENOBLOCKS if the pool holds no block (out[0], [1], [2], [4]
 * are still filled; out[0] is negative when the weights and the reserve exceed the budget, and
 * INT64_MIN when that shortfall is beyond the int64 range). */
int pkv_kv_pool_plan(int64_t device_bytes, int64_t weight_bytes, int64_t reserve_bytes,
                     int32_t utilization_ppm, int utilization_of, int num_layers,
                     int num_kv_heads, int head_dim, int elem_bytes, int block_size,
                     int context_tokens, int max_model_len, int64_t out[8]);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
