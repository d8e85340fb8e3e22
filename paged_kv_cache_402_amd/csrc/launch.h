// Internal launch interface between the C ABI (capi.cpp) and the kernels (*.hip).
// Arguments here are already validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Workgroup shape of the decode kernel: 4 waves of 64 lanes.
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = 4;
// Work-list row flag: the row (flag | idx) stands for the four items stored at idx .. idx + 3
// of the list, one per wave of the workgroup.
constexpr uint32_t kPackedRow = 0x80000000u;
// Shared-prefix pass: the head_dim it is built for, and the block ids of one partition it
// keeps in LDS.
constexpr int kPrefixHeadDim = 128;
constexpr int kPrefixMaxIds = 256;

struct DecodeArgs {
  void* out;                   // [B][Hq][D] of out dtype
  const void* q;               // [B][Hq][D] of kv dtype
  const void* k_cache;         // [NB][Hkv][bs][D]
  const void* v_cache;
  const int32_t* block_tables; // [B][max_blocks]
  const int32_t* seq_lens;     // [B]
  float* ws_ml;                // [B][Hq][pmax][2]: running max (log2 units) and exponent sum
  float* ws_acc;               // [B][Hq][pmax][D]: unnormalised accumulators
  int num_seqs, num_q_heads, num_kv_heads, num_blocks, max_blocks;
  int bs_log2;                 // log2(block_size)
  int part;                    // tokens per partition
  int pmax;                    // partitions of the longest representable sequence
  float scale_log2;            // scale * log2(e): scores are kept in base-2 units
  int out_dtype;               // DType of out
  // Optional list of (sequence << 16 | partition) items, one workgroup per (KV head, item);
  // null: one workgroup per (KV head, partition, sequence) of the full pmax x B grid.
  const uint32_t* work;
  int work_items;
  // Optional appended token: [B][Hkv][D] K and V rows of token seq_lens[b] - 1, read from
  // here instead of the cache and stored into the cache by the pass (null: none).
  const void* k_new;
  const void* v_new;
  // Optional, with k_new: per sequence, the block its last block was just made a private copy
  // of (-1: none). The pass copies it (this KV head's tile, all rows but the new token's)
  // into the sequence's last block and reads the earlier tokens from it (null: no copies).
  const int32_t* cow_src;
  // Measurement only (null: off): workgroup w < timeline_cap of the per-partition pass writes
  // {start, end, HW_ID, XCC_ID} at 4 w (clock: s_memrealtime, 100 MHz).
  uint32_t* timeline;
  int timeline_cap;
  // Scheduling word of a work-list launch (the workspace's first 8 bytes; null: static
  // assignment only): {high 32 bits kSchedCookie once initialised, low 32 bits tickets taken}.
  // Workgroups w >= sched_static of the launch take work unit sched_static + ticket instead
  // of unit w, in the list's order, so units go to workgroups in the order they start; the
  // holder of the last ticket sets the count back to 0. The launch code sets sched_static so
  // that half as many workgroups as are resident at once take tickets (and at least one
  // resident round keeps its static units).
  unsigned long long* sched;
  int sched_static;
  // KV read policy: 0 non-temporal loads (streaming), 1 default cache policy (PKV_KV_CACHED)
  int kv_cached;
  // Fork groups (null: none): work items name groups instead of sequences. Group i lists
  // group_size sequences at groups[i * group_size ..] (-1: an empty place) that attend to the
  // same tokens before their new one: the same length, the same blocks before the new
  // token's block, and the same block (the source of their copies) for its earlier rows. The
  // group's G rows are query head kvh * group_heads + r % group_heads of member r /
  // group_heads; the first member's table and length describe the shared tokens.
  const int32_t* groups;
  int num_groups, group_size, group_heads;
};

// Bytes of the workspace header that holds the scheduling word.
constexpr size_t kWsHeaderBytes = 256;
constexpr unsigned kSchedCookie = 0x5CED0DE1u;
// Writes the initialised scheduling word {kSchedCookie, 0} (a one-lane kernel).
hipError_t launch_sched_init(unsigned long long* sched, hipStream_t stream);

// Process-wide timeline buffer picked up by every later per-partition launch (measurement).
void decode_timeline(uint32_t** buf, int* cap);

// Bytes of dynamic LDS one decode workgroup needs.
size_t decode_lds_bytes(int kv_dtype, int head_dim, int group, int part);

// Launches the per-partition kernel (grid: Hkv x pmax x B, or Hkv x work_items in one
// dimension when a work list is given). With `ticketed` non-null nothing is launched:
// *ticketed receives how many units of a work-list launch with these arguments would be
// handed out by ticket (those at the end of the list; 0 when none would).
hipError_t launch_decode_partitions(const DecodeArgs& a, int kv_dtype, int head_dim, int group,
                                    hipStream_t stream, int* ticketed = nullptr);
// The per-partition pass of launches with copy-on-write sources (DecodeArgs::cow_src set;
// decode_step.hip). launch_decode_partitions forwards such launches here.
hipError_t launch_decode_partitions_cow(const DecodeArgs& a, int kv_dtype, int head_dim,
                                        int group, hipStream_t stream, int* ticketed = nullptr);
// The same over fork groups (DecodeArgs::groups set; decode_groups.hip); rows = query heads
// per KV head x group size.
hipError_t launch_decode_partitions_groups(const DecodeArgs& a, int kv_dtype, int head_dim,
                                           int rows, hipStream_t stream,
                                           int* ticketed = nullptr);
// Launches the partition merge (grid: Hq x B); only multi-partition sequences do work.
hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t stream);

// Shared-prefix pass (prefix.hip): the first prefix_parts partitions of every member
// sequence list the same physical blocks; one workgroup per (KV head, 64 query rows of the
// members, partition) writes the members' partials for those partitions.
struct PrefixArgs {
  void* out;                   // [B][Hq][D] of out_dtype: rows of single-partition members
  int out_dtype;
  const void* q;               // [B][Hq][D]
  const void* k_cache;         // [NB][Hkv][bs][D]
  const void* v_cache;
  const int32_t* block_tables; // [B][max_blocks]; the first member's row gives the blocks
  const int32_t* seq_lens;     // [B]: each member attends only to its own tokens
  const int32_t* members;      // [num_members] sequence indices
  float* ws_ml;                // same layout as DecodeArgs
  float* ws_acc;
  int num_members, prefix_parts;
  int num_seqs, num_q_heads, num_kv_heads, num_blocks, max_blocks, bs_log2, part, pmax;
  float scale_log2;
};
bool prefix_supported(int kv_dtype, int head_dim, int group, int part, int bs_log2);
int prefix_chunk_seqs(int group);   // member sequences per workgroup
hipError_t launch_prefix(const PrefixArgs& a, int kv_dtype, int group, hipStream_t stream);

struct CacheWriteArgs {
  const void* k;            // [T][Hkv][D]
  const void* v;
  void* k_cache;            // [NB][Hkv][bs][D]
  void* v_cache;
  const int32_t* slots;     // [T]
  int num_tokens, num_kv_heads, row_bytes, bs_log2, num_blocks;
};
hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, hipStream_t stream);

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* pairs;     // [n][2]
  int num_pairs, num_blocks;
  int64_t block_bytes;      // bytes of one block of one cache (all heads, all slots)
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Split-K scratch of the allocation-free decode (static_ws.hip): a file-scope device array of
// kStaticWorkspaceBytes per device; *ptr receives its address on the current device.
constexpr size_t kStaticWorkspaceBytes = (size_t)64 << 20;
hipError_t static_workspace(void** ptr);

// Read-bandwidth probe (probe.hip).
struct ProbeArgs {
  const unsigned char* buf;
  const int32_t* tile_ids;   // [num_tiles]
  int64_t num_tile_slots;    // tiles the buffer holds; ids outside [0, slots) are skipped
  int num_tiles, tiles_per_group, tile_log2;
  uint32_t sentinel;
  uint32_t* sink;
  int nontemporal;           // 1: the non-temporal cache policy of the KV-row loads
};
hipError_t launch_read_probe(const ProbeArgs& a, hipStream_t stream);

}  // namespace pkv
