// C ABI of the device operations: host-side validation, workspace layout and dispatch to the
// gfx950 kernels. Nothing here touches device memory contents or synchronises.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <string>
#include <vector>

#include "errors.h"
#include "launch.h"
#include "pagedkv.h"

namespace pkv {

namespace {
std::atomic<uint32_t*> g_timeline{nullptr};
std::atomic<int> g_timeline_cap{0};
}  // namespace

void decode_timeline(uint32_t** buf, int* cap) {
  *cap = g_timeline_cap.load(std::memory_order_acquire);
  *buf = *cap > 0 ? g_timeline.load(std::memory_order_acquire) : nullptr;
}

namespace {

constexpr int kMaxGridYZ = 65535;
constexpr int kMaxListSeqs = 32767;      // work-list items keep their top bit clear
constexpr size_t kMaxDecodeLds = 64 * 1024;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}
int elem_bytes(int dt) { return dt == PKV_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Split-K workspace: a 256-byte header (its first 8 bytes: the scheduling word of the
// per-partition pass over a work list), then (max, sum) floats [B][Hq][pmax][2], padded to a
// multiple of 16 bytes so that the accumulators [B][Hq][pmax][D] floats after them take
// 16-byte loads. Nothing when no sequence can span two partitions.
struct WsLayout {
  size_t ml_off, acc_off, total;
};
WsLayout ws_layout(int64_t num_seqs, int64_t num_q_heads, int64_t pmax, int64_t head_dim) {
  if (pmax <= 1) return {0, 0, 0};
  const size_t rows = (size_t)num_seqs * (size_t)num_q_heads * (size_t)pmax;
  const size_t ml = (rows * 8 + 15) / 16 * 16;
  return {kWsHeaderBytes, kWsHeaderBytes + ml, kWsHeaderBytes + ml + rows * (size_t)head_dim * 4};
}

struct DecodePlan {
  DecodeArgs args;
  int group;
  size_t ws_needed;
};

int plan_decode(DecodePlan* pl, void* out, int out_dtype, const void* q, const void* k_cache,
                const void* v_cache, int kv_dtype, const int32_t* block_tables,
                const int32_t* seq_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                int head_dim, int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                int partition_size, void* workspace, size_t workspace_bytes, int kv_policy) {
  if (!dtype_ok(kv_dtype)) return fail(PKV_EDTYPE, "decode: unknown kv dtype %d", kv_dtype);
  if (kv_policy != PKV_KV_STREAM && kv_policy != PKV_KV_CACHED)
    return fail(PKV_EINVAL, "decode: unknown kv_policy %d", kv_policy);
  if (out_dtype != kv_dtype && out_dtype != PKV_F32)
    return fail(PKV_EDTYPE, "decode: out dtype must equal the kv dtype or be fp32");
  if (num_seqs < 0 || num_seqs > kMaxGridYZ) return fail(PKV_EINVAL, "decode: num_seqs %d out of range", num_seqs);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "decode: query heads must be a positive multiple of kv heads");
  const int group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PKV_EINVAL, "decode: query heads per kv head must be 1, 2, 4 or 8 (got %d)", group);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PKV_EINVAL, "decode: head_dim must be 64, 128 or 256");
  if (head_dim == 256 && group == 8) return fail(PKV_EINVAL, "decode: head_dim 256 supports groups up to 4");
  if ((head_dim * elem_bytes(kv_dtype)) % 128 != 0) return fail(PKV_EINVAL, "decode: row bytes must be a multiple of 128");
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256)
    return fail(PKV_EINVAL, "decode: block_size must be a power of two in [8, 256]");
  if (num_blocks <= 0 || (int64_t)num_blocks * block_size >= INT32_MAX)
    return fail(PKV_EINVAL, "decode: num_blocks out of range");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size >= INT32_MAX)
    return fail(PKV_EINVAL, "decode: max_blocks_per_seq out of range");
  if (partition_size == 0) partition_size = 512;
  if (partition_size < 32 || partition_size > 2048 || partition_size % 32 != 0 || partition_size % block_size != 0)
    return fail(PKV_EINVAL, "decode: partition_size must be a multiple of 32 and of block_size in [32, 2048]");
  if (decode_lds_bytes(kv_dtype, head_dim, group, partition_size) > kMaxDecodeLds)
    return fail(PKV_EINVAL, "decode: partition_size too large for LDS at this group size");
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
  const int64_t pmax = (max_tokens + partition_size - 1) / partition_size;
  if (pmax > kMaxGridYZ) return fail(PKV_EINVAL, "decode: too many partitions per sequence");
  if (num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens))
    return fail(PKV_EINVAL, "decode: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_EINVAL, "decode: out, q and caches must be 16-byte aligned");
  const WsLayout ws = ws_layout(num_seqs, num_q_heads, pmax, head_dim);
  const size_t need = ws.total;
  pl->ws_needed = need;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_EWORKSPACE, "decode: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (need > 0 && !aligned16(workspace))
    return fail(PKV_EINVAL, "decode: workspace must be 16-byte aligned");

  DecodeArgs& a = pl->args;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.ws_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml_off) : nullptr;
  a.ws_acc = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.acc_off) : nullptr;
  a.sched = need ? reinterpret_cast<unsigned long long*>(workspace) : nullptr;
  a.sched_static = 0;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.bs_log2 = log2i(block_size);
  a.part = partition_size;
  a.pmax = (int)pmax;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.out_dtype = out_dtype;
  a.work = nullptr;
  a.work_items = 0;
  a.k_new = nullptr;
  a.cow_src = nullptr;
  a.v_new = nullptr;
  decode_timeline(&a.timeline, &a.timeline_cap);
  a.kv_cached = kv_policy == PKV_KV_CACHED;
  a.groups = nullptr;
  a.num_groups = 0;
  a.group_size = 1;
  a.group_heads = group;
  pl->group = group;
  pl->ws_needed = need;
  return ok();
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

int pkv_version(void) { return 100; }

size_t pkv_decode_workspace_bytes(int num_seqs, int num_q_heads, int max_blocks_per_seq,
                                  int block_size, int head_dim, int partition_size) {
  if (partition_size == 0) partition_size = 512;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || block_size <= 0 ||
      head_dim <= 0 || partition_size <= 0)
    return 0;
  const int64_t pmax = ((int64_t)max_blocks_per_seq * block_size + partition_size - 1) / partition_size;
  return ws_layout(num_seqs, num_q_heads, pmax, head_dim).total;
}

int pkv_paged_attention_partitions(void* out, int out_dtype, const void* q, const void* k_cache,
                                   const void* v_cache, int kv_dtype, const int32_t* block_tables,
                                   const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                   int max_blocks_per_seq, float scale, int partition_size,
                                   void* workspace, size_t workspace_bytes, int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  return hip_status(launch_decode_partitions(pl.args, kv_dtype, head_dim, pl.group, (hipStream_t)stream),
                    "decode partitions launch");
}

}  // extern "C"

namespace {

int check_list_args(const char* who, int num_seqs, int max_blocks_per_seq, int block_size,
                    int partition_size) {
  if (num_seqs < 0 || num_seqs > kMaxListSeqs)
    return fail(PKV_EINVAL, "%s: num_seqs %d out of range [0, %d]", who, num_seqs, kMaxListSeqs);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256)
    return fail(PKV_EINVAL, "%s: block_size must be a power of two in [8, 256]", who);
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size >= INT32_MAX)
    return fail(PKV_EINVAL, "%s: max_blocks_per_seq out of range", who);
  if (partition_size < 32 || partition_size > 2048 || partition_size % 32 != 0 ||
      partition_size % block_size != 0)
    return fail(PKV_EINVAL, "%s: bad partition_size", who);
  const int64_t cap_tokens = (int64_t)max_blocks_per_seq * block_size;
  if ((cap_tokens + partition_size - 1) / partition_size > 65535)
    return fail(PKV_EINVAL, "%s: too many partitions per sequence", who);
  return PKV_OK;
}

// Items (b << 16 | p) of every partition that holds tokens, except the first skip[b]
// partitions of sequence b (skip may be null): full partitions in (sequence, partition) order,
// then the last, shorter partitions longest first, ties in sequence order.
std::vector<uint32_t> build_work_list(const int32_t* seq_lens, int num_seqs, int64_t cap_tokens,
                                      int partition_size, const std::vector<int>* skip) {
  std::vector<uint32_t> full;
  std::vector<std::pair<int, uint32_t>> tail;  // (-tokens, item)
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t L = std::min<int64_t>(std::max(seq_lens[b], 0), cap_tokens);
    const int64_t np = L == 0 ? 1 : (L + partition_size - 1) / partition_size;
    const int64_t first = skip ? (*skip)[b] : 0;
    for (int64_t p = first; p < np; ++p) {
      const int64_t n = std::min<int64_t>(partition_size, L - p * partition_size);
      const uint32_t item = ((uint32_t)b << 16) | (uint32_t)p;
      if (n == partition_size) full.push_back(item);
      else tail.emplace_back(-(int)n, item);
    }
  }
  std::stable_sort(tail.begin(), tail.end(),
                   [](const std::pair<int, uint32_t>& x, const std::pair<int, uint32_t>& y) {
                     return x.first < y.first;
                   });
  for (const auto& t : tail) full.push_back(t.second);
  return full;
}

// Rows of a packed list: each item of more than pack_tokens tokens as a row of its own, and
// one row (kPackedRow | idx) per four consecutive shorter items, which are stored after the
// rows from index idx (the last group padded with items naming sequence 0xFFFF, which every
// launch skips). items are in build_work_list order, so the short ones are its tail, longest
// first. The rows run in decreasing order of the tokens one wave of the row goes through:
// a plain item's four waves share its tokens, a packed wave takes its whole item, so a packed
// row weighs as much as its longest item and a plain one a quarter of its tokens (ties: list
// order, plain rows first). The launch then starts the rows that take longest first.
std::vector<uint32_t> pack_work_list(const std::vector<uint32_t>& items, const int32_t* seq_lens,
                                     int64_t cap_tokens, int partition_size, int pack_tokens,
                                     int* rows) {
  auto tokens = [&](uint32_t it) {
    const int64_t L = std::min<int64_t>(std::max(seq_lens[it >> 16], 0), cap_tokens);
    return std::min<int64_t>(partition_size, L - (int64_t)(it & 0xFFFFu) * partition_size);
  };
  size_t first = items.size();
  while (first > 0 && tokens(items[first - 1]) <= pack_tokens) --first;
  const size_t nshort = items.size() - first;
  const size_t groups = (nshort + 3) / 4;
  const size_t base = first + groups;
  std::vector<std::pair<int64_t, uint32_t>> keyed;   // (-tokens per wave, row)
  keyed.reserve(base);
  for (size_t i = 0; i < first; ++i)
    keyed.emplace_back(-((tokens(items[i]) + kDecodeWaves - 1) / kDecodeWaves), items[i]);
  for (size_t g = 0; g < groups; ++g)
    keyed.emplace_back(-tokens(items[first + 4 * g]), kPackedRow | (uint32_t)(base + 4 * g));
  std::stable_sort(keyed.begin(), keyed.end(),
                   [](const std::pair<int64_t, uint32_t>& x, const std::pair<int64_t, uint32_t>& y) {
                     return x.first < y.first;
                   });
  std::vector<uint32_t> out;
  out.reserve(base + 4 * groups);
  for (const auto& k : keyed) out.push_back(k.second);
  *rows = (int)out.size();
  for (size_t i = 0; i < 4 * groups; ++i)
    out.push_back(i < nshort ? items[first + i] : 0xFFFF0000u);
  return out;
}

int emit_list(const char* who, const std::vector<uint32_t>& items, int32_t* work_list,
              int capacity) {
  if ((int64_t)items.size() > INT32_MAX / 8) return fail(PKV_EINVAL, "%s: too many items", who);
  const int total = (int)items.size();
  if (work_list == nullptr) return total;     // size query
  if (capacity < total) return fail(PKV_EINVAL, "%s: %d items, capacity %d", who, total, capacity);
  for (int i = 0; i < total; ++i) work_list[i] = (int32_t)items[i];
  return total;
}

}  // namespace

extern "C" {

int pkv_decode_default_partition(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      head_dim <= 0 || !is_pow2(block_size) || block_size < 8 || block_size > 256 ||
      max_blocks_per_seq <= 0)
    return fail(PKV_EINVAL, "default_partition: bad argument");
  const int group = num_q_heads / num_kv_heads;
  const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
  // the longest partition (a multiple of 256 tokens, and of the block size) whose workgroup
  // takes no more than its share of a compute unit's 160 KiB of LDS at the occupancy the
  // kernel's registers allow, and that still gives the machine work: at least kMinGroups
  // workgroups even if every sequence were as long as its table allows. Up to G = 4 the
  // kernels fit four workgroups per compute unit (40 KiB each); the G = 8 kernels hold more
  // than 128 VGPRs, so three (53 KiB each): longer partitions there cost no occupancy.
  constexpr int64_t kMinGroups = 1024;
  const size_t lds_share = group == 8 ? 160 * 1024 / 3 : 40 * 1024;
  static const int kCandidates[] = {2048, 1792, 1536, 1280, 1024, 768, 512, 256};
  int part = 256;
  for (int c : kCandidates) {
    if (c % block_size != 0) continue;
    const int64_t groups = (int64_t)num_seqs * num_kv_heads * ((tokens + c - 1) / c);
    if (decode_lds_bytes(PKV_BF16, head_dim, group, c) <= lds_share && groups >= kMinGroups) {
      part = c;
      break;
    }
  }
  ok();
  return part;
}

int pkv_decode_kv_policy(const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                         int max_blocks_per_seq, int block_size, int num_blocks,
                         const int32_t* work_list, int list_len, int partition_size) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || !is_pow2(block_size) ||
      (int64_t)max_blocks_per_seq * block_size >= INT32_MAX || list_len < 0)
    return fail(PKV_EINVAL, "kv_policy: bad sizes");
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return fail(PKV_EINVAL, "kv_policy: null block_tables or seq_lens");
  if (work_list != nullptr && (partition_size <= 0 || partition_size % block_size != 0))
    return fail(PKV_EINVAL, "kv_policy: a work list needs its partition size, a multiple of "
                "block_size");
  // block reads of the launch (every in-pool table entry of the tokens it attends, lengths
  // clamped as the kernel clamps them) against the distinct blocks among them. A block was
  // seen in this call when its stamp equals this call's; the stamps persist per thread, so a
  // call costs O(reads) and not a pass over the whole pool.
  thread_local std::vector<uint32_t> stamp;
  thread_local uint32_t epoch = 0;
  if (stamp.size() < (size_t)num_blocks) stamp.resize((size_t)num_blocks, 0);
  if (++epoch == 0) {                       // wrapped: forget every stamp
    std::fill(stamp.begin(), stamp.end(), 0u);
    epoch = 1;
  }
  int64_t reads = 0, distinct = 0;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  auto read_blocks = [&](int b, int64_t t0, int64_t t1) {   // tokens [t0, t1) of sequence b
    const int32_t* row = block_tables + (size_t)b * max_blocks_per_seq;
    for (int64_t j = t0 / block_size; j < (t1 + block_size - 1) / block_size; ++j) {
      const int32_t id = row[j];
      if (id < 0 || id >= num_blocks) continue;
      ++reads;
      if (stamp[id] != epoch) {
        stamp[id] = epoch;
        ++distinct;
      }
    }
  };
  auto length = [&](int b) { return std::min<int64_t>(std::max(seq_lens[b], 0), cap); };
  if (work_list == nullptr) {
    for (int b = 0; b < num_seqs; ++b) read_blocks(b, 0, length(b));
  } else {
    // plain items (sequence << 16 | partition); packed-row entries (top bit) only point at
    // items stored further on in the same list, which are counted where they stand
    for (int i = 0; i < list_len; ++i) {
      const uint32_t w = (uint32_t)work_list[i];
      if (w & 0x80000000u) continue;
      const int b = (int)(w >> 16), p = (int)(w & 0xFFFFu);
      if (b >= num_seqs) continue;
      const int64_t t0 = (int64_t)p * partition_size;
      const int64_t t1 = std::min<int64_t>(t0 + partition_size, length(b));
      if (t1 > t0) read_blocks(b, t0, t1);
    }
  }
  ok();
  return reads >= 2 * distinct && reads > 0 ? PKV_KV_CACHED : PKV_KV_STREAM;
}

int pkv_decode_work_list(const int32_t* seq_lens, int num_seqs, int max_blocks_per_seq,
                         int block_size, int partition_size, int32_t* work_list, int capacity) {
  if (partition_size == 0) partition_size = 512;
  int st = check_list_args("work_list", num_seqs, max_blocks_per_seq, block_size, partition_size);
  if (st != PKV_OK) return st;
  if (num_seqs > 0 && !seq_lens) return fail(PKV_EINVAL, "work_list: null seq_lens");
  const auto items = build_work_list(seq_lens, num_seqs, (int64_t)max_blocks_per_seq * block_size,
                                     partition_size, nullptr);
  st = emit_list("work_list", items, work_list, capacity);
  if (st >= 0) ok();
  return st;
}

int pkv_decode_work_list_packed(const int32_t* seq_lens, int num_seqs, int max_blocks_per_seq,
                                int block_size, int partition_size, int pack_tokens,
                                int32_t* work_list, int capacity, int* rows) {
  if (partition_size == 0) partition_size = 512;
  int st = check_list_args("work_list_packed", num_seqs, max_blocks_per_seq, block_size,
                           partition_size);
  if (st != PKV_OK) return st;
  if (num_seqs > 0 && !seq_lens) return fail(PKV_EINVAL, "work_list_packed: null seq_lens");
  if (!rows) return fail(PKV_EINVAL, "work_list_packed: null rows");
  if (pack_tokens < 0 || pack_tokens > partition_size / kDecodeWaves)
    return fail(PKV_EINVAL, "work_list_packed: pack_tokens %d outside [0, partition_size / 4]",
                pack_tokens);
  const int64_t cap_tokens = (int64_t)max_blocks_per_seq * block_size;
  const auto items = build_work_list(seq_lens, num_seqs, cap_tokens, partition_size, nullptr);
  int r = (int)items.size();
  const auto list = pack_tokens > 0
                        ? pack_work_list(items, seq_lens, cap_tokens, partition_size, pack_tokens, &r)
                        : items;
  if ((int64_t)list.size() > (int64_t)(kPackedRow - 1))
    return fail(PKV_EINVAL, "work_list_packed: too many items");
  st = emit_list("work_list_packed", list, work_list, capacity);
  if (st >= 0) {
    *rows = r;
    ok();
  }
  return st;
}

int pkv_decode_ticketed_items(int kv_dtype, int head_dim, int num_q_heads, int num_kv_heads,
                              int block_size, int partition_size, int list_len, int launch_kind,
                              int group_size) {
  if (!dtype_ok(kv_dtype)) return fail(PKV_EDTYPE, "ticketed_items: unknown kv dtype %d", kv_dtype);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "ticketed_items: query heads must be a positive multiple of kv heads");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PKV_EINVAL, "ticketed_items: head_dim must be 64, 128 or 256");
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256)
    return fail(PKV_EINVAL, "ticketed_items: block_size must be a power of two in [8, 256]");
  if (partition_size == 0) partition_size = 512;
  if (partition_size < 32 || partition_size > 2048 || partition_size % 32 != 0 ||
      partition_size % block_size != 0)
    return fail(PKV_EINVAL, "ticketed_items: bad partition_size");
  if (list_len < 0 || (int64_t)list_len * num_kv_heads > INT32_MAX)
    return fail(PKV_EINVAL, "ticketed_items: list_len out of range");
  if (launch_kind != PKV_LAUNCH_PLAIN && launch_kind != PKV_LAUNCH_COPY_ON_WRITE &&
      launch_kind != PKV_LAUNCH_FORK_GROUPS)
    return fail(PKV_EINVAL, "ticketed_items: unknown launch_kind %d", launch_kind);
  const int group = num_q_heads / num_kv_heads;
  const int64_t rows =
      launch_kind == PKV_LAUNCH_FORK_GROUPS ? (int64_t)std::max(group_size, 0) * group : group;
  if (rows != 1 && rows != 2 && rows != 4 && rows != 8)
    return fail(PKV_EINVAL, "ticketed_items: rows per workgroup must be 1, 2, 4 or 8 (got %lld)",
                (long long)rows);
  if (rows == 8 && head_dim > 128)
    return fail(PKV_EINVAL, "ticketed_items: 8 rows need head_dim <= 128");
  if ((head_dim * elem_bytes(kv_dtype)) % 128 != 0)
    return fail(PKV_EINVAL, "ticketed_items: row bytes must be a multiple of 128");
  if (decode_lds_bytes(kv_dtype, head_dim, (int)rows, partition_size) > kMaxDecodeLds)
    return fail(PKV_EINVAL, "ticketed_items: partition_size too large for LDS at this group size");
  if (list_len == 0) return ok();
  // the kernel a launch with these arguments picks depends on the sizes, the dtypes and the
  // kind of launch only (both KV read policies build to the same occupancy)
  DecodeArgs a{};
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.bs_log2 = log2i(block_size);
  a.part = partition_size;
  a.work_items = list_len;
  a.group_size = launch_kind == PKV_LAUNCH_FORK_GROUPS ? group_size : 1;
  a.group_heads = group;
  int ticketed = 0;
  hipError_t e;
  if (launch_kind == PKV_LAUNCH_FORK_GROUPS)
    e = launch_decode_partitions_groups(a, kv_dtype, head_dim, (int)rows, nullptr, &ticketed);
  else if (launch_kind == PKV_LAUNCH_COPY_ON_WRITE)
    e = launch_decode_partitions_cow(a, kv_dtype, head_dim, group, nullptr, &ticketed);
  else
    e = launch_decode_partitions(a, kv_dtype, head_dim, group, nullptr, &ticketed);
  const int st = hip_status(e, "ticketed_items: occupancy query");
  if (st != PKV_OK) return st;
  return (ticketed + num_kv_heads - 1) / num_kv_heads;
}

int pkv_decode_work_list_private_tail(const int32_t* block_tables, const int32_t* seq_lens,
                                      int num_seqs, int max_blocks_per_seq, int block_size,
                                      int num_blocks, int partition_size, int tail_items,
                                      int32_t* work_list, int list_len) {
  if (partition_size == 0) partition_size = 512;
  int st = check_list_args("private_tail", num_seqs, max_blocks_per_seq, block_size,
                           partition_size);
  if (st != PKV_OK) return st;
  if (num_blocks <= 0) return fail(PKV_EINVAL, "private_tail: num_blocks must be positive");
  if (tail_items < 0 || list_len < 0)
    return fail(PKV_EINVAL, "private_tail: negative tail_items or list_len");
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return fail(PKV_EINVAL, "private_tail: null block_tables or seq_lens");
  if (list_len > 0 && !work_list) return fail(PKV_EINVAL, "private_tail: null work_list");
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  for (int i = 0; i < list_len; ++i) {
    const uint32_t w = (uint32_t)work_list[i];
    if (w & kPackedRow) return fail(PKV_EINVAL, "private_tail: packed lists are not reordered");
    if ((int)(w >> 16) >= num_seqs)
      return fail(PKV_EINVAL, "private_tail: item %d names sequence %d of %d", i, (int)(w >> 16),
                  num_seqs);
  }
  const int T = std::min(tail_items, list_len);
  if (T == 0) return ok();
  auto tokens = [&](uint32_t w) {   // tokens of the item's partition (0 past the end)
    const int64_t L = std::min<int64_t>(std::max(seq_lens[w >> 16], 0), cap);
    return std::max<int64_t>(0, std::min<int64_t>(partition_size,
                                                  L - (int64_t)(w & 0xFFFFu) * partition_size));
  };
  // how many reads each block gets from the whole list (in-pool table entries of every item's
  // tokens); per-thread stamps keep a call at O(reads) rather than a pass over the pool
  thread_local std::vector<uint32_t> stamp, count;
  thread_local uint32_t epoch = 0;
  if (stamp.size() < (size_t)num_blocks) {
    stamp.resize((size_t)num_blocks, 0);
    count.resize((size_t)num_blocks, 0);
  }
  if (++epoch == 0) {
    std::fill(stamp.begin(), stamp.end(), 0u);
    epoch = 1;
  }
  auto for_blocks = [&](uint32_t w, auto&& f) {
    const int64_t n = tokens(w);
    if (n == 0) return;
    const int64_t t0 = (int64_t)(w & 0xFFFFu) * partition_size;
    const int32_t* row = block_tables + (size_t)(w >> 16) * max_blocks_per_seq;
    for (int64_t j = t0 / block_size; j < (t0 + n + block_size - 1) / block_size; ++j)
      if (row[j] >= 0 && row[j] < num_blocks) f(row[j]);
  };
  for (int i = 0; i < list_len; ++i)
    for_blocks((uint32_t)work_list[i], [&](int32_t id) {
      if (stamp[id] != epoch) {
        stamp[id] = epoch;
        count[id] = 0;
      }
      ++count[id];
    });
  std::vector<char> shared((size_t)list_len, 0);
  for (int i = 0; i < list_len; ++i)
    for_blocks((uint32_t)work_list[i], [&](int32_t id) {
      if (count[id] > 1) shared[i] = 1;
    });
  int before = 0;
  int64_t longest = 0;
  for (int i = list_len - T; i < list_len; ++i) {
    before += shared[i];
    longest = std::max(longest, tokens((uint32_t)work_list[i]));
  }
  if (before == 0) return ok();
  // the new tail: the last T private items of the list, walking back from its end and
  // stopping at the first private item more than a quarter longer than the old tail's
  // longest (a long item at the end of the launch would lengthen its drain by more than the
  // re-read it saves)
  const int64_t limit = longest + longest / 4;
  std::vector<char> moved((size_t)list_len, 0);
  int k = 0;
  for (int i = list_len - 1; i >= 0 && k < T; --i) {
    if (shared[i]) continue;
    if (tokens((uint32_t)work_list[i]) > limit) break;
    moved[i] = 1;
    ++k;
  }
  if (k == T - before) return ok();   // no private item to spare: the list stays as it is
  std::vector<int32_t> out;
  out.reserve((size_t)list_len);
  for (int i = 0; i < list_len; ++i)
    if (!moved[i]) out.push_back(work_list[i]);
  for (int i = 0; i < list_len; ++i)
    if (moved[i]) out.push_back(work_list[i]);
  std::copy(out.begin(), out.end(), work_list);
  int after = 0;
  for (int i = list_len - T; i < list_len; ++i) {
    const uint32_t w = (uint32_t)out[i];
    bool sh = false;
    for_blocks(w, [&](int32_t id) { sh = sh || count[id] > 1; });
    after += sh;
  }
  ok();
  return before - after;
}

int pkv_decode_plan_fork_groups(const int32_t* block_tables, const int32_t* seq_lens,
                                const int32_t* cow_src, int num_seqs, int max_blocks_per_seq,
                                int block_size, int num_blocks, int group_size, int32_t* groups,
                                int32_t* group_lens, int capacity) {
  if (num_seqs < 0 || num_seqs > kMaxListSeqs)
    return fail(PKV_EINVAL, "plan_fork_groups: num_seqs %d out of range [0, %d]", num_seqs,
                kMaxListSeqs);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256)
    return fail(PKV_EINVAL, "plan_fork_groups: block_size must be a power of two in [8, 256]");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size >= INT32_MAX)
    return fail(PKV_EINVAL, "plan_fork_groups: max_blocks_per_seq out of range");
  if (num_blocks <= 0) return fail(PKV_EINVAL, "plan_fork_groups: num_blocks must be positive");
  if (group_size < 1) return fail(PKV_EINVAL, "plan_fork_groups: group_size must be >= 1");
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return fail(PKV_EINVAL, "plan_fork_groups: null tables or seq_lens");
  const int64_t cap_tokens = (int64_t)max_blocks_per_seq * block_size;
  const int shift = log2i(block_size);
  struct Key {
    int64_t len;     // clamped length, the new token included
    int64_t blocks;  // blocks before the new token's block
    int src;         // block its earlier rows come from (-1: none)
  };
  std::vector<Key> key(num_seqs);
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t L = std::min<int64_t>(std::max(seq_lens[b], 0), cap_tokens);
    Key k{L, L > 0 ? (L - 1) >> shift : 0, -1};
    if (L > 0 && ((L - 1) & (block_size - 1)) != 0) {
      const int c = cow_src ? cow_src[b] : -1;
      k.src = (unsigned)c < (unsigned)num_blocks
                  ? c
                  : block_tables[(size_t)b * max_blocks_per_seq + (size_t)k.blocks];
    }
    key[b] = k;
  }
  auto row = [&](int b) { return block_tables + (size_t)b * max_blocks_per_seq; };
  auto less = [&](int x, int y) {
    const Key &a = key[x], &b = key[y];
    if (a.len != b.len) return a.len < b.len;
    if (a.src != b.src) return a.src < b.src;
    return std::lexicographical_compare(row(x), row(x) + a.blocks, row(y), row(y) + b.blocks);
  };
  auto same = [&](int x, int y) {
    // a sequence of length 0 attends to nothing and shares with nobody
    return key[x].len > 0 && !less(x, y) && !less(y, x);
  };
  std::vector<int> order(num_seqs);
  for (int b = 0; b < num_seqs; ++b) order[b] = b;
  std::stable_sort(order.begin(), order.end(), less);
  // runs of equal keys (in increasing sequence order), in chunks of group_size
  std::vector<std::vector<int>> out;
  for (size_t i = 0; i < order.size();) {
    size_t j = i + 1;
    while (j < order.size() && same(order[i], order[j])) ++j;
    for (size_t c = i; c < j; c += (size_t)group_size)
      out.emplace_back(order.begin() + (long)c, order.begin() + (long)std::min(j, c + group_size));
    i = j;
  }
  std::sort(out.begin(), out.end(), [](const std::vector<int>& x, const std::vector<int>& y) {
    return x[0] < y[0];
  });
  const int n = (int)out.size();
  if (!groups && !group_lens) {   // size query
    ok();
    return n;
  }
  if (!groups || !group_lens) return fail(PKV_EINVAL, "plan_fork_groups: null output");
  if (capacity < n) return fail(PKV_EINVAL, "plan_fork_groups: %d groups, capacity %d", n, capacity);
  for (int g = 0; g < n; ++g) {
    for (int j = 0; j < group_size; ++j)
      groups[(size_t)g * group_size + j] = j < (int)out[g].size() ? out[g][j] : -1;
    group_lens[g] = (int32_t)key[out[g][0]].len;
  }
  ok();
  return n;
}

int pkv_decode_plan_shared_prefix(const int32_t* block_tables, const int32_t* seq_lens,
                                  int num_seqs, int max_blocks_per_seq, int block_size,
                                  int partition_size, int min_members, int32_t* members,
                                  int* num_members, int* prefix_partitions, int32_t* work_list,
                                  int capacity) {
  if (partition_size == 0) partition_size = 512;
  int st = check_list_args("plan_shared_prefix", num_seqs, max_blocks_per_seq, block_size,
                           partition_size);
  if (st != PKV_OK) return st;
  if (num_seqs > 0 && (!block_tables || !seq_lens))
    return fail(PKV_EINVAL, "plan_shared_prefix: null tables or seq_lens");
  if (!members || !num_members || !prefix_partitions)
    return fail(PKV_EINVAL, "plan_shared_prefix: null output");
  const int64_t cap_tokens = (int64_t)max_blocks_per_seq * block_size;
  const int bpp = partition_size / block_size;                 // blocks per partition
  auto len = [&](int b) { return std::min<int64_t>(std::max(seq_lens[b], 0), cap_tokens); };
  auto row = [&](int b) { return block_tables + (size_t)b * max_blocks_per_seq; };
  // candidates: sequences with a full first partition and more tokens after it, grouped by
  // the block ids of that partition; the largest group wins (ties: lowest first sequence)
  std::vector<int> order;
  for (int b = 0; b < num_seqs; ++b)
    if (len(b) > partition_size) order.push_back(b);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return std::lexicographical_compare(row(x), row(x) + bpp, row(y), row(y) + bpp);
  });
  int best_start = 0, best_n = 0;
  for (size_t i = 0; i < order.size();) {
    size_t j = i + 1;
    while (j < order.size() && std::equal(row(order[i]), row(order[i]) + bpp, row(order[j]))) ++j;
    const int n = (int)(j - i);
    const int first = *std::min_element(order.begin() + i, order.begin() + j);
    const int best_first = best_n ? *std::min_element(order.begin() + best_start,
                                                      order.begin() + best_start + best_n)
                                  : INT32_MAX;
    if (n > best_n || (n == best_n && first < best_first)) {
      best_start = (int)i;
      best_n = n;
    }
    i = j;
  }
  std::vector<int> skip(num_seqs, 0);
  int pp = 0, nm = 0;
  if (best_n >= std::max(2, min_members)) {
    std::vector<int> grp(order.begin() + best_start, order.begin() + best_start + best_n);
    std::sort(grp.begin(), grp.end());
    // shared partitions: all members list the first member's blocks, and every member has
    // tokens after them
    const int rep = grp[0];
    pp = (int)((cap_tokens + partition_size - 1) / partition_size);
    for (int b : grp) {
      int q = 0;
      const int64_t max_q = (len(b) - 1) / partition_size;
      while (q < max_q && q < pp &&
             std::equal(row(rep) + (size_t)q * bpp, row(rep) + (size_t)(q + 1) * bpp,
                        row(b) + (size_t)q * bpp))
        ++q;
      pp = std::min(pp, q);
    }
    for (int b : grp) {
      members[nm++] = b;
      skip[b] = pp;
    }
  }
  *num_members = pp > 0 ? nm : 0;
  *prefix_partitions = pp;
  const auto items = build_work_list(seq_lens, num_seqs, cap_tokens, partition_size,
                                     pp > 0 ? &skip : nullptr);
  st = emit_list("plan_shared_prefix", items, work_list, capacity);
  if (st >= 0) ok();
  return st;
}

static int partitions_list(const DecodePlan& pl0, int kv_dtype, int head_dim,
                           const int32_t* work_list, int work_items, void* stream) {
  if (work_items < 0) return fail(PKV_EINVAL, "decode: negative work_items");
  if (work_items == 0) return ok();
  if (!work_list) return fail(PKV_EINVAL, "decode: null work_list");
  // an item's top bit marks a packed row, so listed sequences stay below 32768
  if (pl0.args.num_seqs > kMaxListSeqs)
    return fail(PKV_EINVAL, "decode: a work list takes at most %d sequences", kMaxListSeqs);
  if ((int64_t)work_items * pl0.args.num_kv_heads > INT32_MAX)
    return fail(PKV_EINVAL, "decode: work list too long");
  DecodePlan pl = pl0;
  pl.args.work = reinterpret_cast<const uint32_t*>(work_list);
  pl.args.work_items = work_items;
  return hip_status(launch_decode_partitions(pl.args, kv_dtype, head_dim, pl.group, (hipStream_t)stream),
                    "decode partitions launch");
}

int pkv_paged_attention_partitions_list(void* out, int out_dtype, const void* q,
                                        const void* k_cache, const void* v_cache, int kv_dtype,
                                        const int32_t* block_tables, const int32_t* seq_lens,
                                        int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int block_size, int num_blocks,
                                        int max_blocks_per_seq, float scale, int partition_size,
                                        const int32_t* work_list, int work_items, void* workspace,
                                        size_t workspace_bytes, int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  return partitions_list(pl, kv_dtype, head_dim, work_list, work_items, stream);
}

int pkv_paged_attention_decode_list(void* out, int out_dtype, const void* q, const void* k_cache,
                                    const void* v_cache, int kv_dtype,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, int max_blocks_per_seq,
                                    float scale, int partition_size, const int32_t* work_list,
                                    int work_items, void* workspace, size_t workspace_bytes,
                                    int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = partitions_list(pl, kv_dtype, head_dim, work_list, work_items, stream);
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

static int append_args(DecodePlan* pl, const void* k_new, const void* v_new) {
  if (!k_new || !v_new) return fail(PKV_EINVAL, "decode_append: null k_new or v_new");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_EINVAL, "decode_append: k_new and v_new must be 16-byte aligned");
  pl->args.k_new = k_new;
  pl->args.v_new = v_new;
  return PKV_OK;
}

static int partitions_any(const DecodePlan& pl, int kv_dtype, int head_dim,
                          const int32_t* work_list, int work_items, void* stream) {
  if (work_list == nullptr && work_items == 0)
    return hip_status(launch_decode_partitions(pl.args, kv_dtype, head_dim, pl.group,
                                               (hipStream_t)stream),
                      "decode partitions launch");
  return partitions_list(pl, kv_dtype, head_dim, work_list, work_items, stream);
}

int pkv_paged_attention_decode_append(void* out, int out_dtype, const void* q, const void* k_new,
                                      const void* v_new, void* k_cache, void* v_cache,
                                      int kv_dtype, const int32_t* block_tables,
                                      const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int num_blocks, int max_blocks_per_seq, float scale,
                                      int partition_size, const int32_t* work_list,
                                      int work_items, void* workspace, size_t workspace_bytes,
                                      int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  if ((st = append_args(&pl, k_new, v_new)) != PKV_OK) return st;
  st = partitions_any(pl, kv_dtype, head_dim, work_list, work_items, stream);
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

int pkv_paged_attention_partitions_append(void* out, int out_dtype, const void* q,
                                          const void* k_new, const void* v_new, void* k_cache,
                                          void* v_cache, int kv_dtype,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_dim, int block_size, int num_blocks,
                                          int max_blocks_per_seq, float scale,
                                          int partition_size, const int32_t* work_list,
                                          int work_items, void* workspace,
                                          size_t workspace_bytes, int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  if ((st = append_args(&pl, k_new, v_new)) != PKV_OK) return st;
  return partitions_any(pl, kv_dtype, head_dim, work_list, work_items, stream);
}

int pkv_paged_attention_decode_step(void* out, int out_dtype, const void* q, const void* k_new,
                                    const void* v_new, const int32_t* cow_src, void* k_cache,
                                    void* v_cache, int kv_dtype, const int32_t* block_tables,
                                    const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int max_blocks_per_seq, float scale,
                                    int partition_size, const int32_t* work_list, int work_items,
                                    void* workspace, size_t workspace_bytes, int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  if ((st = append_args(&pl, k_new, v_new)) != PKV_OK) return st;
  if (!cow_src) return fail(PKV_EINVAL, "decode_step: null cow_src");
  pl.args.cow_src = cow_src;
  st = partitions_any(pl, kv_dtype, head_dim, work_list, work_items, stream);
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

int pkv_paged_attention_partitions_step(void* out, int out_dtype, const void* q,
                                        const void* k_new, const void* v_new,
                                        const int32_t* cow_src, void* k_cache, void* v_cache,
                                        int kv_dtype, const int32_t* block_tables,
                                        const int32_t* seq_lens, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, int max_blocks_per_seq, float scale,
                                        int partition_size, const int32_t* work_list,
                                        int work_items, void* workspace, size_t workspace_bytes,
                                        int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  if ((st = append_args(&pl, k_new, v_new)) != PKV_OK) return st;
  if (!cow_src) return fail(PKV_EINVAL, "partitions_step: null cow_src");
  pl.args.cow_src = cow_src;
  return partitions_any(pl, kv_dtype, head_dim, work_list, work_items, stream);
}

// The per-partition pass of a one-pass step over fork groups: work items name groups.
static int groups_pass(const DecodePlan& pl0, int kv_dtype, int head_dim, const int32_t* cow_src,
                       const int32_t* groups, int num_groups, int group_size,
                       const int32_t* work_list, int work_items, void* stream) {
  if (group_size < 1 || num_groups < 0 || work_items < 0)
    return fail(PKV_EINVAL, "step_groups: bad group_size, num_groups or work_items");
  const int64_t rows = (int64_t)group_size * pl0.group;
  if (rows != 1 && rows != 2 && rows != 4 && rows != 8)
    return fail(PKV_EINVAL, "step_groups: group_size x query heads per KV head must be 1, 2, 4 "
                "or 8 (got %lld)", (long long)rows);
  if (rows == 8 && head_dim > 128)
    return fail(PKV_EINVAL, "step_groups: 8 rows need head_dim <= 128");
  if (num_groups > kMaxListSeqs)
    return fail(PKV_EINVAL, "step_groups: at most %d groups", kMaxListSeqs);
  if (pl0.args.num_seqs > kMaxListSeqs)
    return fail(PKV_EINVAL, "step_groups: at most %d sequences", kMaxListSeqs);
  if (num_groups == 0 || work_items == 0) return ok();
  if (!groups || !work_list) return fail(PKV_EINVAL, "step_groups: null groups or work_list");
  if ((int64_t)work_items * pl0.args.num_kv_heads > INT32_MAX)
    return fail(PKV_EINVAL, "step_groups: work list too long");
  DecodePlan pl = pl0;
  DecodeArgs& a = pl.args;
  a.cow_src = cow_src;
  a.groups = groups;
  a.num_groups = num_groups;
  a.group_size = group_size;
  a.group_heads = pl0.group;
  a.work = reinterpret_cast<const uint32_t*>(work_list);
  a.work_items = work_items;
  return hip_status(launch_decode_partitions_groups(a, kv_dtype, head_dim, (int)rows,
                                                    (hipStream_t)stream),
                    "decode partitions (fork groups) launch");
}

int pkv_paged_attention_partitions_step_groups(
    void* out, int out_dtype, const void* q, const void* k_new, const void* v_new,
    const int32_t* cow_src, void* k_cache, void* v_cache, int kv_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
    float scale, int partition_size, const int32_t* groups, int num_groups, int group_size,
    const int32_t* work_list, int work_items, void* workspace, size_t workspace_bytes,
    int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  if ((st = append_args(&pl, k_new, v_new)) != PKV_OK) return st;
  return groups_pass(pl, kv_dtype, head_dim, cow_src, groups, num_groups, group_size, work_list,
                     work_items, stream);
}

int pkv_paged_attention_decode_step_groups(
    void* out, int out_dtype, const void* q, const void* k_new, const void* v_new,
    const int32_t* cow_src, void* k_cache, void* v_cache, int kv_dtype,
    const int32_t* block_tables, const int32_t* seq_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
    float scale, int partition_size, const int32_t* groups, int num_groups, int group_size,
    const int32_t* work_list, int work_items, void* workspace, size_t workspace_bytes,
    int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  if ((st = append_args(&pl, k_new, v_new)) != PKV_OK) return st;
  st = groups_pass(pl, kv_dtype, head_dim, cow_src, groups, num_groups, group_size, work_list,
                   work_items, stream);
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

static int prefix_pass(const DecodePlan& pl, int kv_dtype, int head_dim, int block_size,
                       const int32_t* members, int num_members, int prefix_partitions,
                       void* stream) {
  if (num_members < 0 || prefix_partitions < 0)
    return fail(PKV_EINVAL, "prefix: negative member or partition count");
  if (num_members == 0 || prefix_partitions == 0) return ok();
  if (!members) return fail(PKV_EINVAL, "prefix: null members");
  const DecodeArgs& d = pl.args;
  if (!prefix_supported(kv_dtype, head_dim, pl.group, d.part, d.bs_log2))
    return fail(PKV_EINVAL, "prefix: needs fp16/bf16 KV, head_dim 128 and at most 256 blocks "
                "per partition");
  if ((int64_t)prefix_partitions * d.part > (int64_t)d.max_blocks * block_size ||
      prefix_partitions >= d.pmax)
    return fail(PKV_EINVAL, "prefix: %d shared partitions leave no partition of the sequences' "
                "own", prefix_partitions);
  const int per = prefix_chunk_seqs(pl.group);
  if ((int64_t)d.num_kv_heads * ((num_members + per - 1) / per) > INT32_MAX)
    return fail(PKV_EINVAL, "prefix: too many members");
  PrefixArgs a;
  a.out = d.out;
  a.out_dtype = d.out_dtype;
  a.seq_lens = d.seq_lens;
  a.q = d.q;
  a.k_cache = d.k_cache;
  a.v_cache = d.v_cache;
  a.block_tables = d.block_tables;
  a.members = members;
  a.ws_ml = d.ws_ml;
  a.ws_acc = d.ws_acc;
  a.num_members = num_members;
  a.prefix_parts = prefix_partitions;
  a.num_seqs = d.num_seqs;
  a.num_q_heads = d.num_q_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.num_blocks = d.num_blocks;
  a.max_blocks = d.max_blocks;
  a.bs_log2 = d.bs_log2;
  a.part = d.part;
  a.pmax = d.pmax;
  a.scale_log2 = d.scale_log2;
  return hip_status(launch_prefix(a, kv_dtype, pl.group, (hipStream_t)stream),
                    "shared-prefix launch");
}

int pkv_paged_attention_prefix(void* out, int out_dtype, const void* q, const void* k_cache,
                               const void* v_cache, int kv_dtype, const int32_t* block_tables,
                               const int32_t* seq_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, float scale, int partition_size,
                               const int32_t* members, int num_members, int prefix_partitions,
                               void* workspace, size_t workspace_bytes, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables,
                       seq_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, scale, partition_size, workspace,
                       workspace_bytes, PKV_KV_STREAM);
  if (st != PKV_OK || num_seqs == 0) return st;
  return prefix_pass(pl, kv_dtype, head_dim, block_size, members, num_members, prefix_partitions,
                     stream);
}

int pkv_paged_attention_decode_shared(void* out, int out_dtype, const void* q,
                                      const void* k_cache, const void* v_cache, int kv_dtype,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int num_seqs, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks,
                                      int max_blocks_per_seq, float scale, int partition_size,
                                      const int32_t* members, int num_members,
                                      int prefix_partitions, const int32_t* work_list,
                                      int work_items, void* workspace, size_t workspace_bytes,
                                      int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = prefix_pass(pl, kv_dtype, head_dim, block_size, members, num_members, prefix_partitions,
                   stream);
  if (st != PKV_OK) return st;
  st = partitions_list(pl, kv_dtype, head_dim, work_list, work_items, stream);
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

int pkv_paged_attention_reduce(void* out, int out_dtype, const int32_t* seq_lens, int num_seqs,
                               int num_q_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int partition_size, const void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (out_dtype != PKV_F32 && out_dtype != PKV_F16 && out_dtype != PKV_BF16)
    return fail(PKV_EDTYPE, "reduce: unknown out dtype %d", out_dtype);
  if (num_seqs < 0 || num_seqs > 65535 || num_q_heads <= 0) return fail(PKV_EINVAL, "reduce: bad sizes");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return fail(PKV_EINVAL, "reduce: bad head_dim");
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256) return fail(PKV_EINVAL, "reduce: bad block_size");
  if (max_blocks_per_seq <= 0 || (int64_t)max_blocks_per_seq * block_size >= INT32_MAX)
    return fail(PKV_EINVAL, "reduce: max_blocks_per_seq out of range");
  if (partition_size == 0) partition_size = 512;
  if (partition_size < 32 || partition_size > 2048 || partition_size % 32 != 0 || partition_size % block_size != 0)
    return fail(PKV_EINVAL, "reduce: bad partition_size");
  const int64_t pmax = ((int64_t)max_blocks_per_seq * block_size + partition_size - 1) / partition_size;
  if (pmax <= 1 || num_seqs == 0) return ok();  // nothing spans two partitions
  if (pmax > 65535) return fail(PKV_EINVAL, "reduce: too many partitions per sequence");
  const WsLayout ws = ws_layout(num_seqs, num_q_heads, pmax, head_dim);
  if (!workspace || workspace_bytes < ws.total)
    return fail(PKV_EWORKSPACE, "reduce: workspace of %zu bytes needed, %zu given", ws.total, workspace_bytes);
  if (!aligned16(workspace)) return fail(PKV_EINVAL, "reduce: workspace must be 16-byte aligned");
  if (!out || !seq_lens) return fail(PKV_EINVAL, "reduce: null pointer");
  if (!aligned16(out)) return fail(PKV_EINVAL, "reduce: out must be 16-byte aligned");
  DecodeArgs a = {};
  a.out = out;
  a.seq_lens = seq_lens;
  a.ws_ml = (float*)((const char*)workspace + ws.ml_off);
  a.ws_acc = (float*)((const char*)workspace + ws.acc_off);
  a.sched = nullptr;
  a.sched_static = 0;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_blocks = max_blocks_per_seq;
  a.bs_log2 = log2i(block_size);
  a.part = partition_size;
  a.pmax = (int)pmax;
  a.out_dtype = out_dtype;
  return hip_status(launch_decode_reduce(a, head_dim, (hipStream_t)stream), "decode reduce launch");
}

int pkv_paged_attention_decode(void* out, int out_dtype, const void* q, const void* k_cache,
                               const void* v_cache, int kv_dtype, const int32_t* block_tables,
                               const int32_t* seq_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, float scale, int partition_size,
                               void* workspace, size_t workspace_bytes, int kv_policy, void* stream) {
  DecodePlan pl;
  int st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, kv_policy);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = hip_status(launch_decode_partitions(pl.args, kv_dtype, head_dim, pl.group, (hipStream_t)stream),
                  "decode partitions launch");
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

int pkv_paged_attention_decode_noalloc(void* out, int out_dtype, const void* q,
                                       const void* k_cache, const void* v_cache, int kv_dtype,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks,
                                       int max_blocks_per_seq, float scale, int partition_size,
                                       int kv_policy, void* stream) {
  void* ws = nullptr;
  int st = hip_status(static_workspace(&ws), "decode_noalloc: static scratch address");
  if (st != PKV_OK) return st;
  DecodePlan pl;
  st = plan_decode(&pl, out, out_dtype, q, k_cache, v_cache, kv_dtype, block_tables, seq_lens,
                   num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, scale, partition_size, ws, kStaticWorkspaceBytes, kv_policy);
  if (st == PKV_EWORKSPACE)
    return fail(PKV_EWORKSPACE, "decode_noalloc: these shapes need %zu bytes of split-K scratch; "
                "the static area holds %zu (use pkv_paged_attention_decode with a workspace, "
                "or longer partitions)", pl.ws_needed, kStaticWorkspaceBytes);
  if (st != PKV_OK || num_seqs == 0) return st;
  st = hip_status(launch_decode_partitions(pl.args, kv_dtype, head_dim, pl.group, (hipStream_t)stream),
                  "decode partitions launch");
  if (st != PKV_OK || pl.args.pmax <= 1) return st;
  return hip_status(launch_decode_reduce(pl.args, head_dim, (hipStream_t)stream), "decode reduce launch");
}

int pkv_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return ok();
  if (!workspace || workspace_bytes < kWsHeaderBytes)
    return fail(PKV_EINVAL, "workspace_init: a workspace holds at least %zu bytes", kWsHeaderBytes);
  if (!aligned16(workspace)) return fail(PKV_EINVAL, "workspace_init: workspace must be 16-byte aligned");
  return hip_status(launch_sched_init(static_cast<unsigned long long*>(workspace), (hipStream_t)stream),
                    "workspace init launch");
}

int pkv_debug_timeline(void* buf, int capacity) {
  if (capacity < 0 || (capacity > 0 && !buf)) return fail(PKV_EINVAL, "debug_timeline: bad buffer");
  if (capacity > 0 && (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return fail(PKV_EINVAL, "debug_timeline: buffer must be 16-byte aligned");
  g_timeline_cap.store(0, std::memory_order_release);
  g_timeline.store(static_cast<uint32_t*>(buf), std::memory_order_release);
  g_timeline_cap.store(capacity, std::memory_order_release);
  return ok();
}

int pkv_read_probe(const void* buf, size_t buf_bytes, int tile_bytes, const int32_t* tile_ids,
                   int num_tiles, int tiles_per_group, int flags, uint32_t sentinel,
                   uint32_t* sink, void* stream) {
  if (flags & ~PKV_PROBE_NONTEMPORAL) return fail(PKV_EINVAL, "read_probe: unknown flag bits");
  if (!is_pow2(tile_bytes) || tile_bytes < 256 || tile_bytes > (1 << 20))
    return fail(PKV_EINVAL, "read_probe: tile_bytes must be a power of two in [256, 1 MiB]");
  if (num_tiles < 0 || tiles_per_group < 1 || tiles_per_group > 1024)
    return fail(PKV_EINVAL, "read_probe: num_tiles >= 0 and tiles_per_group in [1, 1024]");
  if (num_tiles == 0) return ok();
  if (!buf || !tile_ids || !sink) return fail(PKV_EINVAL, "read_probe: null pointer");
  if (!aligned16(buf)) return fail(PKV_EINVAL, "read_probe: buffer must be 16-byte aligned");
  if (buf_bytes < (size_t)tile_bytes) return fail(PKV_EINVAL, "read_probe: buffer holds no tile");
  ProbeArgs a;
  a.buf = static_cast<const unsigned char*>(buf);
  a.tile_ids = tile_ids;
  a.num_tile_slots = (int64_t)(buf_bytes / (size_t)tile_bytes);
  a.num_tiles = num_tiles;
  a.tiles_per_group = tiles_per_group;
  a.tile_log2 = log2i(tile_bytes);
  a.sentinel = sentinel;
  a.sink = sink;
  a.nontemporal = (flags & PKV_PROBE_NONTEMPORAL) != 0;
  return hip_status(launch_read_probe(a, (hipStream_t)stream), "read probe launch");
}

int pkv_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache, int dtype,
                          const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, void* stream) {
  if (!dtype_ok(dtype)) return fail(PKV_EDTYPE, "reshape_and_cache: unknown dtype %d", dtype);
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "reshape_and_cache: bad sizes");
  const int64_t row_bytes = (int64_t)head_dim * elem_bytes(dtype);
  if (row_bytes % 16 != 0) return fail(PKV_EINVAL, "reshape_and_cache: head_dim*elem_bytes must be a multiple of 16");
  if ((int64_t)num_kv_heads * row_bytes / 16 > 65535LL * 256)
    return fail(PKV_EINVAL, "reshape_and_cache: token rows too large");
  if (!is_pow2(block_size) || block_size > 256) return fail(PKV_EINVAL, "reshape_and_cache: block_size must be a power of two <= 256");
  if (num_blocks <= 0 || (int64_t)num_blocks * block_size >= INT32_MAX)
    return fail(PKV_EINVAL, "reshape_and_cache: num_blocks out of range");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return fail(PKV_EINVAL, "reshape_and_cache: null pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_EINVAL, "reshape_and_cache: buffers must be 16-byte aligned");
  CacheWriteArgs a;
  a.k = k;
  a.v = v;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.row_bytes = (int)row_bytes;
  a.bs_log2 = log2i(block_size);
  a.num_blocks = num_blocks;
  return hip_status(launch_reshape_and_cache(a, (hipStream_t)stream), "reshape_and_cache launch");
}

int pkv_copy_blocks(void* k_cache, void* v_cache, int dtype, const int32_t* src_dst_pairs,
                    int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    void* stream) {
  if (!dtype_ok(dtype)) return fail(PKV_EDTYPE, "copy_blocks: unknown dtype %d", dtype);
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "copy_blocks: bad sizes");
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return fail(PKV_EINVAL, "copy_blocks: block bytes must be a multiple of 16");
  if ((block_bytes / 16 + 4095) / 4096 > 65535) return fail(PKV_EINVAL, "copy_blocks: blocks too large");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !src_dst_pairs) return fail(PKV_EINVAL, "copy_blocks: null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(PKV_EINVAL, "copy_blocks: caches must be 16-byte aligned");
  CopyBlocksArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.pairs = src_dst_pairs;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.block_bytes = block_bytes;
  return hip_status(launch_copy_blocks(a, (hipStream_t)stream), "copy_blocks launch");
}

}  // extern "C"
