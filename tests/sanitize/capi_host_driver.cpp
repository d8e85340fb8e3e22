// Host-side logic of the C ABI (capi.cpp, shapes.cpp, errors.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU. The kernel launches are replaced by stubs that check
// what the validated arguments say and launch nothing; the device pointers passed in are
// never dereferenced on the host, so any aligned non-null value stands for one.
//
// usage: capi_host_driver SEED SCENARIOS     prints "ok N scenarios" on success
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <initializer_list>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "launch.h"
#include "pagedkv.h"

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(2);                                                         \
    }                                                                       \
  } while (0)

// ---- stubs for the device side ----------------------------------------------------------
static int g_launches = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace pkv {
static void check_decode_args(const DecodeArgs& a) {
  CHECK(a.num_seqs > 0 && a.num_q_heads > 0 && a.num_kv_heads > 0);
  CHECK(a.num_q_heads % a.num_kv_heads == 0);
  CHECK(a.part >= 32 && a.part <= 2048 && a.part % 32 == 0);
  CHECK((a.part >> a.bs_log2) << a.bs_log2 == a.part);
  CHECK(a.pmax >= 1 && (int64_t)a.pmax * a.part >= (int64_t)a.max_blocks << a.bs_log2);
  CHECK(a.kv_cached == 0 || a.kv_cached == 1);
  CHECK(a.work == nullptr || a.work_items > 0);
  CHECK(a.pmax <= 1 || (a.ws_ml != nullptr && a.ws_acc != nullptr));
}
// the occupancy query of pkv_decode_ticketed_items: no kernel, a made-up resident count
static hipError_t ticket_query(const DecodeArgs& a, int* ticketed) {
  CHECK(a.work_items > 0 && a.num_kv_heads > 0);
  const int units = a.num_kv_heads * a.work_items;
  *ticketed = units > 3 * 512 / 2 ? 256 : 0;
  return hipSuccess;
}
hipError_t launch_decode_partitions(const DecodeArgs& a, int, int, int group, hipStream_t,
                                    int* ticketed) {
  if (ticketed) return ticket_query(a, ticketed);
  check_decode_args(a);
  CHECK(group == a.num_q_heads / a.num_kv_heads);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_partitions_cow(const DecodeArgs& a, int, int, int group, hipStream_t,
                                        int* ticketed) {
  CHECK(ticketed != nullptr);   // capi reaches the copy-on-write kernels directly only to query
  CHECK(group == a.num_q_heads / a.num_kv_heads);
  return ticket_query(a, ticketed);
}
hipError_t launch_decode_partitions_groups(const DecodeArgs& a, int, int head_dim, int rows,
                                           hipStream_t, int* ticketed) {
  if (ticketed) {
    CHECK(rows == a.group_size * a.group_heads);
    return ticket_query(a, ticketed);
  }
  check_decode_args(a);
  CHECK(a.groups != nullptr && a.num_groups > 0 && a.group_size >= 1);
  CHECK(a.group_heads == a.num_q_heads / a.num_kv_heads);
  CHECK(rows == a.group_size * a.group_heads);
  CHECK(rows == 1 || rows == 2 || rows == 4 || rows == 8);
  CHECK(rows < 8 || head_dim <= 128);
  CHECK(a.work != nullptr && a.k_new != nullptr && a.v_new != nullptr);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t) {
  CHECK(a.pmax > 1 && a.ws_ml != nullptr && a.ws_acc != nullptr);
  CHECK(head_dim == 64 || head_dim == 128 || head_dim == 256);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefix(const PrefixArgs& a, int, int, hipStream_t) {
  CHECK(a.num_members > 0 && a.prefix_parts > 0 && a.prefix_parts < a.pmax);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_reshape_and_cache(const CacheWriteArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_copy_blocks(const CopyBlocksArgs&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_read_probe(const ProbeArgs& a, hipStream_t) {
  CHECK(a.num_tiles > 0 && a.tiles_per_group >= 1 && a.tiles_per_group <= 1024);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_sched_init(unsigned long long*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t static_workspace(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull));
  return hipSuccess;
}
}  // namespace pkv

// ---- random inputs -------------------------------------------------------------------------
static uint64_t g_state = 1;
static uint32_t rnd() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
static int pick(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }
template <class T> static T choose(std::initializer_list<T> v) {
  return *(v.begin() + rnd() % v.size());
}

static void* fake(uintptr_t tag) { return reinterpret_cast<void*>(0x100000ull * tag); }

struct Batch {
  int B, W, bs, NB;
  std::vector<int32_t> tables, lens;
};

// tables with some shared leading blocks, some out-of-pool entries, ragged lengths
static Batch random_batch() {
  Batch t;
  t.B = pick(0, 40);
  t.bs = choose<int>({8, 16, 32, 64});
  t.W = pick(1, 24);
  t.NB = pick(1, 200);
  t.tables.assign((size_t)std::max(t.B, 1) * t.W, -1);
  t.lens.assign((size_t)std::max(t.B, 1), 0);
  const int share = pick(0, t.W);
  for (int b = 0; b < t.B; ++b) {
    for (int j = 0; j < t.W; ++j) {
      const int r = pick(0, 19);
      int32_t id = pick(0, t.NB - 1);
      if (j < share && b > 0 && r < 15) id = t.tables[j];  // first sequence's block
      if (r == 19) id = choose<int>({-1, -7, t.NB, t.NB + 5});
      t.tables[(size_t)b * t.W + j] = id;
    }
    t.lens[b] = choose<int>({pick(0, t.W * t.bs), pick(-5, 0), t.W * t.bs + pick(0, 100),
                        pick(1, t.bs)});
  }
  return t;
}

static void work_lists(const Batch& t) {
  const int part = choose<int>({32, 64, 128, 256, 512, 1024, 2048, 0, 48, 4096});
  int n = pkv_decode_work_list(t.lens.data(), t.B, t.W, t.bs, part, nullptr, 0);
  if (n >= 0) {
    std::vector<int32_t> items((size_t)n + 1);
    CHECK(pkv_decode_work_list(t.lens.data(), t.B, t.W, t.bs, part, items.data(), n) == n);
    if (n > 0) CHECK(pkv_decode_work_list(t.lens.data(), t.B, t.W, t.bs, part, items.data(), n - 1) < 0);
    const int policy = pkv_decode_kv_policy(t.tables.data(), t.lens.data(), t.B, t.W, t.bs, t.NB,
                                            items.data(), n, part == 0 ? 512 : part);
    if (part == 0 || part % t.bs == 0) CHECK(policy == PKV_KV_STREAM || policy == PKV_KV_CACHED);
    // the private tail: a permutation of the list, whatever the tail
    std::vector<int32_t> re(items.begin(), items.begin() + n);
    const int tail = choose<int>({0, 1, pick(0, n + 3), n, -1});
    const int moved = pkv_decode_work_list_private_tail(t.tables.data(), t.lens.data(), t.B, t.W,
                                                        t.bs, t.NB, part, tail, re.data(), n);
    CHECK(moved <= std::max(tail, 0));
    if (moved == 0) CHECK(std::equal(re.begin(), re.end(), items.begin()));
    std::vector<int32_t> a(items.begin(), items.begin() + n), b2(re);
    std::sort(a.begin(), a.end());
    std::sort(b2.begin(), b2.end());
    CHECK(a == b2);
  }
  {
    const int hkv = choose<int>({1, 8, 40, 0});
    const int ti = pkv_decode_ticketed_items(choose<int>({PKV_F16, PKV_BF16, PKV_F32, 9}),
                                             choose<int>({64, 128, 256, 100}),
                                             hkv * choose<int>({1, 2, 4, 8, 3}), hkv, t.bs,
                                             choose<int>({0, 512, 2048, 48}), pick(-1, 5000),
                                             pick(-1, 3), choose<int>({1, 2, 4, 0}));
    CHECK(ti <= 5000);
  }
  int rows = -1;
  const int pack = choose<int>({0, 8, 16, 64, 256, 1000});
  n = pkv_decode_work_list_packed(t.lens.data(), t.B, t.W, t.bs, part, pack, nullptr, 0, &rows);
  if (n >= 0) {
    std::vector<int32_t> items((size_t)n + 1);
    CHECK(pkv_decode_work_list_packed(t.lens.data(), t.B, t.W, t.bs, part, pack, items.data(), n,
                                      &rows) == n);
    CHECK(rows >= 0 && rows <= n);
  }
  const int p = pkv_decode_kv_policy(t.tables.data(), t.lens.data(), t.B, t.W, t.bs, t.NB,
                                     nullptr, 0, 0);
  CHECK(p == PKV_KV_STREAM || p == PKV_KV_CACHED || t.NB <= 0);
}

static void shared_plan(const Batch& t) {
  const int part = choose<int>({32, 64, 128, 256, 512});
  std::vector<int32_t> members((size_t)std::max(t.B, 1));
  int nm = -1, pp = -1;
  const int minm = pick(1, 4);
  const int n = pkv_decode_plan_shared_prefix(t.tables.data(), t.lens.data(), t.B, t.W, t.bs,
                                              part, minm, members.data(), &nm, &pp, nullptr, 0);
  if (n < 0) return;
  std::vector<int32_t> items((size_t)n + 1);
  CHECK(pkv_decode_plan_shared_prefix(t.tables.data(), t.lens.data(), t.B, t.W, t.bs, part, minm,
                                      members.data(), &nm, &pp, items.data(), n) == n);
  CHECK(nm >= 0 && nm <= t.B && pp >= 0);
  pkv_decode_kv_policy(t.tables.data(), t.lens.data(), t.B, t.W, t.bs, t.NB, items.data(), n,
                       part);
}

static void fork_groups(const Batch& t) {
  std::vector<int32_t> cow((size_t)std::max(t.B, 1));
  for (int b = 0; b < t.B; ++b) cow[b] = choose<int>({-1, -1, pick(0, t.NB + 2), -9});
  const int size = choose<int>({1, 2, 3, 4, 8, 0});
  const int32_t* cs = choose({cow.data(), (int32_t*)nullptr});
  const int n = pkv_decode_plan_fork_groups(t.tables.data(), t.lens.data(), cs, t.B, t.W, t.bs,
                                            t.NB, size, nullptr, nullptr, 0);
  if (n < 0) return;
  CHECK(n <= t.B && (t.B == 0 || n >= 1));
  std::vector<int32_t> groups((size_t)std::max(n, 1) * size), glens((size_t)std::max(n, 1));
  CHECK(pkv_decode_plan_fork_groups(t.tables.data(), t.lens.data(), cs, t.B, t.W, t.bs, t.NB,
                                    size, groups.data(), glens.data(), n) == n);
  std::vector<int> seen((size_t)std::max(t.B, 1), 0);
  for (int g = 0; g < n; ++g)
    for (int j = 0; j < size; ++j) {
      const int m = groups[(size_t)g * size + j];
      if (m >= 0) {
        CHECK(m < t.B);
        ++seen[m];
      }
    }
  for (int b = 0; b < t.B; ++b) CHECK(seen[b] == 1);
}

static void decode_calls(const Batch& t) {
  const int kv = choose<int>({PKV_F32, PKV_F16, PKV_BF16, 7});
  const int out_dt = choose<int>({kv, PKV_F32, PKV_F16});
  const int hkv = choose<int>({1, 2, 8, 40});
  const int hq = hkv * choose<int>({1, 2, 3, 4, 8});
  const int d = choose<int>({64, 128, 256, 96});
  const int part = choose<int>({0, 32, 256, 512, 1536, 2048, 4096, 48});
  const int policy = choose<int>({PKV_KV_STREAM, PKV_KV_CACHED, 2});
  const int B = std::min(t.B, 40);
  const size_t need = pkv_decode_workspace_bytes(B, hq, t.W, t.bs, d, part);
  void* ws = need ? fake(9) : nullptr;
  const size_t wsb = need ? need + (size_t)pick(0, 64) * 16 : 0;
  void* out = choose({fake(1), (void*)nullptr, (void*)((char*)fake(1) + 8)});
  const int32_t* tabs = reinterpret_cast<const int32_t*>(fake(5));
  const int32_t* lens = reinterpret_cast<const int32_t*>(fake(6));
  int st = pkv_paged_attention_decode(out, out_dt, fake(2), fake(3), fake(4), kv, tabs, lens, B, hq,
                                      hkv, d, t.bs, t.NB, t.W, 0.1f, part, ws, wsb, policy, nullptr);
  CHECK(st <= 0);
  st = pkv_paged_attention_decode_noalloc(out, out_dt, fake(2), fake(3), fake(4), kv, tabs, lens, B,
                                          hq, hkv, d, t.bs, t.NB, t.W, 0.1f, part, policy, nullptr);
  CHECK(st <= 0);
  // a host work list (its device copy is a fake pointer; the count is what matters here)
  const int p2 = part == 0 ? 512 : part;
  const int n = pkv_decode_work_list(t.lens.data(), B, t.W, t.bs, p2, nullptr, 0);
  const int32_t* wl = reinterpret_cast<const int32_t*>(fake(7));
  if (n >= 0) {
    st = pkv_paged_attention_decode_list(out, out_dt, fake(2), fake(3), fake(4), kv, tabs, lens, B,
                                         hq, hkv, d, t.bs, t.NB, t.W, 0.1f, p2, wl, n, ws, wsb,
                                         policy, nullptr);
    CHECK(st <= 0);
    st = pkv_paged_attention_decode_step(out, out_dt, fake(2), fake(10), fake(11),
                                         reinterpret_cast<const int32_t*>(fake(12)), fake(3),
                                         fake(4), kv, tabs, lens, B, hq, hkv, d, t.bs, t.NB, t.W,
                                         0.1f, p2, choose({wl, (const int32_t*)nullptr}),
                                         choose<int>({n, 0, -1}), ws, wsb, policy, nullptr);
    CHECK(st <= 0);
    st = pkv_paged_attention_decode_step_groups(
        out, out_dt, fake(2), fake(10), fake(11), reinterpret_cast<const int32_t*>(fake(12)),
        fake(3), fake(4), kv, tabs, lens, B, hq, hkv, d, t.bs, t.NB, t.W, 0.1f, p2,
        choose({reinterpret_cast<const int32_t*>(fake(14)), (const int32_t*)nullptr}),
        pick(-1, B), choose<int>({1, 2, 4, 3, 0}), choose({wl, (const int32_t*)nullptr}),
        choose<int>({n, 0, -1}), ws, wsb, policy, nullptr);
    CHECK(st <= 0);
    st = pkv_paged_attention_decode_shared(
        out, out_dt, fake(2), fake(3), fake(4), kv, tabs, lens, B, hq, hkv, d, t.bs, t.NB, t.W,
        0.1f, p2, reinterpret_cast<const int32_t*>(fake(13)), pick(0, B), pick(0, 3), wl, n, ws,
        wsb, policy, nullptr);
    CHECK(st <= 0);
  }
  st = pkv_paged_attention_reduce(out, out_dt, lens, B, hq, d, t.bs, t.W, part, ws, wsb, nullptr);
  CHECK(st <= 0);
  pkv_decode_default_partition(B, hq, hkv, d, t.bs, t.W);
  pkv_decode_workspace_bytes(pick(-1, 70000), pick(-1, 128), pick(-1, 1 << 20), t.bs, d, part);
}

static void cache_calls(const Batch& t) {
  const int dt = choose<int>({PKV_F32, PKV_F16, PKV_BF16, 5});
  const int d = choose<int>({64, 128, 100});
  int st = pkv_reshape_and_cache(fake(1), fake(2), fake(3), fake(4), dt,
                                 reinterpret_cast<const int32_t*>(fake(5)), pick(-1, 300),
                                 pick(0, 40), d, t.bs, t.NB, nullptr);
  CHECK(st <= 0);
  st = pkv_copy_blocks(fake(3), fake(4), dt, reinterpret_cast<const int32_t*>(fake(5)),
                       pick(-1, 300), pick(0, 40), d, t.bs, t.NB, nullptr);
  CHECK(st <= 0);
  st = pkv_read_probe(fake(1), (size_t)pick(0, 1 << 20) << 10, choose({256, 4096, 3000, 1 << 21}),
                      reinterpret_cast<const int32_t*>(fake(2)), pick(-1, 5000), pick(0, 1100),
                      pick(0, 3), 7u, reinterpret_cast<uint32_t*>(fake(3)), nullptr);
  CHECK(st <= 0);
  st = pkv_decode_workspace_init(fake(9), (size_t)pick(0, 1000), nullptr);
  CHECK(st <= 0);
}

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int n = argc > 2 ? std::atoi(argv[2]) : 1000;
  g_state = seed * 0x9E3779B97F4A7C15ull + 1;
  for (int i = 0; i < n; ++i) {
    const Batch t = random_batch();
    work_lists(t);
    shared_plan(t);
    fork_groups(t);
    decode_calls(t);
    cache_calls(t);
    if (i % 97 == 0) {
      uint32_t buf[64];
      pkv_debug_timeline(buf, 8);
      pkv_debug_timeline(nullptr, 0);
    }
  }
  std::printf("ok %d scenarios, %d launches\n", n, g_launches);
  return 0;
}
