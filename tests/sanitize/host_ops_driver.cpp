// Random-operation driver over the host-only part of libpagedkv (block manager, prefix cache,
// continuous-batching scheduler, pool sizing), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py. Every pkv_bm_*, pkv_sched_*
// and pkv_kv_pool_plan entry point is called with valid and invalid arguments; after each
// manager operation the pool accounting is checked (blocks held + available = pool size,
// and refcounts equal the number of table entries naming each block). Exits non-zero on a
// broken invariant; the sanitizers abort on any memory error or undefined behaviour.
//
//   host_ops_driver <seed> <scenarios>
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedkv.h"

namespace {

std::mt19937_64 rng;

int64_t pick(int64_t lo, int64_t hi) {  // uniform on [lo, hi]
  return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
}

#define CHECK(c)                                                                     \
  do {                                                                               \
    if (!(c)) {                                                                      \
      std::fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #c);       \
      std::exit(3);                                                                  \
    }                                                                                \
  } while (0)

void check_pool(const pkv_bm* bm, int nb, const std::vector<int64_t>& live) {
  int64_t st[8];
  CHECK(pkv_bm_stats(bm, st) == PKV_OK);
  CHECK(st[0] + st[1] == nb);
  CHECK(st[5] == (int64_t)live.size());
  std::vector<int> refs(nb, 0);
  std::vector<int32_t> tab(4096);
  for (int64_t s : live) {
    int ntok = -1;
    const int n = pkv_bm_table(bm, s, nullptr, 0, &ntok);   // size query
    CHECK(n >= 0 && ntok >= 0);
    if ((int)tab.size() < n) tab.resize(n);
    CHECK(pkv_bm_table(bm, s, tab.data(), n, nullptr) == n);
    for (int j = 0; j < n; ++j) {
      CHECK(tab[j] >= 0 && tab[j] < nb);
      ++refs[tab[j]];
    }
  }
  int64_t held = 0, shared = 0;
  for (int b = 0; b < nb; ++b) {
    CHECK(pkv_bm_refcount(bm, b) == refs[b]);
    held += refs[b] > 0;
    shared += refs[b] > 1;
  }
  CHECK(shared == st[2]);
  CHECK(held <= st[0]);   // the rest of "held" is nothing: cached blocks count as available
}

void manager_scenario() {
  const int nb = (int)pick(1, 48);
  const int bs = 1 << pick(0, 4);
  std::vector<int32_t> order(nb);
  for (int i = 0; i < nb; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_bm* bm = pkv_bm_create(nb, bs, pick(0, 1) ? order.data() : nullptr);
  CHECK(bm != nullptr);
  std::vector<int64_t> live;
  int64_t next = 0;
  const int ops = (int)pick(1, 120);
  for (int i = 0; i < ops; ++i) {
    const int64_t s = live.empty() ? 12345 : live[pick(0, (int64_t)live.size() - 1)];
    int32_t slot, cs, cd;
    switch (pick(0, 14)) {
      case 0: {
        if (pkv_bm_add_seq(bm, next, (int)pick(0, 3 * bs + 3)) == PKV_OK) live.push_back(next);
        ++next;
        break;
      }
      case 1:
        if (pkv_bm_fork(bm, s, next) == PKV_OK) live.push_back(next);
        ++next;
        break;
      case 2:
        if (pkv_bm_share_prefix(bm, s, next, (int)pick(0, 3)) == PKV_OK) live.push_back(next);
        ++next;
        break;
      case 3:
        pkv_bm_append_slot(bm, s, &slot, pick(0, 1) ? &cs : nullptr, pick(0, 1) ? &cd : nullptr);
        break;
      case 4:
      case 5: {
        const int n = live.empty() ? 0 : (int)pick(0, 4);
        std::vector<int64_t> batch(n);
        for (int k = 0; k < n; ++k) batch[k] = live[pick(0, (int64_t)live.size() - 1)];
        std::vector<int32_t> slots(n + 1), pairs(2 * n + 2), src(n + 1);
        int ncow = -1;
        const int st = pkv_bm_append_step(bm, batch.data(), n, slots.data(), pairs.data(), &ncow,
                                          pick(0, 1) ? src.data() : nullptr);
        if (st == PKV_OK) CHECK(ncow >= 0 && ncow <= n);
        ncow = -1;
        pkv_bm_append_slots(bm, batch.data(), n, slots.data(), pairs.data(), &ncow);
        break;
      }
      case 6:
        pkv_bm_extend(bm, s, (int)pick(0, 2 * bs + 2), pick(0, 1) ? &cs : nullptr, nullptr);
        break;
      case 7:
        if (pkv_bm_free_seq(bm, s) == PKV_OK)
          for (size_t k = 0; k < live.size(); ++k)
            if (live[k] == s) {
              live.erase(live.begin() + (long)k);
              break;
            }
        break;
      case 8: {
        int ntok = 0;
        const int n = pkv_bm_table(bm, s, nullptr, 0, &ntok);
        if (n > 0) {
          std::vector<int32_t> out(n);
          CHECK(pkv_bm_table(bm, s, out.data(), (int)pick(1, n), nullptr) == n);
        }
        if (ntok > 0) {
          const int start = (int)pick(0, ntok - 1);
          std::vector<int32_t> out(ntok);
          CHECK(pkv_bm_slots(bm, s, start, ntok - start, out.data()) == PKV_OK);
        }
        pkv_bm_slots(bm, s, ntok, 1, &slot);           // past the end: refused
        break;
      }
      case 9: {
        const int n = (int)live.size();
        const int width = (int)pick(1, 8);
        std::vector<int32_t> tables((size_t)n * width + 1), lens(n + 1);
        pkv_bm_build_tables(bm, live.data(), n, tables.data(), width, lens.data());
        pkv_bm_build_tables(bm, live.data(), 0, nullptr, width, nullptr);
        break;
      }
      case 10:
      case 11: {
        // prompts over a 2-token vocabulary, so leading blocks repeat and hit the cache
        const int n = (int)pick(0, 3 * bs + 2);
        std::vector<int32_t> toks(n + 1);
        const int64_t pat = pick(0, 1 << 20);
        for (int k = 0; k < n; ++k) toks[k] = (int32_t)((pat >> (k % 20)) & 1);
        int cached = -1;
        if (pkv_bm_add_seq_cached(bm, next, n ? toks.data() : nullptr, n,
                                  pick(0, 1) ? &cached : nullptr) == PKV_OK)
          live.push_back(next);
        ++next;
        int64_t ps[4];
        CHECK(pkv_bm_prefix_stats(bm, ps) == PKV_OK);
        break;
      }
      case 12:
        pkv_bm_refcount(bm, (int32_t)pick(-2, nb + 2));
        break;
      case 13:
        // invalid arguments are refused, never dereferenced
        CHECK(pkv_bm_add_seq(nullptr, 0, 1) < 0);
        CHECK(pkv_bm_add_seq(bm, next, -1) < 0);
        CHECK(pkv_bm_append_step(bm, nullptr, 1, nullptr, nullptr, nullptr, nullptr) < 0);
        CHECK(pkv_bm_table(bm, s, nullptr, 1, nullptr) < 0 || live.empty());
        CHECK(pkv_bm_stats(bm, nullptr) < 0);
        break;
      default:
        pkv_bm_free_seq(bm, 987654321);
        break;
    }
    check_pool(bm, nb, live);
  }
  pkv_bm_destroy(bm);
}

void scheduler_scenario() {
  const int nb = (int)pick(1, 64);
  const int bs = 1 << pick(0, 4);
  pkv_bm* bm = pkv_bm_create(nb, bs, nullptr);
  CHECK(bm != nullptr);
  const int max_seqs = (int)pick(1, 8);
  const int budget = (int)pick(max_seqs, 64);
  const int watermark = (int)pick(0, 2);
  CHECK(pkv_sched_create(bm, bs + 1, max_seqs, budget, watermark) == nullptr || bs + 1 == bs);
  pkv_sched* s = pkv_sched_create(bm, bs, max_seqs, budget, watermark);
  CHECK(s != nullptr);
  std::vector<int64_t> batch(max_seqs), fin(max_seqs), adm(max_seqs), pre(max_seqs);
  std::vector<int64_t> slot_seq(budget);
  std::vector<int32_t> slots(budget), slot_pos(budget), pairs(2 * max_seqs);
  pkv_sched_step_out o{batch.data(), slots.data(), slot_seq.data(), slot_pos.data(),
                       pairs.data(), fin.data(), adm.data(), pre.data(), 0, 0, 0, 0, 0, 0};
  int64_t req = 0;
  const int steps = (int)pick(1, 80);
  for (int i = 0; i < steps; ++i) {
    for (int k = (int)pick(0, 2); k > 0; --k) {
      pkv_sched_add_request(s, req, (int)pick(-1, 24), (int)pick(-1, 12));
      pkv_sched_add_request(s, req, 1, 1);   // the id now exists, or was refused: either way fine
      ++req;
    }
    CHECK(pkv_sched_step(s, &o) == PKV_OK);
    CHECK(o.num_batch >= 0 && o.num_batch <= max_seqs);
    CHECK(o.num_slots >= o.num_batch && o.num_slots <= budget);
    CHECK(o.num_cow >= 0 && o.num_cow <= max_seqs);
    int64_t st[8], bst[8];
    CHECK(pkv_sched_stats(s, st) == PKV_OK);
    CHECK(pkv_bm_stats(bm, bst) == PKV_OK);
    CHECK(bst[0] + bst[1] == nb);
    CHECK(st[1] == bst[5]);   // running requests = live sequences in the manager
  }
  CHECK(pkv_sched_step(s, nullptr) < 0);
  pkv_sched_destroy(s);
  pkv_bm_destroy(bm);
}

void pool_plan_scenario() {
  const int64_t big = INT64_MAX;
  const int64_t choices[] = {0, 1, 7, 1LL << 30, 80000000000LL, 288000000000LL, big / 2, big - 1,
                             big};
  int64_t out[8];
  for (int i = 0; i < 64; ++i) {
    const int64_t dev = choices[pick(0, 8)] - pick(0, 1);
    const int64_t w = choices[pick(0, 8)];
    const int64_t r = choices[pick(0, 8)];
    const int32_t ppm = (int32_t)pick(-1, 1000001);
    pkv_kv_pool_plan(dev, w, r, ppm, (int)pick(-1, 2), (int)pick(0, 4097), (int)pick(0, 4097),
                     (int)pick(0, 4097), (int)pick(0, 5), 1 << pick(0, 13),
                     (int)pick(0, 1 << 30), (int)pick(0, 1 << 30), out);
  }
  CHECK(pkv_kv_pool_plan(1, 0, 0, 1, 0, 1, 1, 1, 2, 16, 1, 1, nullptr) < 0);
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int scenarios = argc > 2 ? std::atoi(argv[2]) : 200;
  rng.seed(seed);
  for (int i = 0; i < scenarios; ++i) {
    manager_scenario();
    scheduler_scenario();
    pool_plan_scenario();
  }
  std::printf("ok %d scenarios\n", scenarios);
  return 0;
}
