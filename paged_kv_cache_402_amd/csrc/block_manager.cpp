// Host block manager: a fixed pool of equal-size KV blocks, one block table per sequence,
// a refcount per block, on-demand growth, fork / prefix sharing and copy-on-write.
//
// Pages cited:
//   P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
//   P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
//   P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)
//
// What the pages fix: any free block can serve any request (P1 §4.1); a table maps logical
// to physical blocks (P1 §4.2; P3 §2.2.3); a block is added only when the last one is full
// and nothing moves on growth (P1 §4.3; P3 §2.2.3); finished or preempted sequences return
// their blocks (P3 §2.2.2); tables may share physical blocks (P1 §6.1; P3 §2.2.3); a write
// into a shared block copies only that block (P1 §6.2; P2 §2.2).
// Readings taken where they are silent: the pool is fixed (the pseudo-code on P2 §3.1 grows
// it; here an unmet request fails with PKV_ENOBLOCKS and changes nothing); "shared" means
// refcount > 1 and the last holder writes in place; free blocks form a LIFO stack seeded by
// a caller-given order, so results are reproducible id for id.
#include <cstdint>
#include <cstring>
#include <list>
#include <string>
#include <unordered_map>
#include <vector>

#include "bm_internal.h"
#include "errors.h"
#include "pagedkv.h"

struct pkv_bm {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> rc;          // refcount per block; 0 = free or cached
  std::unordered_map<int64_t, Seq> seqs;
  int64_t shared = 0;               // blocks with rc > 1
  int64_t cow_copies = 0;
  int64_t alloc_failures = 0;

  // Prefix cache (P1 §7.4; P3 §2.2.8): a full prompt block is registered under its key: the
  // block before it (its id and hand-out generation, or -1) followed by its block_size token
  // ids. By induction the key names the whole token prefix up to that block exactly; the
  // generation, bumped each time a block is handed out, keeps keys that name an evicted
  // block's old contents from ever matching again. Registered blocks whose refcount falls to
  // zero stay cached, in release order; they are handed out again only when the free stack is
  // empty, oldest release first, and then leave the cache.
  std::unordered_map<std::string, int32_t> cache;
  std::vector<uint32_t> gen;                        // hand-outs of each block so far
  std::vector<std::string> block_key;               // "" when the block is not registered
  std::list<int32_t> lru;                           // cached blocks with rc == 0, oldest first
  std::vector<std::list<int32_t>::iterator> lru_it;
  std::vector<char> in_lru;
  int64_t prefix_hits = 0;                          // cached blocks reused by add_seq_cached
  int64_t prefix_lookups = 0;                       // full prompt blocks looked up

  size_t available() const { return free_stack.size() + lru.size(); }

  void lru_push_back(int32_t b) {
    lru_it[b] = lru.insert(lru.end(), b);
    in_lru[b] = 1;
  }
  void lru_push_front(int32_t b) {
    lru_it[b] = lru.insert(lru.begin(), b);
    in_lru[b] = 1;
  }
  void lru_erase(int32_t b) {
    lru.erase(lru_it[b]);
    in_lru[b] = 0;
  }
  void inc(int32_t b) {
    if (rc[b] == 0 && in_lru[b]) lru_erase(b);  // a cached block comes back into use
    if (++rc[b] == 2) ++shared;
  }
  void dec(int32_t b) {
    if (rc[b]-- == 2) --shared;
    if (rc[b] == 0) {
      if (!block_key[b].empty())
        lru_push_back(b);
      else
        free_stack.push_back(b);
    }
  }
  // Hands out a block: the top of the free stack, else the cached block released longest ago
  // (it leaves the cache; its key goes to *evicted so an undo can restore it).
  int32_t take(std::string* evicted = nullptr) {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
      if (evicted) evicted->clear();
    } else {
      b = lru.front();
      lru_erase(b);
      std::string key;
      key.swap(block_key[b]);
      cache.erase(key);
      if (evicted) *evicted = std::move(key);
    }
    rc[b] = 1;
    ++gen[b];
    return b;
  }
  // Undoes the last take(): the block goes back where it came from.
  void untake(int32_t b, const std::string& evicted) {
    rc[b] = 0;
    --gen[b];
    if (evicted.empty()) {
      free_stack.push_back(b);
    } else {
      block_key[b] = evicted;
      cache[evicted] = b;
      lru_push_front(b);
    }
  }
};

namespace {

std::string block_key_of(const pkv_bm* bm, int32_t parent, const int32_t* tokens) {
  const int bs = bm->block_size;
  const uint32_t g = parent >= 0 ? bm->gen[parent] : 0u;
  std::string k((size_t)(bs + 2) * sizeof(int32_t), '\0');
  std::memcpy(&k[0], &parent, sizeof(int32_t));
  std::memcpy(&k[sizeof(int32_t)], &g, sizeof(uint32_t));
  std::memcpy(&k[2 * sizeof(int32_t)], tokens, (size_t)bs * sizeof(int32_t));
  return k;
}

}  // namespace

namespace pkv {
int bm_block_size(const pkv_bm* bm) { return bm->block_size; }
}  // namespace pkv

namespace {

// What one append changed, so a failed batch can be rolled back exactly.
struct AppendUndo {
  pkv_bm::Seq* seq;
  int kind;         // 0: wrote in place, 1: fresh block appended, 2: copy-on-write
  int32_t src, dst;
  std::string evicted;  // cache key of dst if taking it evicted a cached block
};

int append_one(pkv_bm* bm, int64_t id, int32_t* slot, AppendUndo* undo) {
  auto it = bm->seqs.find(id);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "append_slot: unknown sequence %lld", (long long)id);
  pkv_bm::Seq& s = it->second;
  const int bs = bm->block_size;
  if (s.tokens >= (int64_t)INT32_MAX) return pkv::fail(PKV_EINVAL, "append_slot: sequence too long");
  const int off = (int)(s.tokens % bs);
  int32_t blk;
  undo->seq = &s;
  undo->src = undo->dst = -1;
  if (off == 0) {
    if (bm->available() == 0) {
      ++bm->alloc_failures;
      return pkv::fail(PKV_ENOBLOCKS, "append_slot: pool exhausted");
    }
    blk = bm->take(&undo->evicted);
    s.blocks.push_back(blk);
    undo->kind = 1;
    undo->dst = blk;
  } else {
    int32_t last = s.blocks.back();
    if (bm->rc[last] > 1) {
      if (bm->available() == 0) {
        ++bm->alloc_failures;
        return pkv::fail(PKV_ENOBLOCKS, "append_slot: pool exhausted (copy-on-write)");
      }
      blk = bm->take(&undo->evicted);
      bm->dec(last);  // stays > 0: it was shared
      s.blocks.back() = blk;
      ++bm->cow_copies;
      undo->kind = 2;
      undo->src = last;
      undo->dst = blk;
    } else {
      blk = last;
      undo->kind = 0;
    }
  }
  ++s.tokens;
  *slot = blk * bs + off;
  return undo->kind == 2 ? 1 : 0;
}

void undo_one(pkv_bm* bm, const AppendUndo& u) {
  pkv_bm::Seq& s = *u.seq;
  --s.tokens;
  if (u.kind == 1) {
    s.blocks.pop_back();
    bm->untake(u.dst, u.evicted);
  } else if (u.kind == 2) {
    s.blocks.back() = u.src;
    bm->inc(u.src);
    bm->untake(u.dst, u.evicted);
    --bm->cow_copies;
  }
}

}  // namespace

extern "C" {

pkv_bm* pkv_bm_create(int num_blocks, int block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0 || (int64_t)num_blocks * block_size >= INT32_MAX) {
    pkv::fail(PKV_EINVAL, "bm_create: bad pool size");
    return nullptr;
  }
  pkv_bm* bm = new pkv_bm();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->rc.assign(num_blocks, 0);
  bm->block_key.assign(num_blocks, std::string());
  bm->gen.assign(num_blocks, 0u);
  bm->lru_it.resize(num_blocks);
  bm->in_lru.assign(num_blocks, 0);
  bm->free_stack.resize(num_blocks);
  std::vector<char> seen(num_blocks, 0);
  for (int i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      pkv::fail(PKV_EINVAL, "bm_create: free_order is not a permutation of the pool");
      return nullptr;
    }
    seen[b] = 1;
    bm->free_stack[num_blocks - 1 - i] = b;  // order[0] on top
  }
  pkv::ok();
  return bm;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

int pkv_bm_add_seq(pkv_bm* bm, int64_t seq, int num_tokens) {
  if (!bm || num_tokens < 0) return pkv::fail(PKV_EINVAL, "add_seq: bad argument");
  if (bm->seqs.count(seq)) return pkv::fail(PKV_EINVAL, "add_seq: sequence %lld exists", (long long)seq);
  size_t need = ((size_t)num_tokens + bm->block_size - 1) / bm->block_size;
  if (need > bm->available()) {
    ++bm->alloc_failures;
    return pkv::fail(PKV_ENOBLOCKS, "add_seq: %zu blocks needed, %zu free", need, bm->available());
  }
  pkv_bm::Seq s;
  s.blocks.reserve(need + 1);
  for (size_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  s.tokens = num_tokens;
  bm->seqs.emplace(seq, std::move(s));
  return pkv::ok();
}

int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return pkv::fail(PKV_EINVAL, "fork: null manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "fork: unknown parent %lld", (long long)parent);
  if (bm->seqs.count(child)) return pkv::fail(PKV_EINVAL, "fork: child %lld exists", (long long)child);
  pkv_bm::Seq s = it->second;
  for (int32_t b : s.blocks) bm->inc(b);
  bm->seqs.emplace(child, std::move(s));
  return pkv::ok();
}

int pkv_bm_share_prefix(pkv_bm* bm, int64_t src, int64_t dst, int num_prefix_blocks) {
  if (!bm || num_prefix_blocks < 0) return pkv::fail(PKV_EINVAL, "share_prefix: bad argument");
  auto it = bm->seqs.find(src);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "share_prefix: unknown source %lld", (long long)src);
  if (bm->seqs.count(dst)) return pkv::fail(PKV_EINVAL, "share_prefix: %lld exists", (long long)dst);
  if ((int64_t)num_prefix_blocks * bm->block_size > it->second.tokens)
    return pkv::fail(PKV_EINVAL, "share_prefix: only full blocks can be shared");
  pkv_bm::Seq s;
  s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + num_prefix_blocks);
  s.tokens = (int64_t)num_prefix_blocks * bm->block_size;
  for (int32_t b : s.blocks) bm->inc(b);
  bm->seqs.emplace(dst, std::move(s));
  return pkv::ok();
}

int pkv_bm_append_slot(pkv_bm* bm, int64_t seq, int32_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || !slot) return pkv::fail(PKV_EINVAL, "append_slot: bad argument");
  AppendUndo u;
  int st = append_one(bm, seq, slot, &u);
  if (st < 0) return st;
  if (cow_src) *cow_src = u.kind == 2 ? u.src : -1;
  if (cow_dst) *cow_dst = u.kind == 2 ? u.dst : -1;
  pkv::ok();
  return st;
}

int pkv_bm_append_step(pkv_bm* bm, const int64_t* seqs, int n, int32_t* slots,
                       int32_t* cow_pairs, int* num_cow, int32_t* cow_src) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_cow)
    return pkv::fail(PKV_EINVAL, "append_step: bad argument");
  std::vector<AppendUndo> log(n);
  int ncow = 0;
  for (int i = 0; i < n; ++i) {
    int st = append_one(bm, seqs[i], &slots[i], &log[i]);
    if (st < 0) {
      for (int j = i - 1; j >= 0; --j) undo_one(bm, log[j]);
      return st;
    }
    if (st == 1) {
      cow_pairs[2 * ncow] = log[i].src;
      cow_pairs[2 * ncow + 1] = log[i].dst;
      ++ncow;
    }
  }
  // written only once the whole batch has succeeded, so a failure leaves it untouched
  if (cow_src)
    for (int i = 0; i < n; ++i) cow_src[i] = log[i].kind == 2 ? log[i].src : -1;
  *num_cow = ncow;
  return pkv::ok();
}

int pkv_bm_append_slots(pkv_bm* bm, const int64_t* seqs, int n, int32_t* slots,
                        int32_t* cow_pairs, int* num_cow) {
  return pkv_bm_append_step(bm, seqs, n, slots, cow_pairs, num_cow, nullptr);
}

int pkv_bm_extend(pkv_bm* bm, int64_t seq, int num_tokens, int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || num_tokens < 0) return pkv::fail(PKV_EINVAL, "extend: bad argument");
  if (!bm->seqs.count(seq)) return pkv::fail(PKV_ENOSEQ, "extend: unknown sequence %lld", (long long)seq);
  std::vector<AppendUndo> log((size_t)num_tokens);
  int first = 0;
  int32_t slot;
  for (int i = 0; i < num_tokens; ++i) {
    int st = append_one(bm, seq, &slot, &log[i]);
    if (st < 0) {
      for (int j = i - 1; j >= 0; --j) undo_one(bm, log[j]);
      return st;
    }
    if (i == 0) first = st;
  }
  if (cow_src) *cow_src = first == 1 ? log[0].src : -1;
  if (cow_dst) *cow_dst = first == 1 ? log[0].dst : -1;
  pkv::ok();
  return first;
}

int pkv_bm_free_seq(pkv_bm* bm, int64_t seq) {
  if (!bm) return pkv::fail(PKV_EINVAL, "free_seq: null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "free_seq: unknown sequence %lld", (long long)seq);
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t i = blocks.size(); i-- > 0;) bm->dec(blocks[i]);
  bm->seqs.erase(it);
  return pkv::ok();
}

int pkv_bm_table(const pkv_bm* bm, int64_t seq, int32_t* out, int cap, int* num_tokens) {
  if (!bm || cap < 0 || (cap > 0 && !out)) return pkv::fail(PKV_EINVAL, "table: bad argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "table: unknown sequence %lld", (long long)seq);
  const auto& s = it->second;
  int n = (int)s.blocks.size();
  const int m = n < cap ? n : cap;
  if (m > 0) std::memcpy(out, s.blocks.data(), sizeof(int32_t) * (size_t)m);
  if (num_tokens) *num_tokens = (int)s.tokens;
  pkv::ok();
  return n;
}

int pkv_bm_slots(const pkv_bm* bm, int64_t seq, int start, int count, int32_t* out) {
  if (!bm || start < 0 || count < 0 || (count > 0 && !out)) return pkv::fail(PKV_EINVAL, "slots: bad argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "slots: unknown sequence %lld", (long long)seq);
  const auto& s = it->second;
  if ((int64_t)start + count > s.tokens) return pkv::fail(PKV_EINVAL, "slots: positions past the sequence end");
  const int bs = bm->block_size;
  for (int i = 0; i < count; ++i) {
    int t = start + i;
    out[i] = s.blocks[t / bs] * bs + t % bs;
  }
  return pkv::ok();
}

int pkv_bm_build_tables(const pkv_bm* bm, const int64_t* seqs, int n, int32_t* tables, int width,
                        int32_t* seq_lens) {
  if (!bm || n < 0 || width <= 0 || (n > 0 && (!seqs || !tables || !seq_lens)))
    return pkv::fail(PKV_EINVAL, "build_tables: bad argument");
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return pkv::fail(PKV_ENOSEQ, "build_tables: unknown sequence %lld", (long long)seqs[i]);
    const auto& s = it->second;
    if ((int)s.blocks.size() > width) return pkv::fail(PKV_EINVAL, "build_tables: table wider than %d", width);
    int32_t* row = tables + (size_t)i * width;
    if (!s.blocks.empty()) std::memcpy(row, s.blocks.data(), sizeof(int32_t) * s.blocks.size());
    for (int j = (int)s.blocks.size(); j < width; ++j) row[j] = -1;
    seq_lens[i] = (int32_t)s.tokens;
  }
  return pkv::ok();
}

int pkv_bm_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return pkv::fail(PKV_EINVAL, "refcount: bad block");
  return bm->rc[block];
}

int pkv_bm_stats(const pkv_bm* bm, int64_t out[8]) {
  if (!bm || !out) return pkv::fail(PKV_EINVAL, "stats: bad argument");
  out[0] = bm->num_blocks - (int64_t)bm->available();
  out[1] = (int64_t)bm->available();
  out[2] = bm->shared;
  out[3] = bm->cow_copies;
  out[4] = bm->alloc_failures;
  out[5] = (int64_t)bm->seqs.size();
  out[6] = bm->prefix_hits;
  out[7] = bm->prefix_lookups;
  return pkv::ok();
}

int pkv_bm_add_seq_cached(pkv_bm* bm, int64_t seq, const int32_t* token_ids, int num_tokens,
                          int* num_cached_tokens) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !token_ids))
    return pkv::fail(PKV_EINVAL, "add_seq_cached: bad argument");
  if (bm->seqs.count(seq)) return pkv::fail(PKV_EINVAL, "add_seq_cached: sequence %lld exists", (long long)seq);
  const int bs = bm->block_size;
  const int nfull = num_tokens / bs;
  const size_t nblocks = ((size_t)num_tokens + bs - 1) / bs;
  // longest run of leading full blocks already cached
  std::vector<int32_t> hits;
  int32_t parent = -1;
  size_t hits_cached_free = 0;  // hits that sit in the cache unreferenced (not allocatable then)
  for (int j = 0; j < nfull; ++j) {
    auto it = bm->cache.find(block_key_of(bm, parent, token_ids + (size_t)j * bs));
    if (it == bm->cache.end()) break;
    hits.push_back(it->second);
    if (bm->rc[it->second] == 0) ++hits_cached_free;
    parent = it->second;
  }
  const size_t need = nblocks - hits.size();
  if (need > bm->available() - hits_cached_free) {
    ++bm->alloc_failures;
    return pkv::fail(PKV_ENOBLOCKS, "add_seq_cached: %zu blocks needed, %zu free", need,
                     bm->available() - hits_cached_free);
  }
  pkv_bm::Seq s;
  s.blocks.reserve(nblocks + 1);
  for (int32_t b : hits) {
    bm->inc(b);  // leaves the released-block list if it was there
    s.blocks.push_back(b);
  }
  for (size_t j = hits.size(); j < nblocks; ++j) {
    const int32_t b = bm->take();
    s.blocks.push_back(b);
    if ((int)j < nfull) {  // register the new full block under its prefix
      std::string key = block_key_of(bm, parent, token_ids + j * bs);
      bm->cache[key] = b;
      bm->block_key[b] = std::move(key);
      parent = b;
    }
  }
  s.tokens = num_tokens;
  bm->seqs.emplace(seq, std::move(s));
  bm->prefix_hits += (int64_t)hits.size();
  bm->prefix_lookups += nfull;
  if (num_cached_tokens) *num_cached_tokens = (int)hits.size() * bs;
  return pkv::ok();
}

int pkv_bm_prefix_stats(const pkv_bm* bm, int64_t out[4]) {
  if (!bm || !out) return pkv::fail(PKV_EINVAL, "prefix_stats: bad argument");
  out[0] = (int64_t)bm->cache.size();
  out[1] = (int64_t)bm->lru.size();
  out[2] = bm->prefix_hits;
  out[3] = bm->prefix_lookups;
  return pkv::ok();
}

}  // extern "C"
