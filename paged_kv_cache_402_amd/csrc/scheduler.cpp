// Continuous-batching scheduler over the host block manager.
//
// P1 §8.2 and P3 §2.2.12: a request's blocks go back to the pool as soon as it finishes, and
// the freed space is given to waiting requests at once, instead of holding a static batch
// until its longest request ends; P3 §2.2.2 and §2.2.5: when the fixed pool runs out, a
// running request is preempted (its blocks released) and recomputed later.
//
// One call advances one decode step:
//   1. requests that have produced all their tokens are freed;
//   2. waiting requests are admitted first-come first-served while the batch has room, the
//      step's token budget allows their prompt, and the pool keeps `watermark` blocks free
//      after taking the prompt plus one token; admission stops at the first one that does
//      not fit;
//   3. every running request, in admission order, takes one token slot. When the pool is
//      empty, the most recently admitted running request is preempted: its blocks are freed,
//      the tokens it produced join its prompt (to be recomputed), and it goes back to the
//      front of the waiting queue; then the slot is asked for again.
// The step reports the batch to decode, the slots to write (the admitted prompts' tokens,
// then one token per running request) and the requests finished, admitted and preempted.

#include <cstdint>
#include <deque>
#include <unordered_set>
#include <vector>

#include "bm_internal.h"
#include "errors.h"
#include "pagedkv.h"

struct pkv_sched {
  struct Req {
    int64_t id;
    int prompt;     // tokens written at admission
    int output;     // tokens still to produce after admission
    int produced;   // tokens produced since admission
  };
  pkv_bm* bm;
  int block_size;
  int max_num_seqs, max_step_tokens, watermark;
  std::deque<Req> waiting;
  std::vector<Req> running;
  std::unordered_set<int64_t> known;
  int64_t steps = 0, finished_total = 0, admitted_total = 0, preempted_total = 0;
  int64_t decode_tokens = 0, prefill_tokens = 0;
};

namespace {

int64_t available(pkv_bm* bm) {
  int64_t st[8];
  pkv_bm_stats(bm, st);
  return st[1];
}

}  // namespace

extern "C" {

pkv_sched* pkv_sched_create(pkv_bm* bm, int block_size, int max_num_seqs, int max_step_tokens,
                            int watermark_blocks) {
  if (!bm || block_size <= 0 || max_num_seqs <= 0 || max_step_tokens < max_num_seqs ||
      watermark_blocks < 0) {
    pkv::fail(PKV_EINVAL, "sched_create: bad argument (max_step_tokens must be >= max_num_seqs)");
    return nullptr;
  }
  if (block_size != pkv::bm_block_size(bm)) {
    pkv::fail(PKV_EINVAL, "sched_create: block_size %d is not the manager's %d", block_size,
              pkv::bm_block_size(bm));
    return nullptr;
  }
  auto* s = new pkv_sched();
  s->bm = bm;
  s->block_size = block_size;
  s->max_num_seqs = max_num_seqs;
  s->max_step_tokens = max_step_tokens;
  s->watermark = watermark_blocks;
  pkv::ok();
  return s;
}

void pkv_sched_destroy(pkv_sched* s) { delete s; }

int pkv_sched_add_request(pkv_sched* s, int64_t req_id, int prompt_tokens, int output_tokens) {
  if (!s || prompt_tokens < 1 || output_tokens < 1)
    return pkv::fail(PKV_EINVAL, "sched_add_request: bad argument");
  // a preempted request comes back with the tokens it produced added to its prompt, so the
  // whole request must fit the step budget and the pool
  if ((int64_t)prompt_tokens + output_tokens > s->max_step_tokens)
    return pkv::fail(PKV_EINVAL, "sched_add_request: %d + %d tokens exceed the step budget %d",
                     prompt_tokens, output_tokens, s->max_step_tokens);
  int64_t st[8];
  pkv_bm_stats(s->bm, st);
  const int64_t blocks = ((int64_t)prompt_tokens + output_tokens + s->block_size - 1) / s->block_size;
  if (blocks > st[0] + st[1] - s->watermark)
    return pkv::fail(PKV_EINVAL, "sched_add_request: %lld blocks exceed the pool less the "
                     "watermark", (long long)blocks);
  if (!s->known.insert(req_id).second)
    return pkv::fail(PKV_EINVAL, "sched_add_request: request %lld exists", (long long)req_id);
  s->waiting.push_back({req_id, prompt_tokens, output_tokens, 0});
  return pkv::ok();
}

int pkv_sched_step(pkv_sched* s, pkv_sched_step_out* o) {
  if (!s || !o || !o->batch || !o->slots || !o->slot_seq || !o->slot_pos || !o->cow_pairs ||
      !o->finished || !o->admitted || !o->preempted)
    return pkv::fail(PKV_EINVAL, "sched_step: null argument");
  o->num_batch = o->num_slots = o->num_cow = 0;
  o->num_finished = o->num_admitted = o->num_preempted = 0;
  // capacities: batch, finished, admitted, preempted and cow rows hold max_num_seqs entries;
  // slots hold max_step_tokens
  const int bs = s->block_size;

  // 1. finish
  std::vector<pkv_sched::Req> keep;
  keep.reserve(s->running.size());
  for (const auto& r : s->running) {
    if (r.produced >= r.output) {
      int st = pkv_bm_free_seq(s->bm, r.id);
      if (st < 0) return st;
      o->finished[o->num_finished++] = r.id;
      s->known.erase(r.id);
      ++s->finished_total;
    } else {
      keep.push_back(r);
    }
  }
  s->running.swap(keep);

  // 2. admit (first come, first served; the step's budget counts one token per running
  //    request plus the admitted prompts)
  int64_t budget = s->max_step_tokens - (int64_t)s->running.size();
  struct Pending { int64_t id; int prompt; };
  std::vector<Pending> prefill;
  while (!s->waiting.empty() && (int)s->running.size() < s->max_num_seqs) {
    const auto& r = s->waiting.front();
    const int64_t need = (r.prompt + 1 + bs - 1) / bs;
    if (r.prompt + 1 > budget || available(s->bm) - need < s->watermark) break;
    int st = pkv_bm_add_seq(s->bm, r.id, r.prompt);
    if (st < 0) return st;
    prefill.push_back({r.id, r.prompt});
    budget -= r.prompt + 1;
    o->admitted[o->num_admitted++] = r.id;
    ++s->admitted_total;
    s->running.push_back(r);
    s->waiting.pop_front();
  }

  // 3. one token per running request; preempt the newest on an empty pool
  std::vector<int32_t> dec_slot;
  std::vector<int64_t> dec_seq;
  std::vector<int32_t> dec_pos;
  size_t i = 0;
  while (i < s->running.size()) {
    auto& r = s->running[i];
    int32_t slot = -1, cs = -1, cd = -1;
    int st = pkv_bm_append_slot(s->bm, r.id, &slot, &cs, &cd);
    if (st == PKV_ENOBLOCKS) {
      pkv_sched::Req v = s->running.back();
      s->running.pop_back();
      int fs = pkv_bm_free_seq(s->bm, v.id);
      if (fs < 0) return fs;
      for (size_t k = 0; k < prefill.size(); ++k)
        if (prefill[k].id == v.id) {
          prefill.erase(prefill.begin() + (long)k);
          break;
        }
      v.prompt += v.produced;
      v.output -= v.produced;
      v.produced = 0;
      s->waiting.push_front(v);
      o->preempted[o->num_preempted++] = v.id;
      ++s->preempted_total;
      continue;                                   // the slot is asked for again
    }
    if (st < 0) return st;
    if (st == 1) {
      o->cow_pairs[2 * o->num_cow] = cs;
      o->cow_pairs[2 * o->num_cow + 1] = cd;
      ++o->num_cow;
    }
    dec_slot.push_back(slot);
    dec_seq.push_back(r.id);
    dec_pos.push_back(r.prompt + r.produced);
    ++i;
  }

  // outputs: prompt tokens of the admitted requests that are still running, then the decode
  // tokens; the batch in admission order
  for (const auto& p : prefill) {
    int st = pkv_bm_slots(s->bm, p.id, 0, p.prompt, o->slots + o->num_slots);
    if (st < 0) return st;
    for (int t = 0; t < p.prompt; ++t) {
      o->slot_seq[o->num_slots + t] = p.id;
      o->slot_pos[o->num_slots + t] = t;
    }
    o->num_slots += p.prompt;
    s->prefill_tokens += p.prompt;
  }
  for (size_t k = 0; k < dec_slot.size(); ++k) {
    o->slots[o->num_slots] = dec_slot[k];
    o->slot_seq[o->num_slots] = dec_seq[k];
    o->slot_pos[o->num_slots] = dec_pos[k];
    ++o->num_slots;
  }
  for (auto& r : s->running) {
    o->batch[o->num_batch++] = r.id;
    ++r.produced;
  }
  s->decode_tokens += o->num_batch;
  ++s->steps;
  return pkv::ok();
}

int pkv_sched_stats(const pkv_sched* s, int64_t out[8]) {
  if (!s || !out) return pkv::fail(PKV_EINVAL, "sched_stats: bad argument");
  out[0] = (int64_t)s->waiting.size();
  out[1] = (int64_t)s->running.size();
  out[2] = s->finished_total;
  out[3] = s->admitted_total;
  out[4] = s->preempted_total;
  out[5] = s->steps;
  out[6] = s->decode_tokens;
  out[7] = s->prefill_tokens;
  return pkv::ok();
}

}  // extern "C"
