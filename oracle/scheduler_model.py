"""Reference model of the continuous-batching scheduler (oracle; test infrastructure only).

Follows the pages' description of serving on a paged pool:
  - a finished request returns its blocks to the pool at once and the space goes to waiting
    requests in the same step, rather than a whole batch waiting for its longest request
    (openeuler.csdn.net explainer §8.2; aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页
    管理" §2.2.12);
  - the pool is fixed; when it runs out a request is preempted and its blocks released
    (aiknowledge.cn §2.2.2 and §2.2.5).

Readings where the pages are silent (listed in the design doc):
  - admission is first come, first served and stops at the first request that does not fit
    (batch size, the step's token budget, or the pool keeping `watermark` blocks free after
    taking prompt + 1 tokens);
  - preemption takes the most recently admitted running request; the tokens it produced are
    added to its prompt (recomputed when it is admitted again) and it returns to the front of
    the queue;
  - a step gives every running request, in admission order, one token slot; an admitted
    request writes its prompt and takes its first token in the step that admits it.
"""
from collections import deque

from .block_manager_model import ENOBLOCKS


class SchedulerModel:
    def __init__(self, manager, max_num_seqs, max_step_tokens, watermark_blocks=0):
        self.bm = manager
        self.bs = manager.block_size
        self.max_num_seqs = max_num_seqs
        self.max_step_tokens = max_step_tokens
        self.watermark = watermark_blocks
        self.waiting = deque()            # [id, prompt, output, produced]
        self.running = []
        self.totals = dict(finished=0, admitted=0, preempted=0, steps=0, decode_tokens=0,
                           prefill_tokens=0)

    def add_request(self, req_id, prompt, output):
        self.waiting.append([req_id, prompt, output, 0])

    def _available(self):
        return self.bm.stats()["free"]

    def _victim(self):
        """Index in the running list of the request to preempt: the most recently admitted."""
        return len(self.running) - 1

    def step(self):
        out = dict(batch=[], slots=[], slot_seq=[], slot_pos=[], cow_pairs=[], finished=[],
                   admitted=[], preempted=[])
        # 1. requests that produced everything leave and free their blocks
        still = []
        for r in self.running:
            if r[3] >= r[2]:
                self.bm.free_seq(r[0])
                out["finished"].append(r[0])
                self.totals["finished"] += 1
            else:
                still.append(r)
        self.running = still
        # 2. first come, first served
        budget = self.max_step_tokens - len(self.running)
        prefill = []
        while self.waiting and len(self.running) < self.max_num_seqs:
            r = self.waiting[0]
            need = -(-(r[1] + 1) // self.bs)
            if r[1] + 1 > budget or self._available() - need < self.watermark:
                break
            self.bm.add_seq(r[0], r[1])
            prefill.append((r[0], r[1]))
            budget -= r[1] + 1
            out["admitted"].append(r[0])
            self.totals["admitted"] += 1
            self.running.append(self.waiting.popleft())
        # 3. one token each, newest preempted when the pool is empty
        dec = []
        i = 0
        while i < len(self.running):
            r = self.running[i]
            st, slot, cs, cd = self.bm.append_slot(r[0])
            if st == ENOBLOCKS:
                v = self.running.pop(self._victim())
                self.bm.free_seq(v[0])
                prefill = [p for p in prefill if p[0] != v[0]]
                v[1] += v[3]
                v[2] -= v[3]
                v[3] = 0
                self.waiting.appendleft(v)
                out["preempted"].append(v[0])
                self.totals["preempted"] += 1
                continue
            if st == 1:
                out["cow_pairs"].append((cs, cd))
            dec.append((slot, r[0], r[1] + r[3]))
            i += 1
        for rid, n in prefill:
            out["slots"] += self.bm.slots(rid, 0, n)
            out["slot_seq"] += [rid] * n
            out["slot_pos"] += list(range(n))
            self.totals["prefill_tokens"] += n
        for slot, rid, pos in dec:
            out["slots"].append(slot)
            out["slot_seq"].append(rid)
            out["slot_pos"].append(pos)
        for r in self.running:
            out["batch"].append(r[0])
            r[3] += 1
        self.totals["decode_tokens"] += len(out["batch"])
        self.totals["steps"] += 1
        return out

    def stats(self):
        return dict(waiting=len(self.waiting), running=len(self.running), **self.totals)
