"""Python handle on the C++ continuous-batching scheduler of libpagedkv.so (marshalling only).

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理"

Each step frees finished requests, admits waiting ones first come, first served, and gives
every running request one token slot, preempting the newest when the pool is empty (P1 §8.2;
P3 §2.2.2, §2.2.5, §2.2.12). The policy itself is in csrc/scheduler.cpp.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from ._lib import lib, check

SCHED_STAT_KEYS = ("waiting", "running", "finished", "admitted", "preempted", "steps",
                   "decode_tokens", "prefill_tokens")


class _StepOut(ctypes.Structure):
    _fields_ = [("batch", ctypes.POINTER(ctypes.c_int64)),
                ("slots", ctypes.POINTER(ctypes.c_int32)),
                ("slot_seq", ctypes.POINTER(ctypes.c_int64)),
                ("slot_pos", ctypes.POINTER(ctypes.c_int32)),
                ("cow_pairs", ctypes.POINTER(ctypes.c_int32)),
                ("finished", ctypes.POINTER(ctypes.c_int64)),
                ("admitted", ctypes.POINTER(ctypes.c_int64)),
                ("preempted", ctypes.POINTER(ctypes.c_int64)),
                ("num_batch", ctypes.c_int), ("num_slots", ctypes.c_int),
                ("num_cow", ctypes.c_int), ("num_finished", ctypes.c_int),
                ("num_admitted", ctypes.c_int), ("num_preempted", ctypes.c_int)]


@dataclass
class Step:
    batch: np.ndarray        # int64 request ids to decode, admission order
    slots: np.ndarray        # int32 slots to write: admitted prompts, then one per batch entry
    slot_seq: np.ndarray     # int64 request of each slot
    slot_pos: np.ndarray     # int32 token position of each slot
    cow_pairs: np.ndarray    # int32 [n][2]
    finished: list
    admitted: list
    preempted: list


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Scheduler:
    def __init__(self, block_manager, max_num_seqs: int, max_step_tokens: int,
                 watermark_blocks: int = 0):
        self.bm = block_manager                       # keeps the manager alive
        h = lib.pkv_sched_create(block_manager._h, block_manager.block_size, max_num_seqs,
                                 max_step_tokens, watermark_blocks)
        if not h:
            check(-1, "pkv_sched_create")
        self._h = ctypes.c_void_p(h)
        self.max_num_seqs = max_num_seqs
        self.max_step_tokens = max_step_tokens
        n, t = max_num_seqs, max_step_tokens
        self._a = {"batch": np.zeros(n, np.int64), "slots": np.zeros(t, np.int32),
                   "slot_seq": np.zeros(t, np.int64), "slot_pos": np.zeros(t, np.int32),
                   "cow_pairs": np.zeros(2 * n, np.int32), "finished": np.zeros(n, np.int64),
                   "admitted": np.zeros(n, np.int64), "preempted": np.zeros(n, np.int64)}
        a = self._a
        self._out = _StepOut(_ptr(a["batch"], ctypes.c_int64), _ptr(a["slots"], ctypes.c_int32),
                             _ptr(a["slot_seq"], ctypes.c_int64),
                             _ptr(a["slot_pos"], ctypes.c_int32),
                             _ptr(a["cow_pairs"], ctypes.c_int32),
                             _ptr(a["finished"], ctypes.c_int64),
                             _ptr(a["admitted"], ctypes.c_int64),
                             _ptr(a["preempted"], ctypes.c_int64), 0, 0, 0, 0, 0, 0)

    def close(self):
        if getattr(self, "_h", None):
            lib.pkv_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_request(self, req_id: int, prompt_tokens: int, output_tokens: int):
        check(lib.pkv_sched_add_request(self._h, req_id, prompt_tokens, output_tokens),
              "sched_add_request")

    def step(self) -> Step:
        o = self._out
        check(lib.pkv_sched_step(self._h, ctypes.byref(o)), "sched_step")
        a = self._a
        return Step(a["batch"][:o.num_batch].copy(), a["slots"][:o.num_slots].copy(),
                    a["slot_seq"][:o.num_slots].copy(), a["slot_pos"][:o.num_slots].copy(),
                    a["cow_pairs"][:2 * o.num_cow].reshape(-1, 2).copy(),
                    a["finished"][:o.num_finished].tolist(),
                    a["admitted"][:o.num_admitted].tolist(),
                    a["preempted"][:o.num_preempted].tolist())

    def stats(self) -> dict:
        out = np.zeros(8, dtype=np.int64)
        check(lib.pkv_sched_stats(self._h, _ptr(out, ctypes.c_int64)), "sched_stats")
        return {k: int(out[i]) for i, k in enumerate(SCHED_STAT_KEYS)}
