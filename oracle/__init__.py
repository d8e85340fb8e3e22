"""fp64 CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The product path (paged_kv_cache_402_amd) never imports it and shares no code with it.

Pages cited (all three are web pages about vLLM's PagedAttention):
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
  P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)

Modules:
  storage             exact decoding of stored bit patterns to float64
  paged_attention     gather through the block table + textbook softmax attention (fp64)
  cache_ops           reference cache write (slot mapping) and whole-block copy
  block_manager_model reference model of the block manager (free list, refcounts, COW, fork)
  pool_plan           KV-pool sizing from the memory fraction, weights and per-token KV bytes
  scheduler_model     continuous batching: admission, one token per step, preemption

Every function is pinned by tests under tests/ (test_oracle*.py) against values the pages
print, closed forms, brute force at 50 digits, and an independent library routine.
"""
from . import (storage, paged_attention, cache_ops, block_manager_model, pool_plan,  # noqa: F401
               scheduler_model)
