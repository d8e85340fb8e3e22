"""MI355X-native decode attention over a paged KV cache.

    from paged_kv_cache_402_amd import (paged_attention_decode, reshape_and_cache, copy_blocks,
                                        BlockManager)

The device operations run in hand-written HIP kernels for gfx950 inside libpagedkv.so (C ABI in
include/pagedkv.h); the block manager is C++ in the same library. Importing fails loudly if the
library has not been built (python paged_kv_cache_402_amd/build.py).
"""
from ._lib import PagedKVError, check, lib, last_error  # noqa: F401  (raises if missing)
from .block_manager import BlockManager  # noqa: F401
from .scheduler import Scheduler  # noqa: F401
from .pool_plan import kv_pool_plan  # noqa: F401
from .ops import (KV_CACHED, KV_STREAM, copy_blocks, decode_kv_policy,  # noqa: F401
                  decode_ticketed_items, decode_work_list, decode_work_list_packed,
                  decode_work_list_private_tail,
                  decode_workspace_bytes, decode_workspace_init,
                  default_partition,
                  paged_attention_decode, paged_attention_decode_append,
                  paged_attention_decode_step, paged_attention_partitions_step,
                  paged_attention_decode_step_groups, paged_attention_partitions_step_groups,
                  plan_fork_groups,
                  paged_attention_partitions, paged_attention_partitions_append,
                  paged_attention_prefix,
                  paged_attention_reduce, plan_shared_prefix, read_probe,
                  reshape_and_cache)

__version__ = "0.1.0"
