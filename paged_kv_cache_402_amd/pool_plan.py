"""KV-pool sizing through the C ABI (pkv_kv_pool_plan): how many blocks a memory budget
holds and how many requests of a given context length they serve at once.

The arithmetic lives in the library (csrc/pool_plan.cpp); this module only converts the
memory fraction to parts per million and names the eight results.
"""
import ctypes

from . import _lib

PLAN_KEYS = ("pool_bytes", "bytes_per_token", "bytes_per_block", "num_blocks",
             "blocks_per_request", "max_requests", "cache_tensor_bytes",
             "max_requests_contiguous")
UTIL_OF = {"remainder": 0, "device": 1}


def utilization_to_ppm(utilization: float) -> int:
    """The memory fraction in parts per million, rounded to nearest (0.9 -> 900000)."""
    return int(round(float(utilization) * 1_000_000))


def kv_pool_plan(device_bytes, weight_bytes, *, utilization=0.9, utilization_of="remainder",
                 reserve_bytes=0, num_layers, num_kv_heads, head_dim, elem_bytes, block_size,
                 context_tokens, max_model_len=None):
    """Returns a dict of PLAN_KEYS. Raises PagedKVError (code PKV_ENOBLOCKS) when the pool
    holds no block, PKV_EINVAL for arguments out of range."""
    out = (ctypes.c_int64 * 8)()
    code = _lib.lib.pkv_kv_pool_plan(
        int(device_bytes), int(weight_bytes), int(reserve_bytes), utilization_to_ppm(utilization),
        UTIL_OF[utilization_of], int(num_layers), int(num_kv_heads), int(head_dim),
        int(elem_bytes), int(block_size), int(context_tokens),
        int(context_tokens if max_model_len is None else max_model_len), out)
    _lib.check(code, "kv_pool_plan")
    return dict(zip(PLAN_KEYS, list(out)))
