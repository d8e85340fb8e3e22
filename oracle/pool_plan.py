"""Reference KV-pool sizing (oracle; test infrastructure only).

Follows aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理":
  - §2.2.5: the memory fraction fixes, at start-up, how much memory goes to the KV pool;
  - §2.2.7: the pool is what is left once the weights are loaded, taken at that fraction; one
    request's KV is layers x 2 (K and V) x KV width x element bytes x context tokens; the
    number of requests served at once is the pool divided by one request's KV.
Blocks (openeuler.csdn.net explainer §4.1, §4.3): the pool is cut into equal blocks of
block_size tokens and a request of C tokens holds ceil(C / block_size) of them.

Reading where the page is ambiguous (listed in the design doc): its worked figure applies the
fraction to what the weights leave (0.9 of 80 - 40 GB, about 36 GB); the other common reading
caps the whole process at the fraction of the device (0.9 * 80 - 40 = 32 GB). Both are
computed here ("remainder" and "device"). Fractions are exact rationals (Fraction of a
decimal string or of parts per million); every result is an exact integer.
"""
from fractions import Fraction


def pool_bytes(device_bytes, weight_bytes, utilization, utilization_of="remainder",
               reserve_bytes=0):
    """Bytes of the KV pool. `utilization` is a Fraction (or a decimal string)."""
    u = Fraction(utilization)
    if utilization_of == "remainder":
        left = device_bytes - weight_bytes - reserve_bytes
        return (u * left).__floor__() if left > 0 else left
    if utilization_of == "device":
        return (u * device_bytes).__floor__() - weight_bytes - reserve_bytes
    raise ValueError(utilization_of)


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes):
    """P3 §2.2.7: layers x 2 (K, V) x KV width (heads x head_dim) x element bytes."""
    return num_layers * 2 * (num_kv_heads * head_dim) * elem_bytes


def plan(device_bytes, weight_bytes, utilization, utilization_of, reserve_bytes, num_layers,
         num_kv_heads, head_dim, elem_bytes, block_size, context_tokens, max_model_len):
    """The same eight figures as the library's pool plan, by the definitions above; None for
    num_blocks and what follows from it when the pool holds no block."""
    pool = pool_bytes(device_bytes, weight_bytes, utilization, utilization_of, reserve_bytes)
    per_token = kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)
    per_block = per_token * block_size
    blocks_per_request = -(-context_tokens // block_size)
    res = dict(pool_bytes=pool, bytes_per_token=per_token, bytes_per_block=per_block,
               blocks_per_request=blocks_per_request, num_blocks=None, max_requests=None,
               cache_tensor_bytes=None, max_requests_contiguous=None)
    if pool < per_block:
        return res
    nb = pool // per_block
    res.update(num_blocks=nb, max_requests=nb // blocks_per_request,
               cache_tensor_bytes=nb * num_kv_heads * block_size * head_dim * elem_bytes,
               max_requests_contiguous=pool // (per_token * max_model_len))
    return res
