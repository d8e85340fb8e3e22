// KV-pool sizing: how many blocks a fixed memory budget holds, and how many requests of a
// given context length they serve at once.
//
// Follows aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理": §2.2.5 (the memory
// fraction decides the size of the KV pool, which is fixed at start-up) and §2.2.7 (the
// worked estimate: the pool left after the weights, divided by what one request's KV takes,
// where one token's KV is layers x 2 (K and V) x the KV width x the element size). Blocks of
// block_size tokens replace the page's per-token division: a request of C tokens holds
// ceil(C / block_size) blocks (openeuler.csdn.net explainer, §4.3: a block is taken only when
// the last one is full).
//
// All arithmetic is on integers. The memory fraction comes in parts per million, so no
// floating-point rounding decides a byte or block count.

#include <cstdint>

#include "errors.h"
#include "pagedkv.h"

namespace {

constexpr int64_t kPpm = 1000000;

// floor(x * ppm / 1e6) for x >= 0, 0 <= ppm <= 1e6, exact (128-bit intermediate).
int64_t scale_ppm(int64_t x, int64_t ppm) {
  return static_cast<int64_t>((static_cast<__int128>(x) * ppm) / kPpm);
}

}  // namespace

extern "C" int pkv_kv_pool_plan(int64_t device_bytes, int64_t weight_bytes,
                                int64_t reserve_bytes, int32_t utilization_ppm,
                                int utilization_of, int num_layers, int num_kv_heads,
                                int head_dim, int elem_bytes, int block_size, int context_tokens,
                                int max_model_len, int64_t out[8]) {
  using pkv::fail;
  if (out == nullptr) return fail(PKV_EINVAL, "kv_pool_plan: out is NULL");
  for (int i = 0; i < 8; ++i) out[i] = 0;
  if (device_bytes <= 0 || weight_bytes < 0 || reserve_bytes < 0)
    return fail(PKV_EINVAL, "kv_pool_plan: device_bytes must be > 0, weight and reserve >= 0");
  if (utilization_ppm <= 0 || utilization_ppm > kPpm)
    return fail(PKV_EINVAL, "kv_pool_plan: utilization_ppm %d not in (0, 1000000]",
                utilization_ppm);
  if (utilization_of != PKV_UTIL_OF_REMAINDER && utilization_of != PKV_UTIL_OF_DEVICE)
    return fail(PKV_EINVAL, "kv_pool_plan: utilization_of %d is neither 0 nor 1",
                utilization_of);
  if (num_layers < 1 || num_layers > 4096 || num_kv_heads < 1 || num_kv_heads > 4096 ||
      head_dim < 1 || head_dim > 4096 || block_size < 1 || block_size > 4096)
    return fail(PKV_EINVAL, "kv_pool_plan: layers, heads, head_dim, block_size must be in "
                "[1, 4096]");
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4)
    return fail(PKV_EINVAL, "kv_pool_plan: elem_bytes %d is not 1, 2 or 4", elem_bytes);
  if (context_tokens < 1 || max_model_len < 1)
    return fail(PKV_EINVAL, "kv_pool_plan: context_tokens and max_model_len must be >= 1");

  // Bytes left for the pool. Either the fraction applies to what the weights and the reserve
  // leave over (the page's worked figure), or it caps everything the process may use and the
  // weights and the reserve come out of that cap.
  // (128-bit: weights and reserve near the int64 limit must not overflow; a shortfall beyond
  // the int64 range is reported as INT64_MIN, and such a pool holds no block either way)
  __int128 pool128 = 0;
  if (utilization_of == PKV_UTIL_OF_REMAINDER) {
    const __int128 left = static_cast<__int128>(device_bytes) - weight_bytes - reserve_bytes;
    pool128 = left > 0 ? scale_ppm(static_cast<int64_t>(left), utilization_ppm) : left;
  } else {
    pool128 = static_cast<__int128>(scale_ppm(device_bytes, utilization_ppm)) - weight_bytes -
              reserve_bytes;
  }
  const int64_t pool = pool128 < INT64_MIN ? INT64_MIN : static_cast<int64_t>(pool128);
  // at most 4096^3 * 2 * 4 = 2^39 bytes per token, 2^51 per block: no overflow in int64
  const int64_t per_token = static_cast<int64_t>(num_layers) * 2 * num_kv_heads * head_dim *
                            elem_bytes;
  const int64_t per_block = per_token * block_size;
  const int64_t blocks_per_request = (static_cast<int64_t>(context_tokens) + block_size - 1) /
                                     block_size;
  out[0] = pool;
  out[1] = per_token;
  out[2] = per_block;
  out[4] = blocks_per_request;
  if (pool < per_block)
    return fail(PKV_ENOBLOCKS, "kv_pool_plan: %lld bytes left for the pool hold no block of "
                "%lld bytes", static_cast<long long>(pool), static_cast<long long>(per_block));
  const int64_t num_blocks = pool / per_block;
  if (num_blocks > INT32_MAX / block_size)
    return fail(PKV_EINVAL, "kv_pool_plan: %lld blocks of %d tokens overflow the int32 slot "
                "ids", static_cast<long long>(num_blocks), block_size);
  out[3] = num_blocks;
  out[5] = num_blocks / blocks_per_request;
  out[6] = num_blocks * num_kv_heads * block_size * head_dim * elem_bytes;
  // contiguous reservation of max_model_len tokens per request (up to 2^70 bytes: 128-bit)
  out[7] = static_cast<int64_t>(static_cast<__int128>(pool) /
                                (static_cast<__int128>(per_token) * max_model_len));
  return pkv::ok();
}
