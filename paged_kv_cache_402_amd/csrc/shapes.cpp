// Host-side shape rules of the kernels (LDS of the decode pass, the limits of the
// shared-prefix pass): plain host code, so the C ABI's validation builds without the kernels.
#include "launch.h"
#include "pagedkv.h"

namespace pkv {

size_t decode_lds_bytes(int kv_dtype, int head_dim, int group, int part) {
  (void)kv_dtype;
  // per wave: its scores (part / 4 x group floats), reused for its merge data afterwards
  const int per = part / kDecodeWaves > head_dim + 2 ? part / kDecodeWaves : head_dim + 2;
  return (size_t)kDecodeWaves * (size_t)per * (size_t)group * 4;
}

bool prefix_supported(int kv_dtype, int head_dim, int group, int part, int bs_log2) {
  // 16-bit KV only: the pass's products are 16-bit matrix-core products
  return (kv_dtype == PKV_F16 || kv_dtype == PKV_BF16) && head_dim == kPrefixHeadDim &&
         (group == 1 || group == 2 || group == 4 || group == 8) && part % 32 == 0 &&
         (part >> bs_log2) <= kPrefixMaxIds;
}

int prefix_chunk_seqs(int group) { return 4 * (16 / group); }

}  // namespace pkv
