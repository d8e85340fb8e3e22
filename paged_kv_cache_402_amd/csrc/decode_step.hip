// The per-partition decode pass of one-pass decode steps whose launch carries copy-on-write
// sources (P1 §6.2; P2 §2.2): the kernels of decode_kernel.h built with the copy's stores.
// Kept in a translation unit of its own so that both sets of kernels compile in parallel.
#include "decode_kernel.h"

namespace pkv {

hipError_t launch_decode_partitions_cow(const DecodeArgs& a, int kv_dtype, int head_dim,
                                        int group, hipStream_t stream, int* ticketed) {
  switch (kv_dtype) {
    case F32: return launch_d<F32, true>(a, head_dim, group, stream, ticketed);
    case F16: return launch_d<F16, true>(a, head_dim, group, stream, ticketed);
    case BF16: return launch_d<BF16, true>(a, head_dim, group, stream, ticketed);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
