// The per-partition decode pass of one-pass decode steps over fork groups (P2 §2.2: the
// branches of a parallel-sampling fork share their prompt's blocks until each writes its own
// token; P1 §6.2): the kernels of decode_kernel.h whose workgroup rows are the query heads of
// several such branches. Kept in a translation unit of its own so that it compiles in parallel
// with the others.
#include "decode_kernel.h"

namespace pkv {

hipError_t launch_decode_partitions_groups(const DecodeArgs& a, int kv_dtype, int head_dim,
                                           int rows, hipStream_t stream, int* ticketed) {
  switch (kv_dtype) {
    case F32: return launch_d<F32, true, true>(a, head_dim, rows, stream, ticketed);
    case F16: return launch_d<F16, true, true>(a, head_dim, rows, stream, ticketed);
    case BF16: return launch_d<BF16, true, true>(a, head_dim, rows, stream, ticketed);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
