// Internal accessors of the host block manager for the other host modules of the library.
#pragma once

#include "pagedkv.h"

namespace pkv {

// Block size the manager was created with.
int bm_block_size(const pkv_bm* bm);

}  // namespace pkv
