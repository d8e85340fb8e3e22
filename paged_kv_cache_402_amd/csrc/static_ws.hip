// A fixed split-K scratch area in device memory for the decode entry point that allocates
// nothing (pkv_paged_attention_decode_noalloc): callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc) still need the
// per-(sequence, query head, partition) partials of the two-pass decode somewhere.
//
// The area is a file-scope device array: every GPU the library runs on holds its own copy,
// at its own address, from the library's first use on that device until the process ends.
// Host code never uses the array's name as a device address (on the host it names a
// stand-in); the address is resolved once per device with hipGetSymbolAddress, with that
// device current, and kept.
#include <atomic>

#include <hip/hip_runtime.h>

#include "launch.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

hipError_t static_workspace(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace pkv
