// Thread-local error text behind pkv_last_error(). Host code only, so the host block manager,
// scheduler and pool planner build and link without the HIP runtime.
#include "errors.h"

#include <cstdio>
#include <string>

#include "pagedkv.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PKV_OK;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }
