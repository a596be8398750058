// Status strings and per-thread error text for the C ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace pi {

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

pi_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return PI_ERR_HIP;
  }
  return PI_OK;
}

}  // namespace pi

extern "C" const char* pi_status_string(pi_status status) {
  switch (status) {
    case PI_OK: return "ok";
    case PI_ERR_INVALID_ARG: return "invalid argument";
    case PI_ERR_UNSUPPORTED: return "unsupported shape";
    case PI_ERR_WORKSPACE: return "workspace too small";
    case PI_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

extern "C" const char* pi_last_error(void) { return g_last_error; }
