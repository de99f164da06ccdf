// status.cpp -- thread-local error text and version of libsconv.
#include <stdarg.h>
#include <stdio.h>

#include "sconv_host.h"

namespace sconv {

static thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SCONV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return SCONV_OK;
}

}  // namespace sconv

extern "C" const char* sconv_last_error(void) { return sconv::g_error; }

extern "C" const char* sconv_version(void) { return "libsconv 0.1.0 gfx950"; }
