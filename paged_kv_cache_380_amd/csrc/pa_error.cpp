// Per-thread error message of the C ABI (see pa_error.h and pa_last_error in include/pa.h).
#include "pa_error.h"

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"

namespace {
thread_local std::string g_last_error;
}

namespace pa {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }
