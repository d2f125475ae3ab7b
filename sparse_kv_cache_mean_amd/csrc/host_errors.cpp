// host_errors.cpp - the thread-local failure message and the status strings
// of kvoff.h (host code only).
#include "host_errors.h"

#include <cstdarg>
#include <cstdio>

namespace kvoff {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace kvoff

extern "C" {

const char* kvoff_strerror(int status) {
  switch (status) {
    case KVOFF_OK: return "success";
    case KVOFF_EINVAL: return "invalid argument";
    case KVOFF_ENOMEM: return "host memory allocation failed";
    case KVOFF_ENODEV: return "no usable GPU";
    case KVOFF_EHIP: return "HIP runtime error";
    case KVOFF_ERANGE: return "capacity or size exceeded";
    case KVOFF_ESTATE: return "invalid state";
    default: return "unknown status";
  }
}

const char* kvoff_last_error(void) { return kvoff::g_last_error; }

}  // extern "C"
