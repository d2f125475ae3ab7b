// host_errors.h - status reporting shared by every entry point: the
// thread-local message behind kvoff_last_error() and the guard that keeps
// C++ exceptions from crossing the C ABI.  Host code only (no HIP), so the
// host-only parts of the library also build and run under the CPU
// sanitizers.
#pragma once

#include <exception>
#include <new>

#include "../../include/kvoff.h"

namespace kvoff {

// sets the calling thread's message of the last failure
void set_error(const char* fmt, ...);
// sets the message and returns `status`
int fail(int status, const char* fmt, ...);

// Runs an entry point's body and turns any C++ exception (a failed host
// allocation, a worker thread that cannot be created) into a status code, so
// none crosses the C ABI.
template <class F>
int guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(KVOFF_ENOMEM, "host memory allocation failed");
  } catch (const std::exception& e) {
    return fail(KVOFF_ESTATE, "internal error: %s", e.what());
  } catch (...) {
    return fail(KVOFF_ESTATE, "internal error");
  }
}

}  // namespace kvoff
