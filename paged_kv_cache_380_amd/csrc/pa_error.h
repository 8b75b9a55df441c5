// The library's per-thread error message (returned by pa_last_error).
// Plain C++ so that host-only sources can use it without the HIP headers.
#pragma once

namespace pa {

// Records a printf-style message for the calling thread and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns PA_OK (0).
int ok();

}  // namespace pa
