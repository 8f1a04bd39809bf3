// pa_error.h -- the library's per-thread error message (pa_last_error).
#pragma once

namespace pa {

// Record a printf-style message for pa_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char* last_error();

}  // namespace pa
