// pa_error.cpp -- return-code descriptions and the per-thread message
// behind pa_last_error() (host code only; shared by the attention entry
// points and the block allocator).
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"
#include "pa_error.h"

namespace pa {

namespace {
thread_local std::string g_last_error;
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

}  // namespace pa

extern "C" {

const char* pa_strerror(int code) {
  switch (code) {
    case PA_OK: return "success";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "not enough free cache blocks";
  }
  return "unknown error";
}

const char* pa_last_error(void) { return pa::last_error(); }

}  // extern "C"
