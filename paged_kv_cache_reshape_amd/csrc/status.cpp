// Status codes, per-thread error text and the version of libpagedattn.
#include <stdarg.h>
#include <stdio.h>

#include "pagedattn.h"

namespace pa {

static thread_local char g_message[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_message, sizeof(g_message), fmt, ap);
  va_end(ap);
}

void clear_error() { g_message[0] = '\0'; }

}  // namespace pa

extern "C" int32_t pa_version(void) { return 100; }  // 0.1.0

extern "C" const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char* pa_last_error_message(void) { return pa::g_message; }
