// Status codes, per-thread error text, the version of libpagedattn and the
// PAGEDATTN_* overrides.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "options.hpp"
#include "pagedattn.h"

namespace pa {

namespace {

Options read_options() {
  Options o;
  if (const char* v = getenv("PAGEDATTN_HEADS_PER_WG")) o.heads_per_wg = atoi(v);
  if (const char* v = getenv("PAGEDATTN_DECODE_KERNEL")) o.valu_only = strcmp(v, "valu") == 0;
  if (const char* v = getenv("PAGEDATTN_MERGE")) {
    if (strcmp(v, "separate") == 0) o.merge = 1;
    if (strcmp(v, "inkernel") == 0) o.merge = 2;
  }
  if (const char* v = getenv("PAGEDATTN_SCHEDULE")) {
    if (strcmp(v, "fixed") == 0) o.schedule = 1;
    if (strcmp(v, "stream") == 0) o.schedule = 2;
  }
  if (const char* v = getenv("PAGEDATTN_STREAM_WORKERS")) o.stream_workers = atoi(v);
  if (const char* v = getenv("PAGEDATTN_PREFILL_KSPLIT")) {
    if (v[0] == '1') o.prefill_ksplit = 1;
    if (v[0] == '2') o.prefill_ksplit = 2;
  }
  return o;
}

// The options in use; replaced whole (never modified) by pa_reload_options,
// so a call reads one consistent set.
std::atomic<const Options*> g_options{nullptr};

}  // namespace

const Options& options() {
  const Options* o = g_options.load(std::memory_order_acquire);
  if (o == nullptr) {
    const Options* fresh = new Options(read_options());
    const Options* expected = nullptr;
    if (g_options.compare_exchange_strong(expected, fresh, std::memory_order_acq_rel))
      return *fresh;
    delete fresh;
    return *expected;
  }
  return *o;
}

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

// Earlier option sets are kept (a call on another thread may still read
// one); each is a few bytes and this runs only when a test or a tuning run
// changes the environment.
extern "C" void pa_reload_options(void) {
  pa::g_options.store(new pa::Options(pa::read_options()), std::memory_order_release);
}
