// Status strings, ABI version and the last HIP error text.
#include <cstdio>

#include "pagedattn.h"
#include "pa_status.h"

namespace pa {
static thread_local char g_last_error[256] = "";

int32_t record_hip_error(const char* where, int code, const char* name, const char* text) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d): %s", where, name, code, text);
  return PA_ERR_HIP;
}
}  // namespace pa

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    default: return "PA_ERR_UNKNOWN";
  }
}

int32_t pa_version(void) { return 200; }

const char* pa_last_error(void) { return pa::g_last_error; }

}  // extern "C"
