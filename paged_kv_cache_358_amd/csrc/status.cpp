// Status strings and ABI version.
#include "pagedattn.h"

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

int32_t pa_version(void) { return 100; }

}  // extern "C"
