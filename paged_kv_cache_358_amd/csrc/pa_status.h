// Internal: remembering the HIP error behind a PA_ERR_HIP status.
#pragma once

#include <stdint.h>

namespace pa {
// Stores "where: name (code): text" for pa_last_error() and returns PA_ERR_HIP.
int32_t record_hip_error(const char* where, int code, const char* name, const char* text);
}  // namespace pa

// Returns PA_OK if the last HIP call/launch succeeded, else records the error.
#define PA_HIP_STATUS(where, err)                                                                         \
  ((err) == hipSuccess ? PA_OK                                                                          \
                       : ::pa::record_hip_error((where), static_cast<int>(err), hipGetErrorName(err),   \
                                                hipGetErrorString(err)))
