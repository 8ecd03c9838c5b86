// status.h -- error reporting shared by the C-ABI sources of the library.
#pragma once

#include <stdint.h>

namespace atlas {

// Records a printf-style message for atlas_last_error() (per thread) and
// returns status.
int32_t fail(int32_t status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the message and returns ATLAS_OK.
int32_t ok();

// The current thread's last message ("" after a success).
const char *last_error();

}  // namespace atlas
