// Internal helpers of the C ABI layer: thread-local error message.
#pragma once

#include "blockdiag.h"

namespace bd {
// Records a formatted message for blockdiag_last_error() and returns code.
bd_status fail(bd_status code, const char* fmt, ...);
void clear_error();
}  // namespace bd
