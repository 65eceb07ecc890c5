// Host-side internals shared by the C-ABI translation units.
#pragma once
#include <stdarg.h>
#include <stdio.h>

#include "medusa_verify.h"

namespace mv {

char* last_error_buf();

// Record a formatted error message and return `status`.
inline int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(last_error_buf(), 512, fmt, ap);
  va_end(ap);
  return status;
}

}  // namespace mv
