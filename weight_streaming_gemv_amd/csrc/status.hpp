// Error reporting for the C ABI: a thread-local last-error message.
#pragma once
#include <stdarg.h>
#include <stdio.h>

#include "../../include/wsg.h"

namespace wsg {

extern thread_local char g_last_error[512];

inline void clear_error() { g_last_error[0] = 0; }

inline wsg_status fail(wsg_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
inline wsg_status fail(wsg_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace wsg

#define WSG_HIP_CHECK(expr)                                                                  \
  do {                                                                                       \
    const hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess)                                                                    \
      return ::wsg::fail(WSG_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));        \
  } while (0)
