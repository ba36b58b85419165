// swa_error.cpp -- the thread-local message behind swa_last_error() and the
// helper every entry point reports through.  Host code only.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace swa {

static thread_local char g_err[512];

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

}  // namespace swa

extern "C" const char *swa_last_error(void) { return swa::g_err; }
