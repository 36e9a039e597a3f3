// Host-side pieces shared by every entry point: the thread-local error text,
// the launch check and the ABI version.
#include <cstdarg>
#include <cstdio>

#include "td_internal.h"

namespace td {

namespace {
thread_local char g_err[512] = {0};
}

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = 0; }

td_status check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
        return TD_EHIP;
    }
    return TD_OK;
}

}  // namespace td

extern "C" int td_abi_version(void) { return TD_ABI_VERSION; }

extern "C" const char *td_last_error(void) { return td::g_err; }
