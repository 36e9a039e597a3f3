// Host-side pieces shared by every entry point: the thread-local error text,
// the launch check and the ABI version.
#include <cstdarg>
#include <cstdio>

#include "step_launch.h"
#include "td_internal.h"

namespace td {

namespace {
thread_local char g_err[512] = {0};
}

thread_local LaunchEvents t_launch_events = {nullptr, nullptr};

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

using namespace td;

extern "C" td_status td_workspace_status(void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (!workspace || !aligned16(workspace))
        return fail(TD_EINVAL, "td_workspace_status: null or misaligned workspace");
    if (workspace_bytes < kStatusBytes)
        return fail(TD_EINVAL, "td_workspace_status: workspace smaller than its status header");
    hipStream_t s = as_stream(stream);
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        set_error("td_workspace_status: reading the status word failed: %s", hipGetErrorString(e));
        return TD_EHIP;
    }
    if (word == 0) return TD_OK;
    const uint32_t zero = 0;
    e = hipMemcpyAsync(workspace, &zero, sizeof zero, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        set_error("td_workspace_status: clearing the status word failed: %s", hipGetErrorString(e));
        return TD_EHIP;
    }
    set_error("a cross-workgroup hand-off gave up waiting (%s%s%s%s%s); the workspace was not "
              "zero-filled after a shape change, or was shared by overlapping calls",
              (word & kStatusMerge) ? "row merge: lse NaN" : "",
              (word & kStatusMerge) && (word & (kStatusTree | kStatusSplit)) ? ", " : "",
              (word & kStatusTree) ? "tree build: n_nodes -1" : "",
              (word & kStatusTree) && (word & kStatusSplit) ? ", " : "",
              (word & kStatusSplit) ? "context split: attention partials not written" : "");
    return TD_ESYNC;
}
