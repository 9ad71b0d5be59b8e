// Thread-local error text for kvq_last_error() and the launch check.
#include <stdarg.h>
#include <stdio.h>

#include "kvq_common.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace kvq {

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return code;
}

int launch_status(const char *what) {
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) return KVQ_OK;
    int code = (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction ||
                e == hipErrorNoDevice || e == hipErrorInsufficientDriver)
                   ? KVQ_E_UNSUPPORTED
                   : KVQ_E_LAUNCH;
    return fail(code, "%s: launch failed: %s", what, hipGetErrorString(e));
}

}  // namespace kvq

extern "C" const char *kvq_last_error(void) { return g_msg; }

extern "C" int kvq_abi_version(void) { return 100; }
