// Status strings and the thread-local last-error message of the CSA2 C ABI.
#include <string>

#include "csa2_host.h"

namespace csa2 {

static thread_local std::string g_last_error;

csa2_status_t fail(csa2_status_t s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

csa2_status_t check_launch(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CSA2_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return CSA2_OK;
}

}  // namespace csa2

extern "C" const char* csa2_status_string(csa2_status_t status)
{
    switch (status) {
        case CSA2_OK: return "CSA2_OK";
        case CSA2_ERR_NULL: return "CSA2_ERR_NULL";
        case CSA2_ERR_SHAPE: return "CSA2_ERR_SHAPE";
        case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED";
        case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE";
        case CSA2_ERR_LAUNCH: return "CSA2_ERR_LAUNCH";
        case CSA2_ERR_DEVICE_CHECK: return "CSA2_ERR_DEVICE_CHECK";
        default: return "CSA2_ERR_UNKNOWN";
    }
}

extern "C" const char* csa2_last_error(void) { return csa2::g_last_error.c_str(); }

extern "C" int csa2_abi_version(void) { return CSA2_ABI_VERSION; }
