// vox_api.cpp - status codes and error reporting of the libvox C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "vox_host.h"

namespace vox {

static thread_local char g_last_error[512];

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_last_error[0] = 0;
    return VOX_OK;
}

int check_hip(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(VOX_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return VOX_OK;
}

int check_launch(const char *what) { return check_hip(hipGetLastError(), what); }

int cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace vox

extern "C" const char *vox_strerror(int status)
{
    switch (status) {
    case VOX_OK: return "ok";
    case VOX_E_INVAL: return "invalid argument";
    case VOX_E_UNSUPPORTED: return "unsupported shape or layout";
    case VOX_E_WORKSPACE: return "workspace or buffer too small";
    case VOX_E_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

extern "C" const char *vox_last_error(void) { return vox::g_last_error; }
