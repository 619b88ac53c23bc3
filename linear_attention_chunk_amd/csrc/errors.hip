// Status strings, the per-thread error message and the ABI version.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "host_common.hpp"

namespace ttt {
static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}
void clear_error() { g_err[0] = 0; }
}  // namespace ttt

extern "C" int32_t ttt_abi_version(void) { return TTT_ABI_VERSION; }

extern "C" const char* ttt_last_error(void) { return ttt::g_err; }

extern "C" const char* ttt_status_string(ttt_status s) {
    switch (s) {
        case TTT_OK: return "ok";
        case TTT_ERR_INVALID_ARGUMENT: return "invalid argument";
        case TTT_ERR_UNSUPPORTED: return "unsupported combination";
        case TTT_ERR_WORKSPACE: return "workspace missing or too small";
        case TTT_ERR_DEVICE: return "HIP device or launch error";
        default: break;
    }
    return "unknown status";
}

namespace ttt {
bool debug_sync() {
    static const bool on = [] {
        const char* e = getenv("TTT_DEBUG_SYNC");
        return e && e[0] && !(e[0] == '0' && e[1] == 0);
    }();
    return on;
}

ttt_status check_buffer(const void* p, size_t bytes, const char* name) {
    if (!p || bytes == 0) return TTT_OK;
    void* base = nullptr;
    size_t size = 0;
    hipError_t e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
    if (e != hipSuccess) {
        (void)hipGetLastError();  // leave no sticky error for the caller's next HIP call
        int n = 0;
        hipError_t c = hipGetDeviceCount(&n);
        if (c != hipSuccess || n == 0) {
            (void)hipGetLastError();
            return fail(TTT_ERR_DEVICE, "no usable HIP device (%s)", hipGetErrorString(c != hipSuccess ? c : e));
        }
        return fail(TTT_ERR_INVALID_ARGUMENT, "%s (%p) is not in device memory allocated by HIP", name, p);
    }
    const uintptr_t end = (uintptr_t)base + size, x = (uintptr_t)p;
    if (x < (uintptr_t)base || bytes > end - x)
        return fail(TTT_ERR_INVALID_ARGUMENT, "%s: the call reads or writes %zu bytes from %p, its allocation holds %zu",
                    name, bytes, p, (size_t)(end - x));
    return TTT_OK;
}
}  // namespace ttt
