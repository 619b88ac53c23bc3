// Status strings, the per-thread error message and the ABI version.
#include <stdio.h>
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
    }
    return "unknown status";
}
