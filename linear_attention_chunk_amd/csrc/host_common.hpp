// Host-side helpers shared by the C ABI translation units: error reporting and checked launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "ttt.h"

namespace ttt {

void set_error(const char* fmt, ...);
void clear_error();

inline ttt_status fail(ttt_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    set_error("%s", buf);
    return s;
}

// kernel classes of the optional launch profiler (ttt_profile_*)
enum ProfKernel { PK_UP = 0, PK_DOWN, PK_UPDATE, PK_MUON_PREP, PK_NS_INIT, PK_NS_GRAM, PK_NS_STEP, PK_LINATTN,
                  PK_LIN_DELTA, PK_LIN_SCAN, PK_LIN_APPLY };

// Brackets one launch with events on its stream while profiling is enabled; no-op otherwise.
struct ProfScope {
    int id;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(int id_, hipStream_t st_);
    ~ProfScope();
};

inline ttt_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TTT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return TTT_OK;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace ttt
