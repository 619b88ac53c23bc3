// Optional launch profiler: events recorded around each kernel launch on its own stream.
#include <atomic>
#include <mutex>
#include <vector>

#include "host_common.hpp"

namespace ttt {
namespace {
std::atomic<bool> g_on{false};
std::atomic<uint32_t> g_mask{0xFFFFFFFFu};  // kernel classes that are bracketed while enabled
std::mutex g_mu;
struct Rec { int id; hipEvent_t a, b; };
std::vector<Rec> g_recs;
const char* kNames[TTT_PROF_KERNELS] = {"k_up", "k_down", "k_update", "k_muon_prep",
                                        "k_ns_init", "k_ns_gram", "k_ns_step", "k_linattn",
                                        "k_lin_delta", "k_lin_scan", "k_lin_apply"};
}  // namespace

ProfScope::ProfScope(int id_, hipStream_t st_) : id(id_), st(st_) {
    if (!g_on.load(std::memory_order_relaxed) || !((g_mask.load(std::memory_order_relaxed) >> id) & 1u)) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) { a = b = nullptr; return; }
    (void)hipEventRecord(a, st);
}

ProfScope::~ProfScope() {
    if (!a) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back({id, a, b});
}
}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_profile_enable(int32_t on) {
    g_on.store(on != 0);
    return TTT_OK;
}

extern "C" ttt_status ttt_profile_select(uint32_t mask) {
    g_mask.store(mask);
    return TTT_OK;
}

extern "C" ttt_status ttt_profile_read(float* ms, int32_t* count, int32_t n) {
    clear_error();
    if (n < 0 || n > TTT_PROF_KERNELS || (n > 0 && (!ms || !count)))
        return fail(TTT_ERR_INVALID_ARGUMENT, "ttt_profile_read: bad arguments");
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        recs.swap(g_recs);
    }
    for (int i = 0; i < n; ++i) { ms[i] = 0.f; count[i] = 0; }
    ttt_status rc = TTT_OK;
    for (const Rec& r : recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            rc = fail(TTT_ERR_DEVICE, "ttt_profile_read: event query failed");
        else if (r.id < n) { ms[r.id] += t; count[r.id] += 1; }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    return rc;
}

extern "C" const char* ttt_profile_kernel_name(int32_t i) {
    return (i >= 0 && i < TTT_PROF_KERNELS) ? kNames[i] : "";
}
