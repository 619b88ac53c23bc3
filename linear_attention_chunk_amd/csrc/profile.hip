// Optional launch profiler: events recorded around each kernel launch on its own stream.  Also an
// MFMA-loop probe that measures the bf16 matrix-core rate the device reaches.
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
                                        "k_lin_delta", "k_lin_scan", "k_lin_apply", "k_phi", "k_w13_cvt", "k_zero",
                                        "k_par_momentum", "k_swa", "k_swa_qprep", "k_lin_bwd_t",
                                        "k_lin_bwd_n", "k_lin_deta_sum", "k_swa_vprep", "k_w13t_cvt",
                                        "k_phi_dx", "k_dw13", "k_dw_sum", "k_fb_prep", "k_fb_ops",
                                        "k_fb_up", "k_fb_dx", "k_fb_dw", "k_fb_misc", "k_nsb"};
}  // namespace

static thread_local bool t_prof_off = false;
ProfSuppress::ProfSuppress() : was(t_prof_off) { t_prof_off = true; }
ProfSuppress::~ProfSuppress() { t_prof_off = was; }

ProfScope::ProfScope(int id_, hipStream_t st_) : id(id_), st(st_) {
    if (t_prof_off || !g_on.load(std::memory_order_relaxed) || !((g_mask.load(std::memory_order_relaxed) >> id) & 1u))
        return;
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

namespace ttt {
constexpr int kProbeThreads = 256;
typedef __bf16 probe_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float probe_f32x16_t __attribute__((ext_vector_type(16)));

// Every wave runs iters rounds of four independent v_mfma_f32_32x32x16_bf16 on register operands
// (independent accumulators, and two waves per SIMD, cover the MFMA latency), then folds its
// accumulators into out[block] so that nothing is optimised away.  32 x 32 x 16 x 2 FLOP per MFMA.
__global__ __launch_bounds__(kProbeThreads) void k_mfma_probe(float* out, int iters) {
    probe_f32x16_t acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
    probe_bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
        b[e] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + e) & 7));
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[u][r];
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}
}  // namespace ttt

extern "C" ttt_status ttt_probe_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream) {
    clear_error();
    if (blocks < 1 || iters < 1 || !out) return fail(TTT_ERR_INVALID_ARGUMENT, "ttt_probe_mfma_bf16: bad arguments");
    hipLaunchKernelGGL(k_mfma_probe, dim3(blocks), dim3(kProbeThreads), 0, (hipStream_t)stream, out, iters);
    return check_launch("k_mfma_probe", (hipStream_t)stream);
}
