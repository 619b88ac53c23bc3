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
                  PK_LIN_DELTA, PK_LIN_SCAN, PK_LIN_APPLY, PK_PHI, PK_W13, PK_ZERO, PK_PAR_MOM, PK_SWA,
                  PK_SWA_PREP, PK_LIN_BWD_T, PK_LIN_BWD_N, PK_LIN_DETA, PK_SWA_VPREP, PK_W13T, PK_PHI_DX,
                  PK_DW13, PK_DW_SUM, PK_FB_PREP, PK_FB_OPS, PK_FB_UP, PK_FB_DX, PK_FB_DW, PK_FB_MISC,
                  PK_FB_NSB };

// Brackets one launch with events on its stream while profiling is enabled; no-op otherwise.
struct ProfScope {
    int id;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(int id_, hipStream_t st_);
    ~ProfScope();
};

// Whether TTT_DEBUG_SYNC is set (to anything but "" or "0") in the environment, read once: then every
// launch is followed by a synchronisation of its stream, so that a kernel that fails is reported by
// the call that launched it (a debugging aid; it serialises the host with the device, and a stream
// under graph capture cannot be synchronised, so such a call returns TTT_ERR_DEVICE).
bool debug_sync();

// While one exists on a thread, launches on that thread are not bracketed by the profiler (whose
// events are created per launch): used by the entry point that must not allocate.
struct ProfSuppress {
    bool was;
    ProfSuppress();
    ~ProfSuppress();
};

inline ttt_status check_launch(const char* what, hipStream_t st) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TTT_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    if (debug_sync()) {
        e = hipStreamSynchronize(st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(TTT_ERR_DEVICE, "%s (TTT_DEBUG_SYNC): %s", what, hipGetErrorString(e));
        }
    }
    return TTT_OK;
}

// Argument check for one device buffer: p must lie in memory that HIP allocated on a device, with at
// least `bytes` of that allocation from p on.  A host pointer, a stale or foreign address, or a buffer
// too short for the call is refused before anything is enqueued (a null p or zero bytes passes).
// Without a usable HIP device the answer is TTT_ERR_DEVICE.
ttt_status check_buffer(const void* p, size_t bytes, const char* name);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The chunk-parallel linear-attention path (chunked masks) as a building block, also used by the
// TTT layer's parallel form.  State of scan s on entry: S0 + (s0_heads ? s % s0_heads : s) *
// s0_stride (zero if S0 is null); on exit it goes to Sout + s * sout_stride (if not null).  Each
// updating chunk then adds, reps times, u = dsign * dS_c, either directly (S <- S + u) or, with
// mom, through a running term m <- beta m + u, S <- S + m, where m starts as msign * M0[s]
// (zero if M0 is null) and leaves as msign * m in Mout[s] (both m_stride apart).
struct LinStateIO {
    const float* S0 = nullptr;
    int64_t s0_stride = 0;
    int s0_heads = 0;
    float* Sout = nullptr;
    int64_t sout_stride = 0;
    const float* M0 = nullptr;
    float* Mout = nullptr;
    int64_t m_stride = 0;
    int mom = 0;
    float beta = 0.f, msign = 1.f, dsign = 1.f;
    int reps = 1;
    // Optional step between the chunk updates and the scan: called with dS (nscan x nchunks
    // matrices of d_v x d_k, fp32; chunks a strided mask skips hold no data), it enqueues work on
    // the stream and sets *src to the buffer of the same layout that the scan then reads as dS.
    ttt_status (*between)(void* ctx, float* dS, const float** src, hipStream_t st) = nullptr;
    void* between_ctx = nullptr;
};
// workspace of lin_chunked_run: dS_c (fp32) and S_c (one plane of es-byte elements) per chunk
size_t lin_chunked_ws_bytes(int64_t nscan, int64_t nchunks, int d_k, int d_v, size_t es);
// D.mask is a chunked mask (not TOKEN_CAUSAL); flags holds the strided update bits (bit j = chunk j)
template <typename T>
ttt_status lin_chunked_run(const linattn_desc& D, const uint32_t (&flags)[32], const T* q, const T* k, const T* v,
                           const float* eta, T* o, const LinStateIO& io, char* ws, hipStream_t st);

// The checks of a TTT layer descriptor shared by the forward and the backward entry points
ttt_status validate_ttt_desc(const ttt_desc* D);

// The backward of the chunked path as a building block (also driven by the TTT layer's backward).
// S0 of scan s at S0 + (s0_heads ? s % s0_heads : s) * s0_stride (null: zeros); dS_out of scan s at
// dS_out + s * dso_stride (null: zeros); dS0 of scan s to dS0 + s * ds0_stride (null: not written).
// The forward's updating chunks added u = dsign * sum eta v k^T to the state reps times, directly
// or (mom) through a running term m <- beta m + u, S <- S + m that started at zero and whose final
// value is not part of the loss; with norm every step's S then had its rows L2-normalized.
// gate[0], gate[1]: both null, or [S][N][2 d_k] buffers of io-dtype factors u | w for dq and dk:
// then dq and dk are not written; each gate row becomes dq u | dq w (dk u | dk w) in place.
struct LinBwdIO {
    const float* S0 = nullptr;
    int64_t s0_stride = 0;
    int s0_heads = 0;
    const float* dS_out = nullptr;
    int64_t dso_stride = 0;
    float* dS0 = nullptr;
    int64_t ds0_stride = 0;
    float dsign = 1.f;
    int reps = 1;
    int mom = 0;
    float beta = 0.f;
    int norm = 0;  // each step ends in the L2 norm of the state's rows (over d_k), w / max(|w|, 1e-6)
    void* gate[2] = {nullptr, nullptr};
};
// the backward's checks of a linear-attention descriptor
ttt_status validate_lin_desc_bwd(const linattn_desc* D);
// workspace of lin_chunked_bwd (norm, reps: those of the LinBwdIO the call will take)
size_t lin_chunked_bwd_ws_bytes(const linattn_desc& D, int norm = 0, int reps = 1);
// D.mask is a chunked mask (not TOKEN_CAUSAL); flags as for lin_chunked_run.  dq, dk [S][N][d_k],
// dv [S][N][d_v], deta [S][N] as for linattn_backward.
template <typename T>
ttt_status lin_chunked_bwd(const linattn_desc& D, const uint32_t (&flags)[32], const T* q, const T* k, const T* v,
                           const float* eta, const T* dO, const LinBwdIO& io, T* dq, T* dk, T* dv, float* deta,
                           char* ws, hipStream_t st);

// The forward recurrence run for its record: the weights before each update at hist + i S 3 d m
// (i = 0 .. updates, the last one the final weights) and, with the norm, each update's row norms
// (|W - U| of the 2m + d rows) at nrm + i S (2m + d).  ws: ttt_history_ws_bytes.
// With Muon each update's U (the input of Newton-Schulz, fp32) goes to urec + i S 3 d m.  o and
// W_out are the forward's outputs (null: not written; with o null nothing is applied).
size_t ttt_history_ws_bytes(const ttt_desc& D);
template <typename T>
ttt_status ttt_run_history(const ttt_desc& D, const T* q, const T* k, const T* v, const float* eta, const float* W0,
                           T* o, float* W_out, float* hist, float* nrm, float* urec, char* ws, hipStream_t st);
// Newton-Schulz steps from X_0 at X for the backward: for k < ns_iters the Gram matrix of X_k at
// P + k S 3 p^2 and, but for the last, X_{k+1} at X + (k + 1) S 3 d m (bf16: hi planes, the lo plane
// Xlo carried in place); the learned matrices only (W2 alone with last_layer_only).
template <typename T>
ttt_status ns_steps(const ttt_desc& D, T* X, T* Xlo, T* P, hipStream_t st);

// The backward of the recurrence with all three weights learning (GD or GD + L2, momentum): the
// descriptor checks beyond validate_ttt_desc, the workspace, and the run (arguments as for
// ttt_backward, already checked).
// With a record (from run_forward_record) the forward is not run again and the workspace is
// full_bwd_ws_bytes(D, false); W0 is then not read.
ttt_status validate_full_bwd(const ttt_desc* D);
size_t full_bwd_ws_bytes(const ttt_desc& D, bool own_record = true);
template <typename T>
ttt_status run_full_backward(const ttt_desc& D, const T* q, const T* k, const T* v, const float* eta, const float* W0,
                             const T* dO, const float* dWo, T* dq, T* dk, T* dv, float* deta, float* dW0, char* ws,
                             hipStream_t st, char* record = nullptr);
// The training forward: o and W_out as ttt_forward writes them (momentum from zero), and the record
// the backward of the recurrence reads (full_bwd_record_bytes); workspace ttt_history_ws_bytes.
size_t full_bwd_record_bytes(const ttt_desc& D);
template <typename T>
ttt_status run_forward_record(const ttt_desc& D, const T* q, const T* k, const T* v, const float* eta, const float* W0,
                              T* o, float* W_out, char* record, char* ws, hipStream_t st);

}  // namespace ttt
