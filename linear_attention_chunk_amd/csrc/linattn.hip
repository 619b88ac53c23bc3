// Chunked linear attention on gfx950: the linear, bias-free fast weight S (d_v x d_k) under plain GD
// with the dot-product loss, S <- S + sum_i eta_i v_i k_i^T, o = S q ("Test-Time Training with KV
// Binding Is Secretly Linear Attention", Thm. 5.2 and Sec. 6.1 Step 6), with the chunk orders of
// the PaperTrace notes' section 1.1 and the token-causal limit ("From Linear Attention to Test-Time
// Training", causal linear attention).
//
// One workgroup owns one (batch, head) scan and a 32-row slice of S's d_v rows, and walks the
// sequence in sub-blocks of TB tokens.  The slice of S stays in MFMA accumulators (fp32) for the
// whole sequence; the update is an MFMA accumulation over the sub-block's tokens.  The apply reads
// S from LDS, where it is kept as a bf16 hi + lo pair (fp32 in fp32 mode) refreshed at chunk ends,
// so the query products see S to about 16 bits.  Token-causal mode adds the masked intra-block term
// tril(Q K^T) (eta o V) and refreshes S after every sub-block.  The next sub-block's q, k, v and eta
// are loaded into registers while the current one is computed.
#include <algorithm>

#include "host_common.hpp"
#include "tile.hpp"

namespace ttt {

template <typename T> struct LinArgs {
    const T* q; const T* k; const T* v; const float* eta; const float* S0; T* o; float* Sout;
    int64_t N; int dv; int chunk; int mode; int nvt; int vt;
    uint32_t flags[32];  // STRIDED: bit j = chunk j updates
};

// C[i][j] += sum_k A[i][k] B[j][k]; A, B k-contiguous in LDS (pitches pa, pb), kbytes % 64 == 0
template <typename T, int FM, int FN>
__device__ __forceinline__ void lds_mma(f32x4_t (&acc)[FM][FN], const char* A, int pa, int ar0, const char* B,
                                        int pb, int br0, int kbytes) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lk = (lane >> 4) * 16;
    for (int kk = 0; kk < kbytes; kk += 64) {
        u32x4_t af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(A + (ar0 + i * 16 + lr) * pa + kk + lk);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const u32x4_t*>(B + (br0 + j * 16 + lr) * pb + kk + lk);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) Elt<T>::mma(acc[i][j], af[i], bfr[j]);
    }
}

__device__ __forceinline__ u32x4_t scale_vec(const u32x4_t& x, float s, uint16_t) {
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float lo = bf2f((uint16_t)(x[w] & 0xFFFFu)) * s, hi = bf2f((uint16_t)(x[w] >> 16)) * s;
        r[w] = (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
    }
    return r;
}
__device__ __forceinline__ u32x4_t scale_vec(const u32x4_t& x, float s, float) {
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w) r[w] = __float_as_uint(__uint_as_float(x[w]) * s);
    return r;
}

template <typename T, int DK, bool CAUSAL, int VT_> struct LinCfg {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VEC = 16 / ES;
    static constexpr int TB = ES == 2 ? 64 : 32;  // tokens per sub-block
    static constexpr int VT = VT_;                 // d_v rows of S per workgroup (16 or 32)
    static constexpr int PQ = DK * ES + 16;        // LDS pitch of rows of DK elements
    static constexpr int PT = TB * ES + 16;        // LDS pitch of rows of TB elements
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_KT = OFF_Q + TB * PQ;
    static constexpr int OFF_VT = OFF_KT + DK * PT;
    static constexpr int OFF_SH = OFF_VT + VT * PT;
    static constexpr int OFF_SL = OFF_SH + VT * PQ;
    static constexpr int OFF_K = OFF_SL + (ES == 2 ? VT * PQ : 0);  // causal only
    static constexpr int OFF_P = OFF_K + (CAUSAL ? TB * PQ : 0);     // causal only
    static constexpr int LDS = OFF_P + (CAUSAL ? TB * PT : 0);
    // apply / intra-block tiling: 16 token rows per wave, AWN waves across columns
    static constexpr int AWN = TB == 64 ? 1 : 2;
    static constexpr int AFN = VT / 16 / AWN;
    static constexpr int PFN = TB / 16 / AWN;
    // state tiling: WSV x WSK waves over VT x DK, 16-wide MFMA blocks
    static constexpr int WSV = VT / 16, WSK = 4 / WSV;
    static constexpr int SFN = DK / 16 / WSK;
    static_assert(DK % (16 * WSK) == 0 && (VT == 32 || TB == 64), "state tiling");
    // register staging of one sub-block: q rows, and k and v in VEC x VEC (token x feature) blocks
    static constexpr int QV = TB * DK * ES / 16;
    static constexpr int QPER = (QV + kThreads - 1) / kThreads;
    static constexpr int KU = (TB / VEC) * (DK / VEC);
    static constexpr int KPER = (KU + kThreads - 1) / kThreads;
    static constexpr int VU = (TB / VEC) * (VT / VEC);
    static_assert(VU <= kThreads, "v staging");
};

// One unit of work of a workgroup: a sub-block of at most TB tokens of one chunk, applied and/or
// used for the update, in the order the mask fixes (notes section 1.1).  Apply-then-update walks
// each chunk once; update-then-apply walks a chunk's sub-blocks for the update, then again for
// the apply; token-causal treats every sub-block as its own chunk with the intra-block term.
struct LinTask {
    int64_t sb;
    int n;
    bool apply, update, causal, refresh;
};

struct LinIter {
    int64_t N, chunk, j, lo, hi, sb;
    int mode, tb, phase;
    bool done;
    const uint32_t* flags;
    __device__ void begin_chunk() {
        lo = j * chunk;
        hi = lo + chunk < N ? lo + chunk : N;
        sb = lo;
        phase = 0;
    }
    __device__ void init(int64_t N_, int chunk_, int mode_, int tb_, const uint32_t* flags_) {
        N = N_;
        mode = mode_;
        tb = tb_;
        flags = flags_;
        chunk = mode == TTT_MASK_TOKEN_CAUSAL ? tb : chunk_;
        j = 0;
        done = N <= 0;
        if (!done) begin_chunk();
    }
    __device__ bool updates(int64_t jj) const {
        return mode != TTT_MASK_STRIDED || ((flags[jj >> 5] >> (jj & 31)) & 1u);
    }
    __device__ LinTask cur() const {
        LinTask t;
        t.sb = sb;
        t.n = (int)(hi - sb < tb ? hi - sb : tb);
        const bool last = sb + tb >= hi;
        t.causal = false;
        if (mode == TTT_MASK_TOKEN_CAUSAL) {
            t.apply = t.update = t.causal = t.refresh = true;
        } else if (mode == TTT_MASK_APPLY_THEN_UPDATE || mode == TTT_MASK_STRIDED) {
            const bool u = updates(j);
            t.apply = true;
            t.update = u;
            t.refresh = u && last;
        } else {  // update then apply, and the one-chunk FULL mask
            t.apply = phase == 1;
            t.update = phase == 0;
            t.refresh = phase == 0 && last;
        }
        return t;
    }
    __device__ void next() {
        sb += tb;
        if (sb < hi) return;
        if ((mode == TTT_MASK_UPDATE_THEN_APPLY || mode == TTT_MASK_FULL) && phase == 0) {
            phase = 1;
            sb = lo;
            return;
        }
        ++j;
        if (j * chunk >= N) {
            done = true;
            return;
        }
        begin_chunk();
    }
};

// The next sub-block's q, k, v and eta, held in registers while the current one is computed.
template <typename T, int DK, bool CAUSAL, int VT_> struct LinStage {
    using C = LinCfg<T, DK, CAUSAL, VT_>;
    static constexpr int VEC = C::VEC, TB = C::TB, VT = C::VT;
    u32x4_t q[C::QPER];
    u32x4_t k[C::KPER][VEC];
    u32x4_t v[VEC];
    float e[VEC];

    __device__ __forceinline__ void load(const LinTask& t, const T* Q, const T* K, const T* V, int64_t dv,
                                         const float* eta) {
        const int tid = threadIdx.x;
        if (t.apply) {
#pragma unroll
            for (int i = 0; i < C::QPER; ++i) {
                const int idx = tid + i * kThreads;
                const int row = idx / (DK / VEC), c = idx % (DK / VEC);
                u32x4_t x = {0u, 0u, 0u, 0u};
                if ((C::QV % kThreads == 0 || idx < C::QV) && row < t.n)
                    x = *reinterpret_cast<const u32x4_t*>(Q + (t.sb + row) * DK + c * VEC);
                q[i] = x;
            }
        }
        if (t.update) {
#pragma unroll
            for (int i = 0; i < C::KPER; ++i) {
                const int u = tid + i * kThreads;
                const int tb = u % (TB / VEC), db = u / (TB / VEC);
#pragma unroll
                for (int r = 0; r < VEC; ++r) {
                    const int si = tb * VEC + r;
                    u32x4_t x = {0u, 0u, 0u, 0u};
                    if ((C::KU % kThreads == 0 || u < C::KU) && si < t.n)
                        x = *reinterpret_cast<const u32x4_t*>(K + (t.sb + si) * DK + db * VEC);
                    k[i][r] = x;
                }
            }
            if (tid < C::VU) {
                const int tb = tid % (TB / VEC), vb = tid / (TB / VEC);
#pragma unroll
                for (int r = 0; r < VEC; ++r) {
                    const int si = tb * VEC + r;
                    u32x4_t x = {0u, 0u, 0u, 0u};
                    float ev = 0.f;
                    if (si < t.n) {
                        x = *reinterpret_cast<const u32x4_t*>(V + (t.sb + si) * dv + vb * VEC);
                        ev = eta[t.sb + si];
                    }
                    v[r] = x;
                    e[r] = ev;
                }
            }
        }
    }

    // q rows into Qs; k transposed into Kt (feature rows, token columns) and, for the causal
    // intra-block term, as token rows into Ks; eta o v transposed into Vt
    __device__ __forceinline__ void store(const LinTask& t, char* smem) const {
        const int tid = threadIdx.x;
        if (t.apply) {
#pragma unroll
            for (int i = 0; i < C::QPER; ++i) {
                const int idx = tid + i * kThreads;
                if (C::QV % kThreads == 0 || idx < C::QV) {
                    const int row = idx / (DK / VEC), c = idx % (DK / VEC);
                    *reinterpret_cast<u32x4_t*>(smem + C::OFF_Q + row * C::PQ + c * 16) = q[i];
                }
            }
        }
        if (t.update) {
#pragma unroll
            for (int i = 0; i < C::KPER; ++i) {
                const int u = tid + i * kThreads;
                if (C::KU % kThreads == 0 || u < C::KU) {
                    const int tb = u % (TB / VEC), db = u / (TB / VEC);
                    u32x4_t tr[VEC];
                    Elt<T>::transpose(k[i], tr);
#pragma unroll
                    for (int r = 0; r < VEC; ++r)
                        *reinterpret_cast<u32x4_t*>(smem + C::OFF_KT + (db * VEC + r) * C::PT + tb * 16) = tr[r];
                    if constexpr (CAUSAL) {
#pragma unroll
                        for (int r = 0; r < VEC; ++r)
                            *reinterpret_cast<u32x4_t*>(smem + C::OFF_K + (tb * VEC + r) * C::PQ + db * 16) = k[i][r];
                    }
                }
            }
            if (tid < C::VU) {
                const int tb = tid % (TB / VEC), vb = tid / (TB / VEC);
                u32x4_t sc[VEC], tr[VEC];
#pragma unroll
                for (int r = 0; r < VEC; ++r) sc[r] = scale_vec(v[r], e[r], T{});
                Elt<T>::transpose(sc, tr);
#pragma unroll
                for (int r = 0; r < VEC; ++r)
                    *reinterpret_cast<u32x4_t*>(smem + C::OFF_VT + (vb * VEC + r) * C::PT + tb * 16) = tr[r];
            }
        }
    }
};

template <typename T, int DK, bool CAUSAL, int VT_>
__global__ __launch_bounds__(kThreads) void k_linattn(LinArgs<T> a) {
    using C = LinCfg<T, DK, CAUSAL, VT_>;
    constexpr int ES = C::ES, TB = C::TB, VT = C::VT, PQ = C::PQ, PT = C::PT;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    char* Qs = smem + C::OFF_Q;
    char* Kt = smem + C::OFF_KT;
    char* Vt = smem + C::OFF_VT;
    char* Sh = smem + C::OFF_SH;
    char* Sl = smem + C::OFF_SL;
    char* Ks = smem + C::OFF_K;
    char* Ps = smem + C::OFF_P;

    const int lb = xcd_block(gridDim.x);
    const int scan = lb / a.nvt, v0 = (lb % a.nvt) * VT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t N = a.N;
    const T* Q = a.q + (int64_t)scan * N * DK;
    const T* K = a.k + (int64_t)scan * N * DK;
    const T* V = a.v + (int64_t)scan * N * a.dv + v0;
    const float* eta = a.eta + (int64_t)scan * N;
    T* O = a.o + (int64_t)scan * N * a.dv + v0;

    // state slice: wave (wv, wk) holds rows [16 wv, +16) x cols [wk DK/WSK, +DK/WSK)
    const int wv = wave / C::WSK, wk = wave % C::WSK;
    f32x4_t sacc[1][C::SFN];
#pragma unroll
    for (int j = 0; j < C::SFN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int vv = 16 * wv + 4 * (lane >> 4) + r, kk = wk * (DK / C::WSK) + j * 16 + (lane & 15);
            sacc[0][j][r] = a.S0 ? a.S0[((int64_t)scan * a.dv + v0 + vv) * DK + kk] : 0.f;
        }
    auto refresh = [&]() {
#pragma unroll
        for (int j = 0; j < C::SFN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int vv = 16 * wv + 4 * (lane >> 4) + r, kk = wk * (DK / C::WSK) + j * 16 + (lane & 15);
                const float x = sacc[0][j][r];
                if constexpr (ES == 2) {
                    const uint16_t hi = f2bf(x);
                    *reinterpret_cast<uint16_t*>(Sh + vv * PQ + kk * 2) = hi;
                    *reinterpret_cast<uint16_t*>(Sl + vv * PQ + kk * 2) = f2bf(x - bf2f(hi));
                } else {
                    *reinterpret_cast<float*>(Sh + vv * PQ + kk * 4) = x;
                }
            }
    };
    refresh();

    const int at0 = (wave / C::AWN) * 16;
    const int av0 = (wave % C::AWN) * (VT / C::AWN);
    const int pc0 = (wave % C::AWN) * (TB / C::AWN);

    auto apply = [&](const LinTask& t) {
        f32x4_t oacc[1][C::AFN];
#pragma unroll
        for (int j = 0; j < C::AFN; ++j) oacc[0][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lds_mma<T, 1, C::AFN>(oacc, Qs, PQ, at0, Sh, PQ, av0, DK * ES);
        if constexpr (ES == 2) lds_mma<T, 1, C::AFN>(oacc, Qs, PQ, at0, Sl, PQ, av0, DK * ES);
        if constexpr (CAUSAL) {
            f32x4_t pacc[1][C::PFN];
#pragma unroll
            for (int j = 0; j < C::PFN; ++j) pacc[0][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            lds_mma<T, 1, C::PFN>(pacc, Qs, PQ, at0, Ks, PQ, pc0, DK * ES);
#pragma unroll
            for (int j = 0; j < C::PFN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tt = at0 + 4 * (lane >> 4) + r, ss = pc0 + j * 16 + (lane & 15);
                    const float val = (ss <= tt && ss < t.n) ? pacc[0][j][r] : 0.f;
                    *reinterpret_cast<T*>(Ps + tt * PT + ss * ES) = Elt<T>::st(val);
                }
            lds_barrier();
            lds_mma<T, 1, C::AFN>(oacc, Ps, PT, at0, Vt, PT, av0, TB * ES);
        }
#pragma unroll
        for (int j = 0; j < C::AFN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = at0 + 4 * (lane >> 4) + r, vv = av0 + j * 16 + (lane & 15);
                if (tt < t.n) O[(t.sb + tt) * a.dv + vv] = Elt<T>::st(oacc[0][j][r]);
            }
    };

    LinIter it;
    it.init(N, a.chunk, a.mode, TB, a.flags);
    LinStage<T, DK, CAUSAL, VT_> g;
    LinTask cur{};
    if (!it.done) {
        cur = it.cur();
        g.load(cur, Q, K, V, a.dv, eta);
    }
    lds_barrier();  // S is in LDS
    while (!it.done) {
        g.store(cur, smem);
        lds_barrier();
        it.next();
        LinTask nxt{};
        if (!it.done) {  // the next sub-block's loads are in flight while this one is computed
            nxt = it.cur();
            g.load(nxt, Q, K, V, a.dv, eta);
        }
        if (cur.apply) apply(cur);
        if (cur.update) lds_mma<T, 1, C::SFN>(sacc, Vt, PT, 16 * wv, Kt, PT, wk * (DK / C::WSK), TB * ES);
        if (cur.refresh) {
            lds_barrier();  // every wave is done reading S for this sub-block
            refresh();
        }
        lds_barrier();
        cur = nxt;
    }
    if (a.Sout) {
#pragma unroll
        for (int j = 0; j < C::SFN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int vv = 16 * wv + 4 * (lane >> 4) + r, kk = wk * (DK / C::WSK) + j * 16 + (lane & 15);
                a.Sout[((int64_t)scan * a.dv + v0 + vv) * DK + kk] = sacc[0][j][r];
            }
    }
}

static ttt_status validate_lin(const linattn_desc* D) {
    if (!D) return fail(TTT_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (D->B < 0 || D->H < 0 || D->N < 0) return fail(TTT_ERR_INVALID_ARGUMENT, "B, H, N must be >= 0");
    if (D->d_k < 32 || D->d_k > 256 || D->d_k % 32)
        return fail(TTT_ERR_INVALID_ARGUMENT, "d_k=%d must be a multiple of 32 in [32, 256]", D->d_k);
    if (D->d_v < 32 || D->d_v > 4096 || D->d_v % 32)
        return fail(TTT_ERR_INVALID_ARGUMENT, "d_v=%d must be a multiple of 32 in [32, 4096]", D->d_v);
    if (D->chunk < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "chunk must be >= 1");
    if (D->io_dtype != TTT_F32 && D->io_dtype != TTT_BF16) return fail(TTT_ERR_INVALID_ARGUMENT, "bad io_dtype");
    if (D->mask < TTT_MASK_FULL || D->mask > TTT_MASK_TOKEN_CAUSAL) return fail(TTT_ERR_INVALID_ARGUMENT, "bad mask");
    if (D->mask == TTT_MASK_FULL && D->chunk < D->N)
        return fail(TTT_ERR_INVALID_ARGUMENT, "MASK_FULL needs chunk >= N (one chunk)");
    if (D->mask == TTT_MASK_STRIDED) {
        if (!D->update_chunks && D->N > 0) return fail(TTT_ERR_INVALID_ARGUMENT, "MASK_STRIDED needs update_chunks");
        if (cdiv(D->N, D->chunk) > 32 * 32)
            return fail(TTT_ERR_UNSUPPORTED, "MASK_STRIDED supports at most 1024 chunks");
    }
    if ((int64_t)D->B * D->H > (1 << 20)) return fail(TTT_ERR_INVALID_ARGUMENT, "B*H too large");
    return TTT_OK;
}

template <typename T, int DK>
static ttt_status launch_lin(LinArgs<T>& a, int grid, hipStream_t st) {
    {
        ProfScope ps(PK_LINATTN, st);
        if (a.vt == 16) {
            if constexpr (sizeof(T) == 2 && DK % 64 == 0) {
                if (a.mode == TTT_MASK_TOKEN_CAUSAL)
                    hipLaunchKernelGGL((k_linattn<T, DK, true, 16>), dim3(grid), dim3(kThreads), 0, st, a);
                else
                    hipLaunchKernelGGL((k_linattn<T, DK, false, 16>), dim3(grid), dim3(kThreads), 0, st, a);
            }
        } else if (a.mode == TTT_MASK_TOKEN_CAUSAL) {
            hipLaunchKernelGGL((k_linattn<T, DK, true, 32>), dim3(grid), dim3(kThreads), 0, st, a);
        } else {
            hipLaunchKernelGGL((k_linattn<T, DK, false, 32>), dim3(grid), dim3(kThreads), 0, st, a);
        }
    }
    return check_launch("k_linattn");
}

template <typename T>
static ttt_status run_lin(const linattn_desc& D, LinArgs<T>& a, hipStream_t st) {
    const int grid = D.B * D.H * a.nvt;
    switch (D.d_k) {
        case 32: return launch_lin<T, 32>(a, grid, st);
        case 64: return launch_lin<T, 64>(a, grid, st);
        case 96: return launch_lin<T, 96>(a, grid, st);
        case 128: return launch_lin<T, 128>(a, grid, st);
        case 160: return launch_lin<T, 160>(a, grid, st);
        case 192: return launch_lin<T, 192>(a, grid, st);
        case 224: return launch_lin<T, 224>(a, grid, st);
        case 256: return launch_lin<T, 256>(a, grid, st);
    }
    return fail(TTT_ERR_UNSUPPORTED, "d_k=%d", D.d_k);
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status linattn_workspace_bytes(const linattn_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_lin(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = 0;
    return TTT_OK;
}

extern "C" ttt_status linattn_forward(const linattn_desc* desc, const void* q, const void* k, const void* v,
                                      const float* eta, const float* S0, void* o, float* S_out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    clear_error();
    ttt_status rc = validate_lin(desc);
    if (rc != TTT_OK) return rc;
    const linattn_desc& D = *desc;
    const int64_t S = (int64_t)D.B * D.H;
    if (S == 0) return TTT_OK;
    if (D.N > 0 && (!q || !k || !v || !eta || !o))
        return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, eta and o are required");
    const void* p16[] = {q, k, v, o};
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, o must be 16-byte aligned");
    if ((eta && !aligned(eta, 4)) || (S0 && !aligned(S0, 4)) || (S_out && !aligned(S_out, 4)))
        return fail(TTT_ERR_INVALID_ARGUMENT, "eta, S0, S_out must be 4-byte aligned");
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const size_t qb = (size_t)S * D.N * D.d_k * es, vb = (size_t)S * D.N * D.d_v * es;
    if (overlaps(o, vb, q, qb) || overlaps(o, vb, k, qb) || overlaps(o, vb, v, vb) ||
        overlaps(o, vb, eta, (size_t)S * D.N * 4))
        return fail(TTT_ERR_INVALID_ARGUMENT, "o overlaps an input");
    const size_t sb = (size_t)S * D.d_v * D.d_k * 4;
    if (overlaps(S_out, sb, S0, sb)) return fail(TTT_ERR_INVALID_ARGUMENT, "S_out overlaps S0");
    hipStream_t st = (hipStream_t)stream;
    // 32-row slices of S: measured faster than 16-row slices, whose extra workgroups double the
    // re-reads of q and k (the 16-row instantiation is kept for the bf16 kernel)
    const int vt = 32;
    const int nvt = D.d_v / vt;
    if (D.io_dtype == TTT_BF16) {
        LinArgs<uint16_t> a{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta, S0, (uint16_t*)o, S_out,
                            D.N, D.d_v, D.chunk, D.mask, nvt, vt, {}};
        if (D.mask == TTT_MASK_STRIDED)
            for (int64_t j = 0; j < cdiv(D.N, D.chunk); ++j)
                if (D.update_chunks[j]) a.flags[j >> 5] |= 1u << (j & 31);
        return run_lin<uint16_t>(D, a, st);
    }
    LinArgs<float> a{(const float*)q, (const float*)k, (const float*)v, eta, S0, (float*)o, S_out, D.N, D.d_v,
                     D.chunk, D.mask, nvt, vt, {}};
    if (D.mask == TTT_MASK_STRIDED)
        for (int64_t j = 0; j < cdiv(D.N, D.chunk); ++j)
            if (D.update_chunks[j]) a.flags[j >> 5] |= 1u << (j & 31);
    return run_lin<float>(D, a, st);
}
