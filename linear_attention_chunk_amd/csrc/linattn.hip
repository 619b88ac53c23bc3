// Chunked linear attention on gfx950: the linear, bias-free fast weight S (d_v x d_k) under plain GD
// with the dot-product loss, S <- S + sum_i eta_i v_i k_i^T, o = S q ("Test-Time Training with KV
// Binding Is Secretly Linear Attention", Thm. 5.2 and Sec. 6.1 Step 6), with the chunk orders of
// the PaperTrace notes' section 1.1 and the token-causal limit ("From Linear Attention to Test-Time
// Training", causal linear attention).
//
// Two paths.  The chunk-parallel path (large chunks; token-causal mode over 128-token blocks) runs
// three launches: the chunk's own update dS_c = sum over the chunk of eta_i v_i k_i^T for every
// (scan, chunk) in parallel, an elementwise scan over chunks that writes the state each chunk's
// queries see (before or after its own update, as the mask orders them), and the apply
// o = S_c q for every chunk in parallel, plus the block's own masked term in token-causal mode.
// The sequential path below handles small chunks, where the chunk states would cost more traffic
// than they save, and short token-causal sequences.
//
// Sequential path: one workgroup owns one (batch, head) scan and a 32-row slice of S's d_v rows,
// and walks the sequence in sub-blocks of TB tokens.  The slice of S stays in MFMA accumulators (fp32) for the
// whole sequence; the update is an MFMA accumulation over the sub-block's tokens.  The apply reads
// S from LDS, where it is kept as a bf16 hi + lo pair (fp32 in fp32 mode) refreshed at chunk ends,
// so the query products see S to about 16 bits.  Token-causal mode adds the masked intra-block term
// tril(Q K^T) (eta o V) and refreshes S after every sub-block.  The next sub-block's q, k, v and eta
// are loaded into registers while the current one is computed.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

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
    const float* S0 = a.S0;
    float* Sout = a.Sout ? a.Sout + (int64_t)scan * a.dv * DK : nullptr;

    // state slice: wave (wv, wk) holds rows [16 wv, +16) x cols [wk DK/WSK, +DK/WSK)
    const int wv = wave / C::WSK, wk = wave % C::WSK;
    f32x4_t sacc[1][C::SFN];
#pragma unroll
    for (int j = 0; j < C::SFN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int vv = 16 * wv + 4 * (lane >> 4) + r, kk = wk * (DK / C::WSK) + j * 16 + (lane & 15);
            sacc[0][j][r] = S0 ? S0[((int64_t)scan * a.dv + v0 + vv) * DK + kk] : 0.f;
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
    if (Sout) {
#pragma unroll
        for (int j = 0; j < C::SFN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int vv = 16 * wv + 4 * (lane >> 4) + r, kk = wk * (DK / C::WSK) + j * 16 + (lane & 15);
                Sout[(int64_t)(v0 + vv) * DK + kk] = sacc[0][j][r];
            }
    }
}

// ---------------------------------------------------------------------------------------------
// chunk-parallel path: scan over chunks and apply

// dS_c = sum over chunk c's tokens of eta_i v_i k_i^T (d_v x d_k, fp32), contracting over tokens:
// both operands are token-major, so both go through the transposing stager, which also applies
// eta to v (without SCALE the weights are 1 and eta is not read: the backward's sum of dO q^T).
// Chunks a strided mask does not update are skipped (and never read).
template <typename T> struct DeltaArgs {
    const T* k; const T* v; const float* eta; float* dS;
    int64_t N; int dk, dv, chunk, nc, ntv, ntk, mode;
    uint32_t flags[32];
};

constexpr int kDeltaRows = 128, kDeltaCols = 128;

template <typename T, bool SCALE = true>
__global__ __launch_bounds__(kThreads, 3) void k_lin_delta(DeltaArgs<T> a) {
    using TD = Tile<T, kDeltaRows, kDeltaCols, 2, 2, 1, 1, 1, true, true, SCALE, 4, 1>;  // one LDS stage, three per CU
    __shared__ __attribute__((aligned(16))) char smem[TD::LDS];
    const int lb = xcd_block(gridDim.x);
    const int per = a.ntv * a.ntk;
    const int unit = lb / per, t = lb % per;
    const int scan = unit / a.nc, c = unit % a.nc;
    if (a.mode == TTT_MASK_STRIDED && !((a.flags[c >> 5] >> (c & 31)) & 1u)) return;
    const int r0 = (t / a.ntk) * kDeltaRows, c0 = (t % a.ntk) * kDeltaCols;
    const int64_t tok = (int64_t)scan * a.N + (int64_t)c * a.chunk;
    const int nl = (int)std::min<int64_t>(a.chunk, a.N - (int64_t)c * a.chunk);
    Opnd<T> A[1] = {{a.v + tok * a.dv + r0, a.dv, a.dv - r0, nl}};
    if constexpr (SCALE) A[0].kscale = a.eta + tok;
    const Opnd<T> B[1] = {{a.k + tok * a.dk + c0, a.dk, a.dk - c0, nl}};
    TD tl;
    tl.template run<PM1>(A, B, nl, smem);
    // 32-bit offsets from the tile corner
    float* dS = a.dS + (int64_t)unit * a.dv * a.dk + (int64_t)r0 * a.dk + c0;
    if (r0 + TD::BM <= a.dv && c0 + TD::BN <= a.dk) {
        // full tiles: both operands' staging permutes rows and columns, so rows are gathered in
        // LDS and leave as whole 512-byte row segments
        static_assert(TD::RV_LDS <= TD::LDS, "row bands fit the tile's LDS");
        tl.rows_via_lds(smem, [&](int, int, int row, int col, const float4& v) {
            *reinterpret_cast<float4*>(dS + (uint32_t)row * (uint32_t)a.dk + (uint32_t)col) = v;
        });
    } else {
        tl.for_each([&](const float (&v)[1], int row, int col) {
            if (r0 + row < a.dv && c0 + col < a.dk) dS[(uint32_t)row * (uint32_t)a.dk + (uint32_t)col] = v[0];
        });
    }
}

// The state each chunk's queries see, from S0 and the chunk updates dS_c: before chunk c's own
// update (apply-then-update, strided) or after it (update-then-apply, full).  One thread owns 4
// consecutive elements of one scan's state and walks the chunks in fp32, writing each chunk's state
// as `planes` io-dtype planes (bf16: hi, or hi and lo = bf16(x - hi)).  The entry/exit strides,
// the momentum term, the repeats and the sign are those of LinStateIO.  With rev the chunks are
// walked from the last to the first (the backward's suffix sums of the chunks' query gradients:
// there "before its own update" means without the chunk's own term).
template <typename T> struct ScanArgs {
    const float* dS; T* Sc;
    LinStateIO io;
    int64_t dvk;   // d_v * d_k
    int nc, mode, nscan, rev;
    int planes;    // bf16: 2 (hi + lo) or 1 (the state rounded once); fp32: 1
    uint32_t flags[32];
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_lin_scan(ScanArgs<T> a) {
    constexpr int PLANES = sizeof(T) == 2 ? 2 : 1;
    const int64_t per = a.dvk / 4;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= per * a.nscan) return;
    const int64_t scan = g / per, e = (g % per) * 4;
    const LinStateIO& io = a.io;
    f32x4_t st = {0.f, 0.f, 0.f, 0.f}, mom = {0.f, 0.f, 0.f, 0.f};
    if (io.S0) {  // S0, S_out and the momentum are only 4-byte aligned
        const float* s0 = io.S0 + (io.s0_heads ? scan % io.s0_heads : scan) * io.s0_stride + e;
#pragma unroll
        for (int u = 0; u < 4; ++u) st[u] = s0[u];
    }
    if (io.M0)
#pragma unroll
        for (int u = 0; u < 4; ++u) mom[u] = io.msign * io.M0[scan * io.m_stride + e + u];
    const bool post = a.mode == TTT_MASK_UPDATE_THEN_APPLY || a.mode == TTT_MASK_FULL;
    auto put = [&](int c, const f32x4_t& x) {
        T* dst = a.Sc + ((scan * a.nc + c) * a.planes) * a.dvk + e;
        if (PLANES == 2 && a.planes == 2) {
            float lo[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) lo[u] = x[u] - bf2f(f2bf(x[u]));
            Pack4<T>::store(dst, x[0], x[1], x[2], x[3]);
            Pack4<T>::store(dst + a.dvk, lo[0], lo[1], lo[2], lo[3]);
        } else {
            Pack4<T>::store(dst, x[0], x[1], x[2], x[3]);
        }
    };
    if (a.rev && io.mom) {
        // The momentum recurrence transposed, from the last chunk: st is the gradient of the state,
        // mom that of the running term m (zero at the end: the final momentum is not in the loss).
        // Every chunk's D_c adds to st (before its own update's transpose where the chunk's queries
        // see its update, after it otherwise); each step of an updating chunk gives g = mom + st to
        // the chunk's update and sets mom <- beta g.  The chunk's slot receives the sum of its g.
        for (int i = 0; i < a.nc; ++i) {
            const int c = a.nc - 1 - i;
            const bool upd = a.mode != TTT_MASK_STRIDED || ((a.flags[c >> 5] >> (c & 31)) & 1u);
            const f32x4_t d = *reinterpret_cast<const f32x4_t*>(a.dS + (scan * a.nc + c) * a.dvk + e);
            if (post) st += d;
            if (upd) {
                f32x4_t r = {0.f, 0.f, 0.f, 0.f};
                for (int k = 0; k < io.reps; ++k) {
                    const f32x4_t gsum = mom + st;
                    r += gsum;
                    mom = io.beta * gsum;
                }
                put(c, r);
            }
            if (!post) st += d;
        }
        if (io.Sout)
#pragma unroll
            for (int u = 0; u < 4; ++u) io.Sout[scan * io.sout_stride + e + u] = st[u];
        return;
    }
    for (int i = 0; i < a.nc; ++i) {
        const int c = a.rev ? a.nc - 1 - i : i;
        const bool upd = a.mode != TTT_MASK_STRIDED || ((a.flags[c >> 5] >> (c & 31)) & 1u);
        if (!post) put(c, st);
        if (upd) {
            const f32x4_t d = io.dsign * *reinterpret_cast<const f32x4_t*>(a.dS + (scan * a.nc + c) * a.dvk + e);
            for (int r = 0; r < io.reps; ++r) {
                if (io.mom) {
                    mom = io.beta * mom + d;
                    st += mom;
                } else {
                    st += d;
                }
            }
        }
        if (post) put(c, st);
    }
    if (io.Sout)
#pragma unroll
        for (int u = 0; u < 4; ++u) io.Sout[scan * io.sout_stride + e + u] = st[u];
    if (io.Mout)
#pragma unroll
        for (int u = 0; u < 4; ++u) io.Mout[scan * io.m_stride + e + u] = io.msign * mom[u];
}

// The chunk-parallel path keeps the states in fp32 through the scans and hands them to the products
// as one io-dtype plane (bf16: the state rounded once, as the products' other operands are).
constexpr int kStatePlanes = 1;

// The chunk updates and the scan in one pass (when no step runs between them).  A workgroup owns a
// 64 x 64 tile of one scan's state, kept in registers in fp32 in the accumulator layout, and walks
// the chunks in order: each chunk's update of its tile is the delta kernel's eta-weighted product
// over the chunk's tokens (MFMA, accumulators zeroed per chunk), added to the state with the scan's
// momentum, repeats and sign.  The loads run as one pipeline over the whole sequence: a stage is a
// whole 256-token (fp32: 128-token) slice of v and k, and the next stage, which may belong to the
// next updating chunk, is in flight while the current one is in the MFMAs, so that at one
// workgroup per CU a stage's memory latency hides behind the previous stage.  The state each
// chunk's queries see leaves straight from the accumulator layout as one io-dtype plane; S_out and
// the momentum leave as the scan writes them.  dS never reaches memory.  Chunks of half a stage
// (128 tokens in bf16, token-causal mode's blocks) go two to a stage (PAIR): the stage's first
// half of k windows forms one chunk's update, the second half the next chunk's, each in
// accumulators of its own.
constexpr int kDscanTile = 64, kDscanSeg = 8;
template <typename T> struct DscanArgs {
    const T* k; const T* v; const float* eta; T* Sc;
    LinStateIO io;
    int64_t N; int dk, dv, chunk, nc, mode, ntv, ntk;
    uint32_t flags[32];
};
template <typename T>
using DscanTile = Tile<T, kDscanTile, kDscanTile, kDscanSeg, 2, 1, 1, 1, true, true, true, 4, 1>;

template <typename T, bool FULL, bool PAIR>
__global__ __launch_bounds__(kThreads, 1) void k_lin_dscan(DscanArgs<T> a) {
    using TD = DscanTile<T>;
    constexpr int TS = kDscanTile, E = TD::ELEMS, KS = TD::KSTEP;
    constexpr int HW = kDscanSeg;  // k windows in half a stage
    __shared__ __attribute__((aligned(16))) char smem[TD::LDS];
    const int per = a.ntv * a.ntk;
    const int lb = xcd_block(gridDim.x);
    const int scan = lb / per, t = lb % per;
    const int r0 = (t / a.ntk) * TS, c0 = (t % a.ntk) * TS;
    const LinStateIO& io = a.io;
    const bool post = a.mode == TTT_MASK_UPDATE_THEN_APPLY || a.mode == TTT_MASK_FULL;
    const int64_t dvk = (int64_t)a.dv * a.dk;
    auto updates = [&](int c) { return a.mode != TTT_MASK_STRIDED || ((a.flags[c >> 5] >> (c & 31)) & 1u); };
    auto tokens = [&](int c) { return (int)std::min<int64_t>(a.chunk, a.N - (int64_t)c * a.chunk); };
    auto next_upd = [&](int c) {
        while (c < a.nc && !updates(c)) ++c;
        return c;
    };
    // stage s of chunk c: the chunk's v and k slices from token s * KSTEP on (PAIR: chunks c and
    // c + 1, c even, in one stage)
    auto issue = [&](typename TD::Regs& g, int c, int s) {
        const int64_t tok = (int64_t)scan * a.N + (int64_t)c * a.chunk;
        const int nl = PAIR ? (int)std::min<int64_t>(2 * a.chunk, a.N - (int64_t)c * a.chunk) : tokens(c);
        Opnd<T> A[1] = {{a.v + tok * a.dv + r0, a.dv, a.dv - r0, nl}};
        A[0].kscale = a.eta + tok;
        const Opnd<T> B[1] = {{a.k + tok * a.dk + c0, a.dk, a.dk - c0, nl}};
        TD::template issue<FULL>(g, A, B, s * KS);
    };
    float st[E], mm[E];
    TD::for_each_pos([&](int idx, int row, int col) {
        const bool in = FULL || (r0 + row < a.dv && c0 + col < a.dk);
        const int64_t e = (int64_t)(r0 + row) * a.dk + c0 + col;
        st[idx] = (io.S0 && in) ? io.S0[(io.s0_heads ? scan % io.s0_heads : scan) * io.s0_stride + e] : 0.f;
        mm[idx] = (io.M0 && in) ? io.msign * io.M0[(int64_t)scan * io.m_stride + e] : 0.f;
    });
    auto put = [&](int c) {  // the state chunk c's queries see
        T* dst = a.Sc + ((int64_t)scan * a.nc + c) * dvk;
        TD::for_each_pos([&](int idx, int row, int col) {
            if (FULL || (r0 + row < a.dv && c0 + col < a.dk))
                dst[(int64_t)(r0 + row) * a.dk + c0 + col] = Elt<T>::st(st[idx]);
        });
    };
    auto add = [&](const TD& tl) {  // a chunk's update into the state
        TD::for_each_pos([&](int idx, int, int) {
            const int i = idx / (TD::FN * 16), j = (idx / 16) % TD::FN, r = idx % 16;
            const float d = io.dsign * tl.acc[0][i][j][r];
            for (int k = 0; k < io.reps; ++k) {
                if (io.mom) {
                    mm[idx] = io.beta * mm[idx] + d;
                    st[idx] += mm[idx];
                } else {
                    st[idx] += d;
                }
            }
        });
    };
    TD tl;
    typename TD::Regs g;
    if constexpr (PAIR) {
        // one stage per pair of chunks; a pair neither of whose chunks updates is not loaded
        auto pair_upd = [&](int c) { return c < a.nc && (updates(c) || (c + 1 < a.nc && updates(c + 1))); };
        auto next_pair = [&](int c) {
            while (c < a.nc && !pair_upd(c)) c += 2;
            return c;
        };
        TD tl2;
        int ic = next_pair(0);
        if (ic < a.nc) issue(g, ic, 0);
        for (int c = 0; c < a.nc; c += 2) {
            if (c == ic) {
                tl.zero();
                tl2.zero();
                lds_barrier();  // every wave is done with the previous stage
                TD::template put<FULL>(g, smem);
                ic = next_pair(c + 2);
                if (ic < a.nc) issue(g, ic, 0);
                lds_barrier();
                tl.template compute_win<PM1, 0, HW>(smem);
                tl2.template compute_win<PM1, HW, 2 * HW>(smem);
            }
            for (int j = 0; j < 2 && c + j < a.nc; ++j) {
                if (!post) put(c + j);
                if (updates(c + j)) add(j ? tl2 : tl);
                if (post) put(c + j);
            }
        }
    } else {
    int ic = next_upd(0), is = 0;  // the stage in flight in g
    if (ic < a.nc) issue(g, ic, 0);
    for (int c = 0; c < a.nc; ++c) {
        if (!post) put(c);
        if (c == ic) {  // an updating chunk: its stages are the ones in flight
            tl.zero();
            const int ns = (tokens(c) + KS - 1) / KS;
            for (int s = 0; s < ns; ++s) {
                lds_barrier();  // every wave is done with the previous stage
                TD::template put<FULL>(g, smem);
                if (s + 1 < ns) {
                    is = s + 1;
                } else {
                    ic = next_upd(c + 1);
                    is = 0;
                }
                if (ic < a.nc) issue(g, ic, is);
                lds_barrier();
                tl.template compute<PM1>(smem);
            }
            add(tl);
        }
        if (post) put(c);
    }
    }
    TD::for_each_pos([&](int idx, int row, int col) {
        if (FULL || (r0 + row < a.dv && c0 + col < a.dk)) {
            const int64_t e = (int64_t)(r0 + row) * a.dk + c0 + col;
            if (io.Sout) io.Sout[(int64_t)scan * io.sout_stride + e] = st[idx];
            if (io.Mout) io.Mout[(int64_t)scan * io.m_stride + e] = io.msign * mm[idx];
        }
    });
}

// o (chunk c's tokens x d_v) = q_c S_c^T, contracting over d_k
template <typename T> struct ApplyArgs {
    const T* q; const T* Sc; T* o;
    const T* k; const T* v; const float* eta;  // token-causal apply only
    int64_t N; int dk, dv, chunk, nc, ntt, ntv, nscan;
};

constexpr int kApplyRows = 128, kApplyCols = 128;

template <typename T>
__global__ __launch_bounds__(kThreads, 3) void k_lin_apply(ApplyArgs<T> a) {
    constexpr int PLANES = kStatePlanes;
    // 64-wide k-steps in one LDS stage (37 KB), three workgroups per CU
    using TA = Tile<T, kApplyRows, kApplyCols, 2, 2, 1, PLANES, PLANES, false, false, false, 4, 1>;
    using PM = typename std::conditional<PLANES == 2, PMQ, PM1>::type;
    __shared__ __attribute__((aligned(16))) char smem[TA::LDS];
    const int lb = xcd_block(gridDim.x);
    const int per_chunk = a.ntt * a.ntv;
    const int unit = lb / per_chunk, t = lb % per_chunk;
    const int scan = unit / a.nc, c = unit % a.nc;
    const int r0 = (t / a.ntv) * kApplyRows, c0 = (t % a.ntv) * kApplyCols;
    const int64_t tok = (int64_t)scan * a.N + (int64_t)c * a.chunk;
    const int nl = (int)std::min<int64_t>(a.chunk, a.N - (int64_t)c * a.chunk);
    if (r0 >= nl) return;  // a ragged last chunk has fewer token tiles (uniform per workgroup)
    const int64_t dvk = (int64_t)a.dv * a.dk;
    const T* S = a.Sc + (int64_t)unit * PLANES * dvk + (int64_t)c0 * a.dk;
    const Opnd<T> A[1] = {{a.q + (tok + r0) * a.dk, a.dk, nl - r0, a.dk}};
    Opnd<T> B[PLANES];
#pragma unroll
    for (int p = 0; p < PLANES; ++p) B[p] = Opnd<T>{S + p * dvk, a.dk, a.dv - c0, a.dk};
    TA tl;
    tl.template run<PM>(A, B, a.dk, smem);
    T* O = a.o + (tok + r0) * a.dv + c0;
    auto epi = [&](auto check) {
        tl.for_each([&](const float (&v)[PLANES], int row, int col) {
            if (!decltype(check)::value || (r0 + row < nl && c0 + col < a.dv)) {
                float x = v[0];
                if constexpr (PLANES == 2) x += v[1];
                O[(uint32_t)row * (uint32_t)a.dv + (uint32_t)col] = Elt<T>::st(x);
            }
        });
    };
    if (r0 + TA::BM <= nl && c0 + TA::BN <= a.dv) epi(std::false_type{});
    else epi(std::true_type{});
}

// Token-causal mode on the chunk-parallel path.  The sequence is cut into blocks of kCausalBlock
// tokens; the delta and scan kernels give every block the state S_c before it (apply-then-update
// order), and this kernel adds the block's own causal term.  For query token i of the block
//   o_i = S_c q_i + sum over the block's tokens j <= i of eta_j (k_j . q_i) v_j,
// that is o = q S_c^T + tril(q k^T) diag(eta) v.  One workgroup takes 64 query rows of a block and
// 128 columns of d_v (the two row halves of a block are neighbours, so k, v and S_c come from the
// same L2).  q k^T and q S_c^T are one contraction over d_k with two accumulators (q staged once).
// The masked, eta-scaled q k^T rows are rounded to the io dtype straight into the A regions of the
// LDS stages of the P v product (v through the transposing stager), as the sequential kernel rounds
// them; the first half's rows see only the block's first 64 keys, so its P v stops there.  P v is
// added to q S_c^T through an fp32 LDS buffer, because the transposing stager leaves P v in another
// column order.
constexpr int kCausalBlock = 128, kCausalRows = 64;

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_lin_apply_causal(ApplyArgs<T> a) {
    static_assert(kStatePlanes == 1, "q S_c^T is one accumulator");
    using TQ = Tile<T, kCausalRows, kCausalBlock, 2, 2, 1, 2, 2, false, false, false, 4, 1>;  // q k^T, q S_c^T
    using TD = Tile<T, kCausalRows, kApplyCols, 2, 2, 1, 1, 1, false, true>;     // P v, P in LDS
    constexpr int NST = kCausalBlock / TD::KSTEP;  // key-token stages of P v, all resident
    constexpr int OP = kApplyCols + 4;             // fp32 combine-buffer pitch (floats)
    constexpr int LDSB = std::max(std::max(TQ::LDS, NST * TD::STAGE), kCausalRows * OP * 4);
    static_assert(kCausalBlock % TD::KSTEP == 0 && kCausalBlock == 2 * kCausalRows && kApplyCols == kCausalBlock,
                  "block and tile shapes");
    __shared__ __attribute__((aligned(16))) char smem[LDSB];
    const int lb = xcd_block(gridDim.x);
    const int unit = lb / (2 * a.ntv), cv = (lb / 2) % a.ntv, h = lb % 2;
    const int scan = unit / a.nc, c = unit % a.nc;
    const int c0 = cv * kApplyCols, r0 = h * kCausalRows;
    const int64_t tok = (int64_t)scan * a.N + (int64_t)c * kCausalBlock;
    const int nl = (int)std::min<int64_t>(kCausalBlock, a.N - (int64_t)c * kCausalBlock);
    const int nr = nl - r0;  // query rows of this workgroup
    if (nr <= 0) return;     // a ragged last block without a second half
    const int nst = h ? NST : NST / 2;  // the key stages these rows see

    // v's stages are loaded first, so they are in flight during the first contraction
    const Opnd<T> Bv = {a.v + tok * a.dv + c0, a.dv, a.dv - c0, nl};  // rows: d_v columns; k: tokens
    const bool vfull = a.dv - c0 >= kApplyCols && nl == kCausalBlock;
    typename TD::SB gv[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        if (st >= nst) break;
        if (vfull) gv[st].template load<true>(Bv, st * TD::KSTEP);
        else gv[st].template load<false>(Bv, st * TD::KSTEP);
    }
    // eta of the key tokens this lane's P columns belong to (clamped to the block; masked later)
    float ek[TQ::FN];
    TQ::for_each_pos([&](int idx, int, int col) {
        if (idx < TQ::FN * 16 && idx % 16 == 0) ek[idx / 16] = a.eta[tok + std::min(col, nl - 1)];
    });

    // P = q k^T over the block (rows: query tokens, columns: key tokens) and q S_c^T (columns: d_v)
    const int64_t dvk = (int64_t)a.dv * a.dk;
    const Opnd<T> Aq[1] = {{a.q + (tok + r0) * a.dk, a.dk, nr, a.dk}};
    const Opnd<T> Bks[2] = {{a.k + tok * a.dk, a.dk, nl, a.dk},
                            {a.Sc + (int64_t)unit * dvk + (int64_t)c0 * a.dk, a.dk, a.dv - c0, a.dk}};
    TQ tq;
    tq.template run<PMQ>(Aq, Bks, a.dk, smem);
    lds_barrier();  // every wave is done with the contraction's stages
    {
        int idx = 0;
        tq.for_each([&](const float (&v)[2], int row, int col) {
            const float val = (col <= r0 + row && col < nl) ? v[0] * ek[(idx / 16) % TQ::FN] : 0.f;
            ++idx;
            if (col < nst * TD::KSTEP)
                *reinterpret_cast<T*>(smem + (col / TD::KSTEP) * TD::STAGE + row * TD::PITCH +
                                      (col % TD::KSTEP) * (int)sizeof(T)) = Elt<T>::st(val);
        });
    }
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        if (st >= nst) break;
        if (vfull) gv[st].template store<true>(smem + st * TD::STAGE + TD::A_BYTES);
        else gv[st].template store<false>(smem + st * TD::STAGE + TD::A_BYTES);
    }
    lds_barrier();
    TD td;
    td.zero();
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        if (st >= nst) break;
        td.template compute<PM1>(smem + st * TD::STAGE);
    }
    lds_barrier();  // every wave is done with P v's stages
    float* buf = reinterpret_cast<float*>(smem);
    td.for_each([&](const float (&v)[1], int row, int col) { buf[row * OP + col] = v[0]; });
    __syncthreads();
    T* O = a.o + (tok + r0) * a.dv + c0;
    auto epi = [&](auto check) {
        tq.for_each([&](const float (&v)[2], int row, int col) {
            if (!decltype(check)::value || (row < nr && c0 + col < a.dv))
                O[(uint32_t)row * (uint32_t)a.dv + (uint32_t)col] = Elt<T>::st(v[1] + buf[row * OP + col]);
        });
    };
    if (nr >= kCausalRows && c0 + kApplyCols <= a.dv) epi(std::false_type{});
    else epi(std::true_type{});
}

// d_k limits: the sequential kernel is instantiated for d_k up to 256; the chunk-parallel kernels
// take any multiple of 32 (their tiles loop over d_k)
constexpr int kMaxSequentialDk = 256, kMaxParallelDk = 2048;

// The chunk-parallel path writes dS_c and S_c, 2 x 4 bytes per state element per chunk, on top of
// the algorithmic q, k, v, o traffic of 2 (d_k + d_v) bytes (bf16) per token: that extra is
// 4 d_k d_v / (chunk (d_k + d_v)) of it.  It is taken while that ratio is at most 2 (chunk >= 128
// at d_k = d_v = 128), where it runs well ahead of the sequential kernel.  Token-causal mode runs
// it over blocks of kCausalBlock tokens once the sequence holds two of them.
static bool lin_parallel(const linattn_desc& D) {
    if (D.N == 0) return false;
    if (D.mask == TTT_MASK_TOKEN_CAUSAL) return D.N >= 2 * kCausalBlock;
    const int64_t chunk = std::min<int64_t>(D.chunk, D.N);
    return 4LL * D.d_k * D.d_v <= 2LL * chunk * (D.d_k + D.d_v);
}

static ttt_status validate_lin(const linattn_desc* D) {
    if (!D) return fail(TTT_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (D->B < 0 || D->H < 0 || D->N < 0) return fail(TTT_ERR_INVALID_ARGUMENT, "B, H, N must be >= 0");
    if (D->d_k < 32 || D->d_k > kMaxParallelDk || D->d_k % 32)
        return fail(TTT_ERR_INVALID_ARGUMENT, "d_k=%d must be a multiple of 32 in [32, %d]", D->d_k, kMaxParallelDk);
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
    if (D->d_k > kMaxSequentialDk && !lin_parallel(*D))
        return fail(TTT_ERR_UNSUPPORTED,
                    "d_k=%d > %d needs the chunk-parallel path (a chunked mask with 4 d_k d_v <= 2 chunk (d_k + d_v), "
                    "or token-causal mode with N >= 256)",
                    D->d_k, kMaxSequentialDk);
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
    return check_launch("k_linattn", st);
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

// tokens per chunk of the chunk-parallel path: the mask's chunk, or the token-causal block
static int64_t lin_block(const linattn_desc& D) {
    return D.mask == TTT_MASK_TOKEN_CAUSAL ? kCausalBlock : D.chunk;
}

size_t lin_chunked_ws_bytes(int64_t nscan, int64_t nchunks, int d_k, int d_v, size_t es) {
    const size_t n = (size_t)(nscan * nchunks * (int64_t)d_v * d_k);
    return align256(n * 4) + align256(n * es * kStatePlanes);  // dS_c (fp32), then S_c
}

static size_t lin_ws_bytes(const linattn_desc& D) {
    if (!lin_parallel(D)) return 0;
    return lin_chunked_ws_bytes((int64_t)D.B * D.H, cdiv(D.N, lin_block(D)), D.d_k, D.d_v,
                                D.io_dtype == TTT_BF16 ? 2 : 4);
}

// Launch of the delta kernel over every (scan, chunk) of D's sequence: dS_c = sum over the chunk of
// w_i v_i k_i^T with w = eta (SCALE) or 1; a strided mode skips the chunks flags do not set.
template <typename T, bool SCALE>
static ttt_status launch_delta(const linattn_desc& D, int64_t chunk, int64_t nc, int mode, const uint32_t (&flags)[32],
                               const T* k, const T* v, const float* eta, float* dS, hipStream_t st) {
    DeltaArgs<T> da{};
    da.k = k;
    da.v = v;
    da.eta = eta;
    da.dS = dS;
    da.N = D.N;
    da.dk = D.d_k;
    da.dv = D.d_v;
    da.chunk = (int)chunk;
    da.nc = (int)nc;
    da.ntv = (int)cdiv(D.d_v, kDeltaRows);
    da.ntk = (int)cdiv(D.d_k, kDeltaCols);
    da.mode = mode;
    for (int w = 0; w < 32; ++w) da.flags[w] = flags[w];
    const int64_t S = (int64_t)D.B * D.H;
    {
        ProfScope ps(PK_LIN_DELTA, st);
        hipLaunchKernelGGL((k_lin_delta<T, SCALE>), dim3((unsigned)(S * nc * da.ntv * da.ntk)), dim3(kThreads), 0, st,
                           da);
    }
    return check_launch("k_lin_delta", st);
}

// Launch of the scan over the chunks of every scan (forward, or backward with rev)
template <typename T>
static ttt_status launch_scan(const linattn_desc& D, int64_t nc, int mode, const uint32_t (&flags)[32], const float* src,
                              T* Sc, const LinStateIO& io, int rev, int planes, hipStream_t st) {
    const int64_t S = (int64_t)D.B * D.H, dvk = (int64_t)D.d_v * D.d_k;
    ScanArgs<T> sa{};
    sa.dS = src;
    sa.Sc = Sc;
    sa.io = io;
    sa.dvk = dvk;
    sa.nc = (int)nc;
    sa.mode = mode;
    sa.nscan = (int)S;
    sa.rev = rev;
    sa.planes = planes;
    for (int w = 0; w < 32; ++w) sa.flags[w] = flags[w];
    {
        ProfScope ps(PK_LIN_SCAN, st);
        hipLaunchKernelGGL(k_lin_scan<T>, dim3((unsigned)cdiv(S * dvk / 4, kThreads)), dim3(kThreads), 0, st, sa);
    }
    return check_launch("k_lin_scan", st);
}

// Chunk updates and scan in one pass (k_lin_dscan): the states each chunk's queries see, as one
// io-dtype plane per chunk, with the entry/exit state and momentum of io (no step between them).
template <typename T>
static ttt_status launch_dscan(const linattn_desc& D, int64_t chunk, int64_t nc, int mode, const uint32_t (&flags)[32],
                               const T* k, const T* v, const float* eta, T* Sc, const LinStateIO& io, hipStream_t st) {
    const int64_t S = (int64_t)D.B * D.H;
    DscanArgs<T> ds{};
    ds.k = k;
    ds.v = v;
    ds.eta = eta;
    ds.Sc = Sc;
    ds.io = io;
    ds.N = D.N;
    ds.dk = D.d_k;
    ds.dv = D.d_v;
    ds.chunk = (int)chunk;
    ds.nc = (int)nc;
    ds.mode = mode;
    for (int w = 0; w < 32; ++w) ds.flags[w] = flags[w];
    ds.ntv = (int)cdiv(D.d_v, kDscanTile);
    ds.ntk = (int)cdiv(D.d_k, kDscanTile);
    // two chunks to a stage where a chunk is half of one; unmasked staging when every tile is whole
    // and every stage full
    constexpr int KS = DscanTile<T>::KSTEP;
    const bool pair = 2 * chunk == KS;
    const bool full = D.d_v % kDscanTile == 0 && D.d_k % kDscanTile == 0 && (pair || chunk % KS == 0) && D.N % KS == 0;
    const dim3 grid((unsigned)(S * ds.ntv * ds.ntk));
    {
        ProfScope ps(PK_LIN_SCAN, st);
        auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st, ds); };
        if (pair) {
            if (full) go(k_lin_dscan<T, true, true>);
            else go(k_lin_dscan<T, false, true>);
        } else {
            if (full) go(k_lin_dscan<T, true, false>);
            else go(k_lin_dscan<T, false, false>);
        }
    }
    return check_launch("k_lin_dscan", st);
}

// The fused pass is latency-bound (one stage in flight per workgroup), so it pays only where its
// 64 x 64 state tiles make at least one workgroup per CU and the chunk updates it keeps out of
// memory (4 d_v d_k bytes per chunk, written and read back) are at least half of the chunk's k and
// v bytes; d_k and d_v of 256 at most, where the delta kernel's 128-wide MFMA tiles do not win on
// arithmetic.  Token-causal blocks (128 tokens) take it where they go two to a stage (bf16).  The
// environment variable TTT_LIN_PASS, read on every call, overrides the choice ("fused" or
// "split"): both passes give the same bits, so tests run small cases through each.
template <typename T>
static bool dscan_pays(const linattn_desc& D, int64_t S, int64_t chunk) {
    if (const char* e = getenv("TTT_LIN_PASS")) {
        if (!strcmp(e, "fused")) return true;
        if (!strcmp(e, "split")) return false;
    }
    if (D.d_k > 256 || D.d_v > 256) return false;
    if (D.mask == TTT_MASK_TOKEN_CAUSAL && 2 * chunk != DscanTile<T>::KSTEP) return false;
    const int64_t wgs = S * cdiv(D.d_v, kDscanTile) * cdiv(D.d_k, kDscanTile);
    return wgs >= 256 && 4 * (int64_t)D.d_v * D.d_k >= chunk * (D.d_k + D.d_v);
}

template <typename T>
static ttt_status run_lin_parallel(const linattn_desc& D, LinArgs<T> a, char* ws, hipStream_t st,
                                   const LinStateIO& io) {
    const bool causal = D.mask == TTT_MASK_TOKEN_CAUSAL;
    const int64_t chunk = lin_block(D);
    const int64_t S = (int64_t)D.B * D.H, nc = cdiv(D.N, chunk), dvk = (int64_t)D.d_v * D.d_k;
    float* dS = (float*)ws;
    T* Sc = (T*)(ws + align256((size_t)(S * nc * dvk * 4)));  // kStatePlanes io-dtype planes per chunk
    ttt_status rc;
    const int smode = causal ? TTT_MASK_APPLY_THEN_UPDATE : D.mask;  // a causal block sees the state before it
    if (!io.between && dscan_pays<T>(D, S, chunk)) {
        // 1 + 2 in one pass
        if ((rc = launch_dscan<T>(D, chunk, nc, smode, a.flags, a.k, a.v, a.eta, Sc, io, st)) != TTT_OK) return rc;
    } else {
        // 1. per-chunk updates
        rc = launch_delta<T, true>(D, chunk, nc, D.mask, a.flags, a.k, a.v, a.eta, dS, st);
        if (rc != TTT_OK) return rc;
        // (the caller's step between the updates and the scan, which may hand the scan another buffer)
        const float* scan_src = dS;
        if (io.between && (rc = io.between(io.between_ctx, dS, &scan_src, st)) != TTT_OK) return rc;
        // 2. states seen by each chunk, and S_out
        rc = launch_scan<T>(D, nc, smode, a.flags, scan_src, Sc, io, 0, kStatePlanes, st);
        if (rc != TTT_OK) return rc;
    }
    // 3. apply
    ApplyArgs<T> aa{};
    aa.q = a.q;
    aa.Sc = Sc;
    aa.o = a.o;
    aa.N = D.N;
    aa.dk = D.d_k;
    aa.dv = D.d_v;
    aa.chunk = (int)chunk;
    aa.nc = (int)nc;
    aa.ntt = (int)cdiv(std::min<int64_t>(chunk, D.N), kApplyRows);
    aa.ntv = (int)cdiv(D.d_v, kApplyCols);
    aa.nscan = (int)S;
    aa.k = a.k;
    aa.v = a.v;
    aa.eta = a.eta;
    {
        ProfScope ps(PK_LIN_APPLY, st);
        if (causal)  // two workgroups of query rows per block
            hipLaunchKernelGGL(k_lin_apply_causal<T>, dim3((unsigned)(S * nc * aa.ntv * 2)), dim3(kThreads), 0, st, aa);
        else
            hipLaunchKernelGGL(k_lin_apply<T>, dim3((unsigned)(S * nc * aa.ntt * aa.ntv)), dim3(kThreads), 0, st, aa);
    }
    return check_launch(causal ? "k_lin_apply_causal" : "k_lin_apply", st);
}

template <typename T>
ttt_status lin_chunked_run(const linattn_desc& D, const uint32_t (&flags)[32], const T* q, const T* k, const T* v,
                           const float* eta, T* o, const LinStateIO& io, char* ws, hipStream_t st) {
    LinArgs<T> a{q, k, v, eta, io.S0, o, io.Sout, D.N, D.d_v, D.chunk, D.mask, 0, 0, {}};
    for (int w = 0; w < 32; ++w) a.flags[w] = flags[w];
    return run_lin_parallel<T>(D, a, ws, st, io);
}
template ttt_status lin_chunked_run<uint16_t>(const linattn_desc&, const uint32_t (&)[32], const uint16_t*,
                                              const uint16_t*, const uint16_t*, const float*, uint16_t*,
                                              const LinStateIO&, char*, hipStream_t);
template ttt_status lin_chunked_run<float>(const linattn_desc&, const uint32_t (&)[32], const float*, const float*,
                                           const float*, const float*, float*, const LinStateIO&, char*, hipStream_t);

// ---------------------------------------------------------------------------------------------
// Backward of the chunked masks: the outer-loop gradients for training through the parallel form
// ("Test-Time Training with KV Binding Is Secretly Linear Attention", Sec. 6.2 and Fig. 4).
//
// For L = sum_t dO_t . o_t + <dS_out, S_out>: chunk c's queries see S_c, so dq_t = S_c^T dO_t and
// D_c = sum over the chunk of dO_t q_t^T is the gradient of S_c.  Chunk j's update reaches the S_c
// of the chunks after it (and its own under update-then-apply and the full mask) and S_out, so its
// gradient is R_j = dS_out + the suffix sum of those D_c; then dv_s = eta_s R_j k_s,
// dk_s = eta_s R_j^T v_s, deta_s = v_s . (R_j k_s), and dS0 = dS_out + sum_c D_c.  A chunk that a
// strided mask does not update gets zero dk, dv and deta.  Launches: the forward's delta and scan
// (S_c), the delta kernel with unit weights over (q, dO) into the same dS buffer (D_c), the scan
// walked backwards (R_j and dS0), then the two product kernels.  The scans carry fp32; the products
// read S_c and R_j as one io-dtype plane, as the forward's apply reads S_c.
constexpr int kBwdPlanes = kStatePlanes;

// The states of a recurrence whose steps end in the L2 norm of the state's rows, forward and
// transposed: one wave per row of one scan's state (d_k elements, 4 per lane and float4), walking
// the chunks in fp32.  Forward: per updating chunk and step, m <- beta m + dsign dS_c (beta = 0
// without momentum), x = S + m, S <- x / max(|x|, 1e-6) row by row; the step's S and |x| are kept
// for the transpose, and each chunk's state as its queries see it goes out as one io-dtype plane.
// Reverse, from the last chunk, with st and mom the gradients of S and m: every chunk's D_c adds to
// st (where its queries saw it), and each step, last first, takes the norm's transpose
// gx = (st - y (y . st)) / |x| (st / 1e-6 where |x| <= 1e-6; y the step's S), gives g = mom + gx to
// the chunk's update, and sets mom <- beta g, st <- gx; the chunk's slot receives the sum of its g.
constexpr int kRowScanVec = 8;  // float4 per lane: rows of up to 2048 elements
constexpr float kRowNormEps = 1e-6f;

template <typename T> struct RowScanArgs {
    const float* src;  // [S][nc][d_v][d_k] fp32: the chunk updates (forward) or the D_c (reverse)
    T* out;            // [S][nc][d_v][d_k]: the states the chunks' queries see (forward) or R_c (reverse)
    float* y;          // [S][nc * reps][d_v][d_k] fp32: each step's state
    float* nrm;        // [S][nc * reps][d_v]: each step's |x|
    LinStateIO io;     // forward: S0; reverse: S0 = dS_out, Sout = dS0; dsign, reps, beta
    int64_t dvk; int dv, dk, nc, mode, nscan, rev;
    uint32_t flags[32];
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_lin_row_scan(RowScanArgs<T> a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= (int64_t)a.nscan * a.dv) return;  // whole waves; the kernel has no barrier
    const int64_t scan = row / a.dv;
    const int r = (int)(row % a.dv), nv = a.dk / 4;
    const LinStateIO& io = a.io;
    const int reps = io.reps;
    const float beta = io.mom ? io.beta : 0.f;
    const bool post = a.mode == TTT_MASK_UPDATE_THEN_APPLY || a.mode == TTT_MASK_FULL;
    f32x4_t st[kRowScanVec], mm[kRowScanVec];
#pragma unroll
    for (int i = 0; i < kRowScanVec; ++i) {
        st[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mm[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int e = (i * 64 + lane) * 4;
        if (io.S0 && i * 64 + lane < nv) {  // only 4-byte aligned
            const float* s0 = io.S0 + (io.s0_heads ? scan % io.s0_heads : scan) * io.s0_stride + (int64_t)r * a.dk + e;
#pragma unroll
            for (int u = 0; u < 4; ++u) st[i][u] = s0[u];
        }
    }
    auto slot = [&](int c) { return (scan * a.nc + c) * a.dvk + (int64_t)r * a.dk; };
    auto step_slot = [&](int c, int k) { return ((scan * a.nc + c) * reps + k); };
    auto put = [&](int c, const f32x4_t (&x)[kRowScanVec]) {
        T* dst = a.out + slot(c);
#pragma unroll
        for (int i = 0; i < kRowScanVec; ++i)
            if (i * 64 + lane < nv) Pack4<T>::store(dst + (i * 64 + lane) * 4, x[i][0], x[i][1], x[i][2], x[i][3]);
    };
    auto load = [&](const float* p, f32x4_t (&x)[kRowScanVec]) {
#pragma unroll
        for (int i = 0; i < kRowScanVec; ++i)
            x[i] = i * 64 + lane < nv ? *reinterpret_cast<const f32x4_t*>(p + (i * 64 + lane) * 4)
                                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
    };
    auto dot = [&](const f32x4_t (&x)[kRowScanVec], const f32x4_t (&w)[kRowScanVec]) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kRowScanVec; ++i) t += x[i][0] * w[i][0] + x[i][1] * w[i][1] + x[i][2] * w[i][2] + x[i][3] * w[i][3];
        return wave_sum(t);
    };
    f32x4_t d[kRowScanVec];
    if (!a.rev) {
        for (int c = 0; c < a.nc; ++c) {
            const bool upd = a.mode != TTT_MASK_STRIDED || ((a.flags[c >> 5] >> (c & 31)) & 1u);
            if (!post) put(c, st);
            if (upd) {
                load(a.src + slot(c), d);
                for (int k = 0; k < reps; ++k) {
#pragma unroll
                    for (int i = 0; i < kRowScanVec; ++i) {
                        mm[i] = beta * mm[i] + io.dsign * d[i];
                        st[i] += mm[i];
                    }
                    const float n = sqrtf(dot(st, st)), f = 1.f / fmaxf(n, kRowNormEps);
                    float* yp = a.y + step_slot(c, k) * a.dvk + (int64_t)r * a.dk;
#pragma unroll
                    for (int i = 0; i < kRowScanVec; ++i) {
                        st[i] *= f;
                        if (i * 64 + lane < nv) *reinterpret_cast<f32x4_t*>(yp + (i * 64 + lane) * 4) = st[i];
                    }
                    if (lane == 0) a.nrm[step_slot(c, k) * a.dv + r] = n;
                }
            }
            if (post) put(c, st);
        }
        return;
    }
    f32x4_t y[kRowScanVec], rs[kRowScanVec];
    for (int i = 0; i < a.nc; ++i) {
        const int c = a.nc - 1 - i;
        const bool upd = a.mode != TTT_MASK_STRIDED || ((a.flags[c >> 5] >> (c & 31)) & 1u);
        load(a.src + slot(c), d);
        if (post)
#pragma unroll
            for (int j = 0; j < kRowScanVec; ++j) st[j] += d[j];
        if (upd) {
#pragma unroll
            for (int j = 0; j < kRowScanVec; ++j) rs[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int k = reps - 1; k >= 0; --k) {
                load(a.y + step_slot(c, k) * a.dvk + (int64_t)r * a.dk, y);
                const float n = a.nrm[step_slot(c, k) * a.dv + r];
                const float yg = dot(y, st);
                const bool big = n > kRowNormEps;
                const float inv = 1.f / fmaxf(n, kRowNormEps);
#pragma unroll
                for (int j = 0; j < kRowScanVec; ++j) {
                    const f32x4_t gx = big ? (st[j] - yg * y[j]) * inv : st[j] * inv;
                    const f32x4_t g = mm[j] + gx;
                    rs[j] += g;
                    mm[j] = beta * g;
                    st[j] = gx;
                }
            }
            put(c, rs);
        }
        if (!post)
#pragma unroll
            for (int j = 0; j < kRowScanVec; ++j) st[j] += d[j];
    }
    if (io.Sout)
#pragma unroll
        for (int i = 0; i < kRowScanVec; ++i)
            if (i * 64 + lane < nv)
#pragma unroll
                for (int u = 0; u < 4; ++u) io.Sout[scan * io.sout_stride + (int64_t)r * a.dk + (i * 64 + lane) * 4 + u] = st[i][u];
}

// dq = dO S_c and dk = diag(eta) v R_c for one chunk: tokens x d_k, contracting over d_v.  The
// d_v x d_k matrix goes through the transposing stager (its d_k index is the tile column).  One
// launch covers both jobs: the first per_job workgroups do dq, the others dk.  The tile leaves row by
// row through LDS, since the transposed operand permutes the accumulator columns.  The dk job also
// forms deta_s = k_s . w_s with w_s = R^T v_s (its rows before the eta factor) over the tile's d_k
// columns: each thread takes 4 columns of 16 rows; a butterfly over the 32 lanes that share each row
// leaves the row sums on the even lanes.

template <typename T> struct BwdTJob {
    const T* y; const T* M; T* out;
    const float* eta;  // row factors (dk), or null (dq)
    int skip;          // strided mask: rows of chunks that do not update are zero
    const T* kk;       // dk job: the keys, for deta_s = k_s . (R^T v_s) from the unscaled rows
    float* deta;       // dk job: deta, or its per-column-tile partials (ntok apart); null for dq
    T* gate;           // GATE: rows of 2 d_k holding factors u | w, overwritten by g u | g w
};
template <typename T> struct BwdTArgs {
    BwdTJob<T> job[2];
    int64_t N, ntok; int dk, dv, chunk, nc, ntt, ntn, per_job, mode;
    float es;  // dk job: the forward's update scale (eta's factor)
    uint32_t flags[32];
};

// GATE: a job's result g (dq or dk) is not stored; the row's factors u (columns 0 .. d_k-1) and w
// (d_k .. 2 d_k-1) of the job's gate buffer are read and replaced by g u and g w, each element by the
// thread that reads it (the gradient carried on through an elementwise product, e.g. the TTT layer's
// SwiGLU features).
template <typename T, bool GATE>
__global__ __launch_bounds__(kThreads, 2) void k_lin_bwd_t(BwdTArgs<T> a) {
    constexpr int PLANES = kBwdPlanes;
    using TB = Tile<T, kApplyRows, kApplyCols, 1, 2, 1, PLANES, PLANES, false, true>;
    using PM = typename std::conditional<PLANES == 2, PMQ, PM1>::type;
    static_assert(TB::RV_LDS <= TB::LDS, "row bands fit the tile's LDS");
    __shared__ __attribute__((aligned(16))) char smem[TB::LDS];
    const int lb = xcd_block(gridDim.x);
    const bool second = lb >= a.per_job;
    const BwdTJob<T> jb = second ? a.job[1] : a.job[0];
    const int l = second ? lb - a.per_job : lb;
    const int per_chunk = a.ntt * a.ntn;
    const int unit = l / per_chunk, t = l % per_chunk;
    const int scan = unit / a.nc, c = unit % a.nc;
    const int r0 = (t / a.ntn) * kApplyRows, c0 = (t % a.ntn) * kApplyCols;
    const int64_t tok = (int64_t)scan * a.N + (int64_t)c * a.chunk;
    const int nl = (int)std::min<int64_t>(a.chunk, a.N - (int64_t)c * a.chunk);
    if (r0 >= nl) return;  // uniform per workgroup
    const int rows = std::min(kApplyRows, nl - r0), cols = std::min(kApplyCols, a.dk - c0);
    // output rows: dk elements apart, or 2 dk in the gate buffer (g u here, g w dk further on)
    const uint32_t ld = GATE ? 2u * (uint32_t)a.dk : (uint32_t)a.dk;
    T* O = (GATE ? jb.gate : jb.out) + (tok + r0) * ld + c0;
    float* de = jb.deta ? jb.deta + (int64_t)(t % a.ntn) * a.ntok + tok + r0 : nullptr;
    if (jb.skip && a.mode == TTT_MASK_STRIDED && !((a.flags[c >> 5] >> (c & 31)) & 1u)) {
        for (int e = threadIdx.x; e < rows * cols; e += kThreads) {
            const uint32_t off = (uint32_t)(e / cols) * ld + (uint32_t)(e % cols);
            O[off] = Elt<T>::st(0.f);
            if (GATE) O[off + a.dk] = Elt<T>::st(0.f);
        }
        if (de)
            for (int e = threadIdx.x; e < rows; e += kThreads) de[e] = 0.f;
        return;
    }
    const int64_t dvk = (int64_t)a.dv * a.dk;
    const T* M = jb.M + (int64_t)unit * PLANES * dvk + c0;
    const Opnd<T> A[1] = {{jb.y + (tok + r0) * a.dv, a.dv, nl - r0, a.dv}};
    Opnd<T> B[PLANES];
#pragma unroll
    for (int p = 0; p < PLANES; ++p) B[p] = Opnd<T>{M + p * dvk, a.dk, a.dk - c0, a.dv};
    TB tl;
    tl.template run<PM>(A, B, a.dv, smem);
    if constexpr (PLANES == 2) {
#pragma unroll
        for (int i = 0; i < TB::FM; ++i)
#pragma unroll
            for (int j = 0; j < TB::FN; ++j) tl.acc[0][i][j] += tl.acc[1][i][j];
    }
    const float* eta = jb.eta ? jb.eta + tok + r0 : nullptr;
    const T* K = jb.kk ? jb.kk + (tok + r0) * a.dk + c0 : nullptr;
    constexpr int NV = TB::RV_N / PLANES;  // row pieces of a thread (one accumulator)
    static_assert(NV == 16 && TB::BN / 4 == 32, "32 lanes per tile row, 16 rows per lane");
    // the dk job's keys and row factors for the epilogue's positions, all loads issued at once (the
    // staging registers are free by now)
    typename Pack4<T>::raw kr[NV];
    float ef[NV];
    if (K) {  // uniform: the job
        TB::rows_via_lds_pos([&](int idx, int p, int row, int col) {
            if (p == 0) {
                const bool in = row < rows && col < cols;
                kr[idx] = Pack4<T>::load_raw(K + (in ? (uint32_t)row * (uint32_t)a.dk + (uint32_t)col : 0u));
                ef[idx] = eta[in ? row : 0];
            }
        });
    }
    float pd[NV];
    tl.template rows_via_lds<1>(smem, [&](int idx, int, int row, int col, const float4& v) {
        pd[idx] = 0.f;
        if (row < rows && col < cols) {
            const float f = K ? ef[idx] * a.es : 1.f;
            if constexpr (GATE) {
                const uint32_t off = (uint32_t)row * ld + (uint32_t)col;
                float u[4], w[4];
                Pack4<T>::unpack(Pack4<T>::load_raw(O + off), u);
                Pack4<T>::unpack(Pack4<T>::load_raw(O + off + a.dk), w);
                const float g[4] = {v.x * f, v.y * f, v.z * f, v.w * f};
                Pack4<T>::store(O + off, g[0] * u[0], g[1] * u[1], g[2] * u[2], g[3] * u[3]);
                Pack4<T>::store(O + off + a.dk, g[0] * w[0], g[1] * w[1], g[2] * w[2], g[3] * w[3]);
            } else {
                const uint32_t off = (uint32_t)row * (uint32_t)a.dk + (uint32_t)col;
                Pack4<T>::store(O + off, v.x * f, v.y * f, v.z * f, v.w * f);
            }
            if (K) {
                float kv[4];
                Pack4<T>::unpack(kr[idx], kv);
                pd[idx] = v.x * kv[0] + v.y * kv[1] + v.z * kv[2] + v.w * kv[3];
            }
        }
    });
    if (!de) return;  // uniform: the job
    // reduce-scatter: at step s a lane keeps the half of its list picked by bit s of its lane index
    // and adds the partner's copy of that half; then lanes l and l ^ 1 add their last entry, so lane l
    // holds the 32 lanes' sum for entry (l >> 1) & 15
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int sh = 16, n = NV / 2; sh >= 2; sh >>= 1, n >>= 1) {
        const bool up = (lane & sh) != 0;
#pragma unroll
        for (int x = 0; x < n; ++x) {
            const float keep = up ? pd[x + n] : pd[x];
            const float give = up ? pd[x] : pd[x + n];
            pd[x] = keep + __shfl_xor(give, sh);
        }
    }
    pd[0] += __shfl_xor(pd[0], 1);
    if ((lane & 1) == 0) {
        // entry idx = h * RV_K + k covers tile row h * WM + (k * NT + tid) / 32
        const int idx = (lane >> 1) & 15, h = idx / TB::RV_K, k = idx % TB::RV_K;
        const int row = h * TB::WM + (k * TB::NT + wave * 64 + (lane & 32)) / 32;
        if (row < rows) de[row] = pd[0] * a.es;
    }
}

// dv = diag(eta) k R_c^T for one chunk: tokens x d_v, contracting over d_k, R_c row-major (as the
// forward's apply reads S_c).  The rows' eta factors are staged in LDS before the product.
template <typename T> struct BwdNArgs {
    const T* k; const T* R; const float* eta; T* dv;
    int64_t N; int dk, dvn, chunk, nc, ntt, ntn, mode;
    float es;  // the forward's update scale (eta's factor)
    uint32_t flags[32];
};

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_lin_bwd_n(BwdNArgs<T> a) {
    constexpr int PLANES = kBwdPlanes;
    using TA = Tile<T, kApplyRows, kApplyCols, 1, 2, 1, PLANES, PLANES, false, false>;
    using PM = typename std::conditional<PLANES == 2, PMQ, PM1>::type;
    __shared__ __attribute__((aligned(16))) char smem[TA::LDS];
    const int lb = xcd_block(gridDim.x);
    const int per_chunk = a.ntt * a.ntn;
    const int unit = lb / per_chunk, t = lb % per_chunk;
    const int scan = unit / a.nc, c = unit % a.nc;
    const int r0 = (t / a.ntn) * kApplyRows, c0 = (t % a.ntn) * kApplyCols;
    const int64_t tok = (int64_t)scan * a.N + (int64_t)c * a.chunk;
    const int nl = (int)std::min<int64_t>(a.chunk, a.N - (int64_t)c * a.chunk);
    if (r0 >= nl) return;  // uniform per workgroup
    const int rows = std::min(kApplyRows, nl - r0), cols = std::min(kApplyCols, a.dvn - c0);
    T* O = a.dv + (tok + r0) * a.dvn + c0;
    if (a.mode == TTT_MASK_STRIDED && !((a.flags[c >> 5] >> (c & 31)) & 1u)) {
        for (int e = threadIdx.x; e < rows * cols; e += kThreads)
            O[(uint32_t)(e / cols) * (uint32_t)a.dvn + (uint32_t)(e % cols)] = Elt<T>::st(0.f);
        return;
    }
    __shared__ float er[kApplyRows];  // the rows' eta, ordered before the epilogue by run()'s barriers
    if (threadIdx.x < rows) er[threadIdx.x] = a.es * a.eta[tok + r0 + threadIdx.x];
    const int64_t dvk = (int64_t)a.dvn * a.dk;
    const T* R = a.R + (int64_t)unit * PLANES * dvk + (int64_t)c0 * a.dk;
    const Opnd<T> A[1] = {{a.k + (tok + r0) * a.dk, a.dk, nl - r0, a.dk}};
    Opnd<T> B[PLANES];
#pragma unroll
    for (int p = 0; p < PLANES; ++p) B[p] = Opnd<T>{R + p * dvk, a.dk, a.dvn - c0, a.dk};
    TA tl;
    tl.template run<PM>(A, B, a.dk, smem);
    // element r of a thread's block (i, j) lies on tile row wm*WM + i*32 + 8*(r>>2) + 4*(lane>>5) + (r&3)
    // and column wn*WN + j*32 + (lane&31)
    const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / TA::WGN, wn = (threadIdx.x >> 6) % TA::WGN;
#pragma unroll
    for (int i = 0; i < TA::FM; ++i)
#pragma unroll
        for (int j = 0; j < TA::FN; ++j) {
            const int col = wn * TA::WN + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * TA::WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                float u = tl.acc[0][i][j][r];
                if constexpr (PLANES == 2) u += tl.acc[1][i][j][r];
                if (row < rows && col < cols)
                    O[(uint32_t)row * (uint32_t)a.dvn + (uint32_t)col] = Elt<T>::st(u * er[row]);
            }
        }
}

// deta = the sum of the column tiles' partials
__global__ __launch_bounds__(kThreads) void k_lin_deta_sum(const float* part, float* deta, int64_t ntok, int ntn) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= ntok) return;
    float s = 0.f;
    for (int t = 0; t < ntn; ++t) s += part[(int64_t)t * ntok + i];
    deta[i] = s;
}

ttt_status validate_lin_desc_bwd(const linattn_desc* D) {
    ttt_status rc = validate_lin(D);
    if (rc != TTT_OK) return rc;
    if (D->mask == TTT_MASK_TOKEN_CAUSAL)
        return fail(TTT_ERR_UNSUPPORTED, "the backward covers the chunked masks (not TOKEN_CAUSAL)");
    const int64_t S = (int64_t)D->B * D->H, nc = D->N ? cdiv(D->N, D->chunk) : 0;
    const int64_t ntt = D->N ? cdiv(std::min<int64_t>(D->chunk, D->N), kApplyRows) : 0;
    const int64_t tiles = S * nc * ntt * std::max(cdiv(D->d_k, kApplyCols), cdiv(D->d_v, kApplyCols));
    const int64_t dtiles = S * nc * cdiv(D->d_v, kDeltaRows) * cdiv(D->d_k, kDeltaCols);
    if (2 * tiles > INT32_MAX || dtiles > INT32_MAX || S * D->d_v * (int64_t)D->d_k / 4 > INT32_MAX * (int64_t)kThreads)
        return fail(TTT_ERR_UNSUPPORTED, "too many tiles for one launch");
    return TTT_OK;
}

// dS_c (fp32), then S_c and R_c (one io-dtype plane each), then the deta partials; with the row norm
// also every step's state (fp32) and row norms
size_t lin_chunked_bwd_ws_bytes(const linattn_desc& D, int norm, int reps) {
    if (D.N == 0) return 0;
    const int64_t S = (int64_t)D.B * D.H, nc = cdiv(D.N, D.chunk), ntn = cdiv(D.d_k, kApplyCols);
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4, n = (size_t)(S * nc * (int64_t)D.d_v * D.d_k);
    size_t b = align256(n * 4) + 2 * align256(n * es) + (ntn > 1 ? align256((size_t)(ntn * S * D.N * 4)) : 0);
    if (norm) b += align256(n * reps * 4) + align256((size_t)(S * nc * reps * (int64_t)D.d_v * 4));
    return b;
}

template <typename T>
ttt_status lin_chunked_bwd(const linattn_desc& D, const uint32_t (&flags)[32], const T* q, const T* k, const T* v,
                           const float* eta, const T* dO, const LinBwdIO& io, T* dq, T* dk, T* dv, float* deta,
                           char* ws, hipStream_t st) {
    const int64_t S = (int64_t)D.B * D.H, dvk = (int64_t)D.d_v * D.d_k;
    const int64_t chunk = D.chunk, nc = D.N ? cdiv(D.N, chunk) : 0;
    const size_t sb = align256((size_t)(S * nc * dvk * 4)), tb = align256((size_t)(S * nc * dvk) * sizeof(T));
    const int64_t ntk_ = cdiv(D.d_k, kApplyCols);
    const size_t pb = ntk_ > 1 ? align256((size_t)(ntk_ * S * D.N * 4)) : 0;
    float* dS = (float*)ws;
    T* Sc = (T*)(ws + sb);
    T* R = (T*)(ws + sb + tb);
    float* part = (float*)(ws + sb + 2 * tb);
    float* ybuf = (float*)(ws + sb + 2 * tb + pb);  // norm: each step's state, then the row norms
    float* nbuf = (float*)(ws + sb + 2 * tb + pb + align256((size_t)(S * nc * dvk) * io.reps * 4));
    // the row-wise scans of a state whose steps end in the row norm
    auto row_scan = [&](const float* src, T* out, const LinStateIO& sio, int rev) -> ttt_status {
        RowScanArgs<T> ra{};
        ra.src = src;
        ra.out = out;
        ra.y = ybuf;
        ra.nrm = nbuf;
        ra.io = sio;
        ra.dvk = dvk;
        ra.dv = D.d_v;
        ra.dk = D.d_k;
        ra.nc = (int)nc;
        ra.mode = D.mask;
        ra.nscan = (int)S;
        ra.rev = rev;
        for (int w = 0; w < 32; ++w) ra.flags[w] = flags[w];
        {
            ProfScope ps(PK_LIN_SCAN, st);
            hipLaunchKernelGGL(k_lin_row_scan<T>, dim3((unsigned)cdiv(S * D.d_v, kThreads / 64)), dim3(kThreads), 0,
                               st, ra);
        }
        return check_launch("k_lin_row_scan", st);
    };
    uint32_t all[32];
    for (int w = 0; w < 32; ++w) all[w] = ~0u;
    ttt_status rc;
    if (D.N > 0) {
        // the states the chunks' queries saw
        LinStateIO fio;
        fio.S0 = io.S0;
        fio.s0_stride = io.s0_stride;
        fio.s0_heads = io.s0_heads;
        fio.dsign = io.dsign;
        fio.reps = io.reps;
        fio.mom = io.mom;
        fio.beta = io.beta;
        if (!io.norm && dscan_pays<T>(D, S, chunk)) {
            rc = launch_dscan<T>(D, chunk, nc, D.mask, flags, k, v, eta, Sc, fio, st);
        } else {
            if ((rc = launch_delta<T, true>(D, chunk, nc, D.mask, flags, k, v, eta, dS, st)) != TTT_OK) return rc;
            if (io.norm) rc = row_scan(dS, Sc, fio, 0);
            else rc = launch_scan<T>(D, nc, D.mask, flags, dS, Sc, fio, 0, kBwdPlanes, st);
        }
        if (rc != TTT_OK) return rc;
        // D_c = sum over the chunk of dO q^T, every chunk
        if ((rc = launch_delta<T, false>(D, chunk, nc, TTT_MASK_APPLY_THEN_UPDATE, all, q, dO, nullptr, dS, st)) !=
            TTT_OK)
            return rc;
    }
    // R_j (backwards over the chunks, every D_c added; the mask decides whether chunk j's own term is
    // in R_j) and dS0 = dS_out + sum_c D_c
    LinStateIO rio;
    rio.S0 = io.dS_out;
    rio.s0_stride = io.dso_stride;
    rio.Sout = io.dS0;
    rio.sout_stride = io.ds0_stride;
    if (io.mom || io.norm) {  // the recurrence transposed: every D_c adds, the mask's chunks update
        rio.mom = io.mom;
        rio.beta = io.beta;
        rio.reps = io.reps;
    }
    if (D.N > 0 || io.dS0) {
        if (io.norm) rc = row_scan(dS, R, rio, 1);
        else rc = launch_scan<T>(D, nc, D.mask, io.mom ? flags : all, dS, R, rio, 1, kBwdPlanes, st);
        if (rc != TTT_OK) return rc;
    }
    // the gradient of a chunk's update sum eta v k^T: R_j times the update's sign, and (for a plain
    // sum) times its repeats, which the transposed recurrence folds in otherwise
    const float es = (io.mom || io.norm) ? io.dsign : io.dsign * (float)io.reps;
    if (D.N == 0) return TTT_OK;
    const int ntt = (int)cdiv(std::min<int64_t>(chunk, D.N), kApplyRows);
    const int ntk = (int)cdiv(D.d_k, kApplyCols);  // column tiles of dq, dk (and deta partials)
    float* de = ntk > 1 ? part : deta;
    BwdTArgs<T> ta{};
    const bool gate = io.gate[0] != nullptr;
    ta.job[0] = BwdTJob<T>{dO, Sc, dq, nullptr, 0, nullptr, nullptr, (T*)io.gate[0]};
    ta.job[1] = BwdTJob<T>{v, R, dk, eta, 1, k, de, (T*)io.gate[1]};
    ta.N = D.N;
    ta.ntok = S * D.N;
    ta.dk = D.d_k;
    ta.dv = D.d_v;
    ta.chunk = (int)chunk;
    ta.nc = (int)nc;
    ta.ntt = ntt;
    ta.ntn = ntk;
    ta.per_job = (int)(S * nc * ntt * ntk);
    ta.mode = D.mask;
    ta.es = es;
    for (int w = 0; w < 32; ++w) ta.flags[w] = flags[w];
    {
        ProfScope ps(PK_LIN_BWD_T, st);
        if (gate) hipLaunchKernelGGL((k_lin_bwd_t<T, true>), dim3((unsigned)(2 * ta.per_job)), dim3(kThreads), 0, st, ta);
        else hipLaunchKernelGGL((k_lin_bwd_t<T, false>), dim3((unsigned)(2 * ta.per_job)), dim3(kThreads), 0, st, ta);
    }
    if ((rc = check_launch("k_lin_bwd_t", st)) != TTT_OK) return rc;
    BwdNArgs<T> na{};
    na.k = k;
    na.R = R;
    na.eta = eta;
    na.dv = dv;
    na.N = D.N;
    na.dk = D.d_k;
    na.dvn = D.d_v;
    na.chunk = (int)chunk;
    na.nc = (int)nc;
    na.ntt = ntt;
    na.ntn = (int)cdiv(D.d_v, kApplyCols);
    na.mode = D.mask;
    na.es = es;
    for (int w = 0; w < 32; ++w) na.flags[w] = flags[w];
    {
        ProfScope ps(PK_LIN_BWD_N, st);
        hipLaunchKernelGGL(k_lin_bwd_n<T>, dim3((unsigned)(S * nc * ntt * na.ntn)), dim3(kThreads), 0, st, na);
    }
    if ((rc = check_launch("k_lin_bwd_n", st)) != TTT_OK) return rc;
    if (ntk > 1) {
        {
            ProfScope ps(PK_LIN_DETA, st);
            hipLaunchKernelGGL(k_lin_deta_sum, dim3((unsigned)cdiv(S * D.N, kThreads)), dim3(kThreads), 0, st,
                               (const float*)part, deta, S * D.N, ntk);
        }
        if ((rc = check_launch("k_lin_deta_sum", st)) != TTT_OK) return rc;
    }
    return TTT_OK;
}

template ttt_status lin_chunked_bwd<uint16_t>(const linattn_desc&, const uint32_t (&)[32], const uint16_t*,
                                              const uint16_t*, const uint16_t*, const float*, const uint16_t*,
                                              const LinBwdIO&, uint16_t*, uint16_t*, uint16_t*, float*, char*,
                                              hipStream_t);
template ttt_status lin_chunked_bwd<float>(const linattn_desc&, const uint32_t (&)[32], const float*, const float*,
                                           const float*, const float*, const float*, const LinBwdIO&, float*, float*,
                                           float*, float*, char*, hipStream_t);

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status linattn_workspace_bytes(const linattn_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_lin(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = lin_ws_bytes(*desc);
    return TTT_OK;
}

extern "C" ttt_status linattn_forward(const linattn_desc* desc, const void* q, const void* k, const void* v,
                                      const float* eta, const float* S0, void* o, float* S_out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
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
    const size_t need = lin_ws_bytes(D);
    if (need && (!workspace || workspace_bytes < need))
        return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (need && !aligned(workspace, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    {  // every buffer the call touches lies in a device allocation that holds all of it
        const bool t = D.N > 0;
        const struct { const void* p; size_t n; const char* name; } bufs[] = {
            {q, t ? qb : 0, "q"}, {k, t ? qb : 0, "k"}, {v, t ? vb : 0, "v"}, {o, t ? vb : 0, "o"},
            {eta, t ? (size_t)S * D.N * 4 : 0, "eta"}, {S0, sb, "S0"}, {S_out, sb, "S_out"},
            {workspace, need, "workspace"}};
        for (const auto& b : bufs)
            if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    }
    hipStream_t st = (hipStream_t)stream;
    // 32-row slices of S: measured faster than 16-row slices, whose extra workgroups double the
    // re-reads of q and k (the 16-row instantiation is kept for the bf16 kernel)
    const int vt = 32;
    const int nvt = D.d_v / vt;
    auto go = [&](auto* tag) -> ttt_status {
        using T = typename std::remove_pointer<decltype(tag)>::type;
        LinArgs<T> a{(const T*)q, (const T*)k, (const T*)v, eta, S0, (T*)o, S_out, D.N, D.d_v, D.chunk, D.mask,
                     nvt, vt, {}};
        if (D.mask == TTT_MASK_STRIDED)
            for (int64_t j = 0; j < cdiv(D.N, D.chunk); ++j)
                if (D.update_chunks[j]) a.flags[j >> 5] |= 1u << (j & 31);
        if (need) {
            LinStateIO io;
            io.S0 = S0;
            io.s0_stride = (int64_t)D.d_v * D.d_k;
            io.Sout = S_out;
            io.sout_stride = io.s0_stride;
            return run_lin_parallel<T>(D, a, (char*)workspace, st, io);
        }
        return run_lin<T>(D, a, st);
    };
    if (D.io_dtype == TTT_BF16) return go((uint16_t*)nullptr);
    return go((float*)nullptr);
}

extern "C" ttt_status linattn_backward_workspace_bytes(const linattn_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_lin_desc_bwd(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = lin_chunked_bwd_ws_bytes(*desc);
    return TTT_OK;
}

extern "C" ttt_status linattn_backward(const linattn_desc* desc, const void* q, const void* k, const void* v,
                                       const float* eta, const float* S0, const void* dO, const float* dS_out,
                                       void* dq, void* dk, void* dv, float* deta, float* dS0, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    clear_error();
    ttt_status rc = validate_lin_desc_bwd(desc);
    if (rc != TTT_OK) return rc;
    const linattn_desc& D = *desc;
    const int64_t S = (int64_t)D.B * D.H;
    if (S == 0) return TTT_OK;
    const bool t = D.N > 0;
    if (t && (!q || !k || !v || !eta || !dO || !dq || !dk || !dv || !deta))
        return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, eta, dO, dq, dk, dv and deta are required");
    const void* p16[] = {q, k, v, dO, dq, dk, dv};
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, dO, dq, dk, dv must be 16-byte aligned");
    const void* p4[] = {eta, S0, dS_out, deta, dS0};
    for (const void* p : p4)
        if (p && !aligned(p, 4)) return fail(TTT_ERR_INVALID_ARGUMENT, "eta, S0, dS_out, deta, dS0 must be 4-byte aligned");
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const size_t qb = t ? (size_t)S * D.N * D.d_k * es : 0, vb = t ? (size_t)S * D.N * D.d_v * es : 0;
    const size_t eb = t ? (size_t)S * D.N * 4 : 0, sb = (size_t)S * D.d_v * D.d_k * 4;
    const struct { const void* p; size_t n; const char* name; } ins[] = {
        {q, qb, "q"}, {k, qb, "k"}, {v, vb, "v"}, {eta, eb, "eta"}, {S0, sb, "S0"}, {dO, vb, "dO"},
        {dS_out, sb, "dS_out"}};
    const struct { const void* p; size_t n; const char* name; } outs[] = {
        {dq, qb, "dq"}, {dk, qb, "dk"}, {dv, vb, "dv"}, {deta, eb, "deta"}, {dS0, sb, "dS0"}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const auto& in : ins)
            if (overlaps(outs[i].p, outs[i].n, in.p, in.n))
                return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps the input %s", outs[i].name, in.name);
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    const size_t need = lin_chunked_bwd_ws_bytes(D);
    if (need && (!workspace || workspace_bytes < need))
        return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (need && !aligned(workspace, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    for (const auto& b : ins)
        if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    for (const auto& b : outs)
        if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    if ((rc = check_buffer(workspace, need, "workspace")) != TTT_OK) return rc;
    uint32_t flags[32] = {};
    if (D.mask == TTT_MASK_STRIDED)
        for (int64_t j = 0; j < cdiv(D.N, D.chunk); ++j)
            if (D.update_chunks[j]) flags[j >> 5] |= 1u << (j & 31);
    hipStream_t st = (hipStream_t)stream;
    const int64_t dvk = (int64_t)D.d_v * D.d_k;
    LinBwdIO io;
    io.S0 = S0;
    io.s0_stride = dvk;
    io.dS_out = dS_out;
    io.dso_stride = dvk;
    io.dS0 = dS0;
    io.ds0_stride = dvk;
    if (D.io_dtype == TTT_BF16)
        return lin_chunked_bwd<uint16_t>(D, flags, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta,
                                         (const uint16_t*)dO, io, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, deta,
                                         (char*)workspace, st);
    return lin_chunked_bwd<float>(D, flags, (const float*)q, (const float*)k, (const float*)v, eta, (const float*)dO,
                                  io, (float*)dq, (float*)dk, (float*)dv, deta, (char*)workspace, st);
}
