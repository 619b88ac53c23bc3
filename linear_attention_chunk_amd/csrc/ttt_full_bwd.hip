// Backward of the TTT-KVB chunk recurrence with all three fast weights learning (GD or GD + L2,
// with or without momentum): the outer-loop gradients of the layer ("TTT with KV Binding Is
// Secretly Linear Attention", Sec. 6.2) through the recurrence of PaperTrace "5.2.1 LaCT and
// TTT-E2E" (Eqs. (2)-(5), the orders of section 1.1).
//
// The forward is run again first and records the weights before every update (and, with the norm,
// each update's row norms).  Then the versions of the weights are walked from the last to the
// first.  Version t has the queries that read it and, for t < T, the update that takes it to t + 1;
// with dW the gradient of version t + 1 (the caller's dW_out at the top):
//   prep  row by row: the norm's transpose (gx = (g - y (y . g)) / |x|), the momentum (the gradient
//         of M is carried: dMi = dM - gx, dM <- beta dMi) and the gradient of the chunk gradient,
//         Gamma = dMi; dW <- gx.  g is dW plus the partial sums the previous version left
//   ops   Gamma and version t as contraction operands, [Gamma1; Gamma3; W1; W3; Gamma2^T; W2^T]
//   up    tiles of tokens x hidden units.  Query tiles: A = q W1^T, C = q W3^T, P = dO W2 on MFMA,
//         the epilogue writes dA | dC and H = SiLU(A) C of the queries.  Key tiles, two passes:
//         A = k W1^T, C = k W3^T, P = v W2 (kept in a per-thread fp32 scratch), then
//         P1 = k Gamma1^T, P3 = k Gamma3^T, R = v Gamma2; the epilogue is the chain rule through the
//         chunk gradient (SiLU'' included) and writes [DA | DC | dA | dC], [H | dE] and -e dE
//   dx    dk = [DA | DC | dA | dC] [Gamma1; Gamma3; W1; W3], dv = -e [H | dE] [Gamma2^T; W2^T] (with
//         the partial sums of deta = -v . that product), dq = [dA | dC] [W1; W3]
//   dw    dW1 | dW3 = [dA | dC]^T x and dW2 = v^T (-e dE) + dO^T H over the version's key and query
//         tokens, split into token parts whose sums the next prep (or the last step) adds to dW
// with e = +-eta (ascent flips the sign).  Names follow the oracle: E = -e P, DA = E C SiLU'(A),
// DC = E SiLU(A), and the gradients of the chunk gradient's inputs are dA, dC, dE.
#include <algorithm>
#include <vector>

#include "host_common.hpp"
#include "tile.hpp"

namespace ttt {

constexpr int kFbWaves = 8;    // up tiles: 8 waves, one workgroup per CU
constexpr int kFbRows = 128;   // token rows per up tile
constexpr int kFbCols = 128;   // hidden units per up tile
constexpr int kFxRows = 256;   // token rows per dx tile
constexpr int kFxCols = 128;   // columns of d per dx tile
constexpr int kFwTile = 128;   // weight-gradient tiles
constexpr int kFbRowVec = 8;   // prep: float4 per lane, rows of up to 2048 elements
constexpr float kFbEps = 1e-6f;
constexpr int kFbMaxUpdates = 1 << 16;  // updates whose weights the backward records

template <typename T> using FbTQ = Tile<T, kFbRows, kFbCols, 2, 4, 1, 2, 2, false, false, false, kFbWaves>;
template <typename T> using FbTP = Tile<T, kFbRows, kFbCols, 2, 4, 1, 1, 1, false, false, false, kFbWaves>;
template <typename T> using FbTX = Tile<T, kFxRows, kFxCols, 2, 4, 1, 1, 1, false, true, false, 4, 1>;
template <typename T> using FbTW13 = Tile<T, kFwTile, kFwTile, 2, 2, 2, 1, 2, true, true, false, 4, 1>;
template <typename T> using FbTW2 = Tile<T, kFwTile, kFwTile, 2, 2, 1, 1, 1, true, true, false, 4, 1>;

// ---------------------------------------------------------------------------------------------
// prep: one wave per row of a scan's [W1; W3; W2] (2m rows of d, then d rows of m)
struct FbPrepArgs {
    float* dW; const float* part; int nparts; int64_t part_stride;  // [S][3dm]; part p at part + p part_stride
    const float* y; const float* nrm;  // norm: the update's output [S][3dm] and its row norms [S][2m + d]
    float* dM; float beta;             // momentum: the gradient of M [S][3dm], or null
    float* G;                          // out: Gamma [S][3dm], or with Muon the gradient of its output
    int d, m, nscan;
    int muon;                          // G <- -gx (Newton-Schulz's backward and k_nsb_final follow)
    int frozen;                        // rows 0 .. frozen-1 (W1, W3 with last_layer_only) do not update
};

__global__ __launch_bounds__(kThreads) void k_fb_prep(FbPrepArgs a) {
    const int lane = threadIdx.x & 63;
    const int rows = 2 * a.m + a.d;
    const int64_t gr = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (gr >= (int64_t)a.nscan * rows) return;  // whole waves; the kernel has no barrier
    const int64_t s = gr / rows;
    const int r = (int)(gr % rows);
    const int64_t dm = (int64_t)a.d * a.m;
    const int L = r < 2 * a.m ? a.d : a.m, nv = L / 4;
    const int64_t off = s * 3 * dm + (r < 2 * a.m ? (int64_t)r * a.d : 2 * dm + (int64_t)(r - 2 * a.m) * a.m);
    f32x4_t g[kFbRowVec];
#pragma unroll
    for (int i = 0; i < kFbRowVec; ++i) {
        const int c = i * 64 + lane;
        g[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (c < nv) {
            g[i] = *reinterpret_cast<const f32x4_t*>(a.dW + off + 4 * c);
            for (int p = 0; p < a.nparts; ++p)
                g[i] += *reinterpret_cast<const f32x4_t*>(a.part + p * a.part_stride + off + 4 * c);
        }
    }
    const bool fz = r < a.frozen;  // uniform per wave
    if (a.y && !fz) {  // the norm's transpose at this update's row
        f32x4_t y[kFbRowVec];
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kFbRowVec; ++i) {
            const int c = i * 64 + lane;
            y[i] = c < nv ? *reinterpret_cast<const f32x4_t*>(a.y + off + 4 * c) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            t += y[i][0] * g[i][0] + y[i][1] * g[i][1] + y[i][2] * g[i][2] + y[i][3] * g[i][3];
        }
        const float yg = wave_sum(t);
        const float n = a.nrm[s * rows + r];
#pragma unroll
        for (int i = 0; i < kFbRowVec; ++i) g[i] = n > kFbEps ? (g[i] - y[i] * yg) * (1.f / n) : g[i] * (1.f / kFbEps);
    }
#pragma unroll
    for (int i = 0; i < kFbRowVec; ++i) {
        const int c = i * 64 + lane;
        if (c < nv) {
            const int64_t e = off + 4 * c;
            f32x4_t dmi = -g[i];
            if (fz) {
                dmi = f32x4_t{0.f, 0.f, 0.f, 0.f};
            } else if (a.dM && !a.muon) {
                dmi += *reinterpret_cast<const f32x4_t*>(a.dM + e);
                *reinterpret_cast<f32x4_t*>(a.dM + e) = a.beta * dmi;
            }
            *reinterpret_cast<f32x4_t*>(a.G + e) = dmi;
            *reinterpret_cast<f32x4_t*>(a.dW + e) = g[i];
        }
    }
}

// ---------------------------------------------------------------------------------------------
// ops: per scan, op = [Gamma1; Gamma3; W1; W3; Gamma2^T; W2^T], six [m][d] blocks in the io type.
// The first part of the grid copies the four [m][d] blocks (4 floats per thread), the rest
// transposes Gamma2 and W2 ([d][m]) in 32 x 32 tiles through LDS.  Without G (no update at this
// version) the Gamma blocks are not written.
template <typename T> struct FbOpsArgs {
    const float* G; const float* W;  // [S][3dm]
    T* op;                           // [S][6dm]
    int d, m, nscan, ncopy, ntr;     // workgroups per scan: copies, transposes
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_fb_ops(FbOpsArgs<T> a) {
    __shared__ float tile[32][33];
    const int per = a.ncopy + a.ntr;
    const int64_t s = blockIdx.x / per;
    const int b = blockIdx.x % per;
    const int64_t dm = (int64_t)a.d * a.m;
    T* op = a.op + s * 6 * dm;
    if (b < a.ncopy) {
        const int64_t i = (int64_t)b * kThreads + threadIdx.x;  // float4 index in [0, dm)
        if (i >= dm) return;
        const int64_t half = dm / 2;  // float4 of two [m][d] blocks
        const bool gam = i < half;
        if (gam && !a.G) return;
        const int64_t e = 4 * (gam ? i : i - half);
        const float4 w = *reinterpret_cast<const float4*>((gam ? a.G : a.W) + s * 3 * dm + e);
        Pack4<T>::store(op + (gam ? 0 : 2 * dm) + e, w.x, w.y, w.z, w.w);
        return;
    }
    const int tt = b - a.ncopy;
    const int per_mat = (a.d / 32) * (a.m / 32);
    const int which = tt / per_mat, t = tt % per_mat;  // 0: Gamma2, 1: W2
    if (which == 0 && !a.G) return;  // uniform per workgroup
    const int i0 = (t / (a.m / 32)) * 32, j0 = (t % (a.m / 32)) * 32;  // rows of d, columns of m
    const float* src = (which == 0 ? a.G : a.W) + s * 3 * dm + 2 * dm;
    {
        const int i = threadIdx.x / 8, j = (threadIdx.x % 8) * 4;
        const float4 w = *reinterpret_cast<const float4*>(src + (int64_t)(i0 + i) * a.m + j0 + j);
        tile[i][j] = w.x;
        tile[i][j + 1] = w.y;
        tile[i][j + 2] = w.z;
        tile[i][j + 3] = w.w;
    }
    __syncthreads();
    const int j = threadIdx.x / 8, i = (threadIdx.x % 8) * 4;
    Pack4<T>::store(op + (4 + which) * dm + (int64_t)(j0 + j) * a.d + i0 + i, tile[i][j], tile[i + 1][j],
                    tile[i + 2][j], tile[i + 3][j]);
}

// ---------------------------------------------------------------------------------------------
// A key tile's first-pass values A, C, P, kept for the second pass's epilogue.  bf16 operands: in
// registers, rounded to bf16 (two values per register; the planes the epilogue writes are bf16
// too).  fp32 operands: in a per-thread fp32 scratch, element idx's value j at ((idx * 3 + j) * NT +
// thread), written and read by the same thread.
template <typename T, int E, int NT> struct KeyKeep;
template <int E, int NT> struct KeyKeep<uint16_t, E, NT> {
    uint32_t ac[E], pp[E / 2];
    __device__ __forceinline__ void begin(float*) {}
    __device__ __forceinline__ void put(int idx, float x, float c, float p) {
        ac[idx] = (uint32_t)f2bf(x) | ((uint32_t)f2bf(c) << 16);
        const uint32_t h = f2bf(p);
        pp[idx / 2] = (idx & 1) ? (pp[idx / 2] & 0xFFFFu) | (h << 16) : h;
    }
    __device__ __forceinline__ void reopen() {}
    __device__ __forceinline__ void get(int idx, float& x, float& c, float& p) const {
        x = __uint_as_float(ac[idx] << 16);
        c = __uint_as_float(ac[idx] & 0xFFFF0000u);
        p = __uint_as_float((idx & 1) ? (pp[idx / 2] & 0xFFFF0000u) : (pp[idx / 2] << 16));
    }
};
template <int E, int NT> struct KeyKeep<float, E, NT> {
    float* sc;
    const float* sr;
    __device__ __forceinline__ void begin(float* base) { sc = base + threadIdx.x; }
    __device__ __forceinline__ void put(int idx, float x, float c, float p) {
        sc[(idx * 3 + 0) * NT] = x;
        sc[(idx * 3 + 1) * NT] = c;
        sc[(idx * 3 + 2) * NT] = p;
    }
    // the epilogue forms its addresses afresh: the pointer is laundered, so that the first pass's
    // 3 E store addresses are not kept live through the second pass
    __device__ __forceinline__ void reopen() {
        sr = sc;
        asm volatile("" : "+v"(sr));
    }
    __device__ __forceinline__ void get(int idx, float& x, float& c, float& p) const {
        x = sr[(idx * 3 + 0) * NT];
        c = sr[(idx * 3 + 1) * NT];
        p = sr[(idx * 3 + 2) * NT];
    }
};

// ---------------------------------------------------------------------------------------------
// up: query tiles and key tiles of one version (token rows x hidden units).  Planes are token-major
// rows of the version's query range (qa: dA | dC, qh: H) or key chunk (pk: DA | DC | dA | dC,
// pv: H | dE, pe: -e dE).
template <typename T> struct FbUpArgs {
    const T* q; const T* k; const T* v; const T* dO; const float* eta;
    const T* op;          // [S][6dm]
    float* acp;           // fp32 operands: the key tiles' first-pass values, 3 x 128 x 128 floats per tile
    T* qa; T* qh;         // [S][qcap][2m], [S][qcap][m]
    T* pk; T* pv; T* pe;  // [S][bcap][4m], [S][bcap][2m], [S][bcap][m]
    int64_t N, qcap, bcap; int d, m;
    int64_t a0; int la;   // query range
    int64_t u0; int lu;   // key chunk
    int nK, nQ, nct;      // tiles per scan; hidden-unit tiles
    float sign;           // -1: gradient ascent
};

template <typename T>
__global__ __launch_bounds__(64 * kFbWaves, 1) void k_fb_up(FbUpArgs<T> a) {
    using TQ = FbTQ<T>;
    using TP = FbTP<T>;
    constexpr int LDSB = std::max(TQ::LDS, TP::LDS);
    __shared__ __attribute__((aligned(16))) char smem[LDSB];
    static_assert(TQ::ELEMS == TP::ELEMS && TQ::FN == TP::FN, "the two tiles share one wave layout");
    const int per = a.nK + a.nQ;
    const int lb = xcd_block(gridDim.x);
    const int s = lb / per, t = lb % per;
    const int64_t dm = (int64_t)a.d * a.m;
    const int m = a.m;
    const T* op = a.op + (int64_t)s * 6 * dm;
    auto blk = [&](int i, int c0) { return op + i * dm + (int64_t)c0 * a.d; };
    TQ tl;
    TP tp;
    auto at = [](int idx, int& i, int& j, int& r) {
        i = idx / (TQ::FN * 16);
        j = (idx / 16) % TQ::FN;
        r = idx % 16;
    };
    if (t < a.nK) {  // key tiles first: they take two passes
        const int r0 = (t / a.nct) * kFbRows, c0 = (t % a.nct) * kFbCols;
        const int rows = a.lu - r0;
        const int64_t tok = (int64_t)s * a.N + a.u0 + r0;
        const Opnd<T> AK[1] = {{a.k + tok * a.d, a.d, rows, a.d}};
        const Opnd<T> AV[1] = {{a.v + tok * a.d, a.d, rows, a.d}};
        {
            const Opnd<T> B1[2] = {{blk(2, c0), a.d, m - c0, a.d}, {blk(3, c0), a.d, m - c0, a.d}};
            const Opnd<T> B2[1] = {{blk(5, c0), a.d, m - c0, a.d}};
            tl.template run<PMQ>(AK, B1, a.d, smem);
            tp.template run<PM1>(AV, B2, a.d, smem);
        }
        KeyKeep<T, TQ::ELEMS, TQ::NT> keep;
        keep.begin(a.acp ? a.acp + ((int64_t)s * a.nK + t) * (3 * TQ::ELEMS * TQ::NT) : nullptr);
        TQ::for_each_pos([&](int idx, int, int) {
            int i, j, r;
            at(idx, i, j, r);
            keep.put(idx, tl.acc[0][i][j][r], tl.acc[1][i][j][r], tp.acc[0][i][j][r]);
        });
        {
            const Opnd<T> B1[2] = {{blk(0, c0), a.d, m - c0, a.d}, {blk(1, c0), a.d, m - c0, a.d}};
            const Opnd<T> B2[1] = {{blk(4, c0), a.d, m - c0, a.d}};
            tl.template run<PMQ>(AK, B1, a.d, smem);
            tp.template run<PM1>(AV, B2, a.d, smem);
        }
        keep.reopen();
        const float* eta = a.eta + tok;
        const int64_t prow = (int64_t)s * a.bcap + r0;
        T* PK = a.pk + prow * 4 * m + c0;
        T* PV = a.pv + prow * 2 * m + c0;
        T* PE = a.pe + prow * m + c0;
        auto epi = [&](auto check) {
            TQ::for_each_pos([&](int idx, int row, int col) {
                if (!decltype(check)::value || (row < rows && c0 + col < m)) {
                    int i, j, r;
                    at(idx, i, j, r);
                    float x, c, p;
                    keep.get(idx, x, c, p);
                    const float p1 = tl.acc[0][i][j][r], p3 = tl.acc[1][i][j][r], rr = tp.acc[0][i][j][r];
                    const float e = a.sign * eta[row];
                    const float sg = sigmoidf_(x), s0 = x * sg, s1 = sg * (1.f + x * (1.f - sg));
                    const float s2 = sg * (1.f - sg) * (2.f + x * (1.f - 2.f * sg));
                    const float E = -e * p, dH = -e * rr;
                    const float dE = p1 * c * s1 + p3 * s0;
                    const float dC = p1 * E * s1 + dH * s0;
                    const float dA = p1 * E * c * s2 + p3 * E * s1 + dH * c * s1;
                    const uint32_t ok = (uint32_t)row * (uint32_t)(4 * m) + (uint32_t)col;
                    PK[ok] = Elt<T>::st(E * c * s1);
                    PK[ok + m] = Elt<T>::st(E * s0);
                    PK[ok + 2 * m] = Elt<T>::st(dA);
                    PK[ok + 3 * m] = Elt<T>::st(dC);
                    const uint32_t ov = (uint32_t)row * (uint32_t)(2 * m) + (uint32_t)col;
                    PV[ov] = Elt<T>::st(s0 * c);
                    PV[ov + m] = Elt<T>::st(dE);
                    PE[(uint32_t)row * (uint32_t)m + (uint32_t)col] = Elt<T>::st(-e * dE);
                }
            });
        };
        if (r0 + kFbRows <= a.lu && c0 + kFbCols <= m) epi(std::false_type{});
        else epi(std::true_type{});
        return;
    }
    // query tiles
    const int tq = t - a.nK;
    const int r0 = (tq / a.nct) * kFbRows, c0 = (tq % a.nct) * kFbCols;
    const int rows = a.la - r0;
    const int64_t tok = (int64_t)s * a.N + a.a0 + r0;
    const Opnd<T> AQ[1] = {{a.q + tok * a.d, a.d, rows, a.d}};
    const Opnd<T> AO[1] = {{a.dO + tok * a.d, a.d, rows, a.d}};
    const Opnd<T> B1[2] = {{blk(2, c0), a.d, m - c0, a.d}, {blk(3, c0), a.d, m - c0, a.d}};
    const Opnd<T> B2[1] = {{blk(5, c0), a.d, m - c0, a.d}};
    tl.template run<PMQ>(AQ, B1, a.d, smem);
    tp.template run<PM1>(AO, B2, a.d, smem);
    const int64_t prow = (int64_t)s * a.qcap + r0;
    T* QA = a.qa + prow * 2 * m + c0;
    T* QH = a.qh + prow * m + c0;
    auto epi = [&](auto check) {
        TQ::for_each_pos([&](int idx, int row, int col) {
            if (!decltype(check)::value || (row < rows && c0 + col < m)) {
                int i, j, r;
                at(idx, i, j, r);
                const float x = tl.acc[0][i][j][r], c = tl.acc[1][i][j][r], p = tp.acc[0][i][j][r];
                const float sg = sigmoidf_(x), s0 = x * sg, s1 = sg * (1.f + x * (1.f - sg));
                const uint32_t oa = (uint32_t)row * (uint32_t)(2 * m) + (uint32_t)col;
                QA[oa] = Elt<T>::st(p * c * s1);
                QA[oa + m] = Elt<T>::st(p * s0);
                QH[(uint32_t)row * (uint32_t)m + (uint32_t)col] = Elt<T>::st(s0 * c);
            }
        });
    };
    if (r0 + kFbRows <= a.la && c0 + kFbCols <= m) epi(std::false_type{});
    else epi(std::true_type{});
}

// ---------------------------------------------------------------------------------------------
// dx: tiles of 256 tokens x 128 columns of d, contracting over hidden units with the op blocks read
// k-strided.  Jobs: dk (key chunk, K = 4m over op blocks 0-3), dv (K = 2m over blocks 4-5, with
// deta's partial sums), dq (query range, K = 2m over blocks 2-3).  With several inner steps the key
// chunk's dk and dv collect in fp32 (kmode 1: first, 2: add, 3: last, written with the sum).
template <typename T> struct FbDxArgs {
    const T* pk; const T* pv; const T* qa; const T* op;
    const T* v; const float* eta;
    T* dk; T* dv; T* dq;                 // [S][N][d]
    float* acck; float* accv;            // [S][bcap][d]
    float* epart;                        // [ntd][S][bcap]
    int64_t N, qcap, bcap; int d, m, nscan;
    int64_t a0; int la; int64_t u0; int lu;
    int ntu, nta, ntd;                   // token tiles of the key chunk and of the query range; column tiles
    int kmode;                           // 0: write dk, dv; 1: acc = g; 2: acc += g; 3: write acc + g
    float sign;
};

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_fb_dx(FbDxArgs<T> a) {
    using TX = FbTX<T>;
    static_assert(TX::RV_LDS <= TX::LDS && TX::BN / 4 == 32, "row bands fit the LDS; 32 lanes per row");
    __shared__ __attribute__((aligned(16))) char smem[TX::LDS];
    const int lb = xcd_block(gridDim.x);
    const int nk = a.nscan * a.ntu * a.ntd;
    int job, l;
    if (lb < 2 * nk) {
        job = lb / nk;
        l = lb % nk;
    } else {
        job = 2;
        l = lb - 2 * nk;
    }
    const int nt = job < 2 ? a.ntu : a.nta;
    const int s = l / (nt * a.ntd), t = l % (nt * a.ntd);
    const int r0 = (t / a.ntd) * kFxRows, ct = t % a.ntd, c0 = ct * kFxCols;
    const int64_t dm = (int64_t)a.d * a.m;
    const int m = a.m;
    const int len = job < 2 ? a.lu : a.la;
    const int rows = len - r0;
    const T* op = a.op + (int64_t)s * 6 * dm + c0;
    const int K = job == 0 ? 4 * m : 2 * m;
    const T* Ap = job == 0 ? a.pk + ((int64_t)s * a.bcap + r0) * 4 * m
                : job == 1 ? a.pv + ((int64_t)s * a.bcap + r0) * 2 * m
                           : a.qa + ((int64_t)s * a.qcap + r0) * 2 * m;
    const Opnd<T> A[1] = {{Ap, K, rows, K}};
    const Opnd<T> B[1] = {{op + (job == 0 ? 0 : job == 1 ? 4 * dm : 2 * dm), a.d, a.d - c0, K}};
    TX tl;
    tl.template run<PM1>(A, B, K, smem);
    const int64_t tok = (int64_t)s * a.N + (job < 2 ? a.u0 : a.a0) + r0;  // first token of the tile
    const int64_t arow = (int64_t)s * a.bcap + r0;                        // its row in the accumulators
    const int cols = a.d - c0;
    if (job == 2) {
        T* O = a.dq + tok * a.d + c0;
        tl.template rows_via_lds<1>(smem, [&](int, int, int row, int col, const float4& g) {
            if (row < rows && col < cols) Pack4<T>::store(O + (uint32_t)row * (uint32_t)a.d + (uint32_t)col, g.x, g.y, g.z, g.w);
        });
        return;
    }
    T* O = (job == 0 ? a.dk : a.dv) + tok * a.d + c0;
    float* acc = (job == 0 ? a.acck : a.accv);
    acc = acc ? acc + arow * a.d + c0 : nullptr;
    const T* V = a.v + tok * a.d + c0;
    const float* eta = a.eta + tok;
    float* ep = job == 1 ? a.epart + ((int64_t)ct * a.nscan + s) * a.bcap + r0 : nullptr;
    tl.template rows_via_lds<1>(smem, [&](int, int, int row, int col, const float4& g) {
        const bool in = row < rows && col < cols;
        float x[4] = {g.x, g.y, g.z, g.w};
        float pd = 0.f;
        if (in && job == 1) {  // dv = -e dDf, deta's part -v . dDf
            const float e = a.sign * eta[row];
            float vv[4];
            Pack4<T>::unpack(Pack4<T>::load_raw(V + (uint32_t)row * (uint32_t)a.d + (uint32_t)col), vv);
            pd = -(vv[0] * x[0] + vv[1] * x[1] + vv[2] * x[2] + vv[3] * x[3]);
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] *= -e;
        }
        if (in) {
            const uint32_t off = (uint32_t)row * (uint32_t)a.d + (uint32_t)col;
            if (a.kmode == 0) {
                Pack4<T>::store(O + off, x[0], x[1], x[2], x[3]);
            } else {
                f32x4_t* ap = reinterpret_cast<f32x4_t*>(acc + off);
                const f32x4_t xv = {x[0], x[1], x[2], x[3]};
                if (a.kmode == 1) {
                    *ap = xv;
                } else if (a.kmode == 2) {
                    *ap += xv;
                } else {
                    const f32x4_t y = *ap + xv;
                    Pack4<T>::store(O + off, y[0], y[1], y[2], y[3]);
                }
            }
        }
        if (job == 1) {  // the 32 lanes that hold this row's pieces (uniform per workgroup)
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) pd += __shfl_xor(pd, o, 64);
            if ((threadIdx.x & 31) == 0 && row < rows) ep[row] = pd;
        }
    });
}

// deta of the key chunk: the column tiles' partial sums, times the update's sign; first (the last
// inner step, walked first) writes, the others add
__global__ __launch_bounds__(kThreads) void k_fb_deta(const float* epart, float* deta, int64_t N, int64_t u0, int lu,
                                                      int64_t bcap, int nscan, int ntd, float sign, int add) {
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= (int64_t)nscan * lu) return;
    const int64_t s = g / lu;
    const int i = (int)(g % lu);
    float x = 0.f;
    for (int c = 0; c < ntd; ++c) x += epart[((int64_t)c * nscan + s) * bcap + i];
    float* o = deta + s * N + u0 + i;
    *o = add ? *o + sign * x : sign * x;
}

// ---------------------------------------------------------------------------------------------
// dw: weight-gradient partial sums over the version's tokens.  Positions 0 .. lu-1 are the key
// chunk's tokens, lu .. lu+la-1 the query range's; part p takes [p lp, (p + 1) lp) and writes the
// whole [3dm] block of its scan in partial buffer p.  G13 tiles (m x d): dW1 | dW3 = [dA | dC]^T x;
// G2 tiles (d x m): dW2 = v^T (-e dE) + dO^T H.
template <typename T> struct FbDwArgs {
    const T* pk; const T* pe; const T* qa; const T* qh;
    const T* k; const T* v; const T* q; const T* dO;
    float* part;                         // [nparts][S][3dm]
    int64_t N, qcap, bcap, part_stride; int d, m;
    int64_t a0; int la; int64_t u0; int lu;
    int nparts, lp, ntm, ntd;
};

template <typename T, int JOB>  // JOB 0: the G13 tiles, 1: the G2 tiles
__global__ __launch_bounds__(kThreads, 2) void k_fb_dw(FbDwArgs<T> a) {
    using TW = FbTW13<T>;
    using TV = FbTW2<T>;
    constexpr int LDSB = JOB == 0 ? TW::LDS : TV::LDS;
    static_assert(TW::RV_LDS <= TW::LDS && TV::RV_LDS <= TV::LDS, "row bands fit the LDS");
    static_assert(TW::KSTEP == TV::KSTEP, "one stage length");
    __shared__ __attribute__((aligned(16))) char smem[LDSB];
    const int n13 = a.ntm * a.ntd, per = n13;
    const int lb = xcd_block(gridDim.x);
    const int u = lb / per, t = lb % per + (JOB == 0 ? 0 : n13);
    const int s = u / a.nparts, p = u % a.nparts;
    const int64_t dm = (int64_t)a.d * a.m;
    const int m = a.m;
    const int total = a.lu + a.la;
    const int lo = std::min(p * a.lp, total), hi = std::min(lo + a.lp, total);
    float* out = a.part + p * a.part_stride + (int64_t)s * 3 * dm;
    // a part's segments lie in the key chunk, then the query range; all full stages over full tiles
    // take the unmasked loads (one variant per workgroup)
    const bool aligned_k = a.lu % TW::KSTEP == 0 && a.la % TW::KSTEP == 0 && a.lp % TW::KSTEP == 0;
    if constexpr (JOB == 0) {
        const int r0 = (t / a.ntd) * kFwTile, c0 = (t % a.ntd) * kFwTile;
        TW tl;
        tl.zero();
        auto segments = [&](auto full) {
            for (int pos = lo; pos < hi;) {
                const bool key = pos < a.lu;
                const int t0 = key ? pos : pos - a.lu;
                const int kl = key ? std::min(a.lu, hi) - pos : hi - pos;
                const T* G = key ? a.pk + ((int64_t)s * a.bcap + t0) * 4 * m + 2 * m
                                 : a.qa + ((int64_t)s * a.qcap + t0) * 2 * m;
                const int ld = key ? 4 * m : 2 * m;
                const T* X = (key ? a.k + ((int64_t)s * a.N + a.u0 + t0) * a.d : a.q + ((int64_t)s * a.N + a.a0 + t0) * a.d);
                const Opnd<T> A[2] = {{G + r0, ld, m - r0, kl}, {G + m + r0, ld, m - r0, kl}};
                const Opnd<T> B[1] = {{X + c0, a.d, a.d - c0, kl}};
                if (pos > lo) lds_barrier();  // every wave is done with the previous segment's last stage
                tl.template run_<PMG, decltype(full)::value>(A, B, kl, smem, true);
                pos += kl;
            }
        };
        const bool fullt = r0 + TW::BM <= m && c0 + TW::BN <= a.d;
        if (fullt && aligned_k) segments(std::true_type{});
        else segments(std::false_type{});
        float* G1 = out + (int64_t)r0 * a.d + c0;
        float* G3 = G1 + dm;
        if (fullt) {
            tl.rows_via_lds(smem, [&](int, int q, int row, int col, const float4& v) {
                *reinterpret_cast<float4*>((q ? G3 : G1) + (uint32_t)row * (uint32_t)a.d + (uint32_t)col) = v;
            });
        } else {
            tl.for_each([&](const float (&v)[2], int row, int col) {
                if (r0 + row < m && c0 + col < a.d) {
                    const uint32_t off = (uint32_t)row * (uint32_t)a.d + (uint32_t)col;
                    G1[off] = v[0];
                    G3[off] = v[1];
                }
            });
        }
        return;
    } else {
    const int t2 = t - n13;
    const int r0 = (t2 / a.ntm) * kFwTile, c0 = (t2 % a.ntm) * kFwTile;  // rows of d, columns of m
    TV tl;
    tl.zero();
    auto segments = [&](auto full) {
        for (int pos = lo; pos < hi;) {
            const bool key = pos < a.lu;
            const int t0 = key ? pos : pos - a.lu;
            const int kl = key ? std::min(a.lu, hi) - pos : hi - pos;
            const T* X = key ? a.v + ((int64_t)s * a.N + a.u0 + t0) * a.d : a.dO + ((int64_t)s * a.N + a.a0 + t0) * a.d;
            const T* G = key ? a.pe + ((int64_t)s * a.bcap + t0) * m : a.qh + ((int64_t)s * a.qcap + t0) * m;
            const Opnd<T> A[1] = {{X + r0, a.d, a.d - r0, kl}};
            const Opnd<T> B[1] = {{G + c0, m, m - c0, kl}};
            if (pos > lo) lds_barrier();
            tl.template run_<PM1, decltype(full)::value>(A, B, kl, smem, true);
            pos += kl;
        }
    };
    const bool fullt = r0 + TV::BM <= a.d && c0 + TV::BN <= m;
    if (fullt && aligned_k) segments(std::true_type{});
    else segments(std::false_type{});
    float* G2 = out + 2 * dm + (int64_t)r0 * m + c0;
    if (fullt) {
        tl.rows_via_lds(smem, [&](int, int, int row, int col, const float4& v) {
            *reinterpret_cast<float4*>(G2 + (uint32_t)row * (uint32_t)m + (uint32_t)col) = v;
        });
    } else {
        tl.for_each([&](const float (&v)[1], int row, int col) {
            if (r0 + row < a.d && c0 + col < m) G2[(uint32_t)row * (uint32_t)m + (uint32_t)col] = v[0];
        });
    }
    }
}

// ---------------------------------------------------------------------------------------------
// Newton-Schulz walked back (Muon) for every scan's learned matrices at once.  With X the iterate of
// a step and G the gradient of its output, the gradient of its input is
//   wide X (rows <= columns):  1.5 G - 0.5 [(Q + Q^T) X + (X X^T) G],  Q = G X^T
//   tall X:                    1.5 G - 0.5 [G (X^T X) + X (Q + Q^T)],  Q = G^T X
// (the forward steps on the side with the smaller Gram matrix, as the tall form does transposed).
// k_nsb_q writes Q + Q^T, k_nsb_step the new gradient (to the other buffer: every tile reads G), and
// the start X_0 = U / (|U| + 1e-7) is taken back by k_nsb_dot and k_nsb_final.  G is carried in fp32;
// the products take T operands (bf16: G's bf16 shadow, the iterates' hi planes and bf16 Gram
// matrices, as the forward's steps take them; fp32: the fp32 values themselves).
struct PMD { static constexpr int a[2] = {0, 1}; static constexpr int b[2] = {0, 1}; };
constexpr int kNsbQ = 64;                      // Q tiles
constexpr int kNsbRows = 128, kNsbCols = 64;   // step tiles
constexpr int kNsbElems = 4096;                // elements per block of the elementwise kernels

template <typename T> struct NsbArgs {
    const float* G; const T* Gs;     // the gradient [S][3dm] (fp32) and its operand copy
    float* Gout; T* Gsout;           // the next gradient and its operand copy (fp32: the same buffer)
    const T* X;                      // the step's iterate [S][3dm]
    const T* P;                      // its Gram matrix [S][3 p^2]
    T* Q;                            // Q + Q^T [S][3 p^2]
    int d, m, mat0, nmat, tiles;     // tiles per matrix
};

// one LDS stage (37 KB), so that four workgroups share a CU and hide each other's pipeline fill
template <typename T>
__global__ __launch_bounds__(kThreads, 4) void k_nsb_q(NsbArgs<T> a) {
    using TW = Tile<T, kNsbQ, kNsbQ, 2, 2, 2, 2, 2, false, false, false, 4, 1>;
    using TT = Tile<T, kNsbQ, kNsbQ, 2, 2, 2, 2, 2, true, true, false, 4, 1>;
    constexpr int LDSB = std::max(TW::LDS, TT::LDS);
    __shared__ __attribute__((aligned(16))) char smem[LDSB];
    const int per = a.nmat * a.tiles;
    const int lb = xcd_block(gridDim.x);
    const int s = lb / per;
    int t = lb % per;
    const int mat = a.mat0 + t / a.tiles;
    t %= a.tiles;
    const int r = mat < 2 ? a.m : a.d, c = mat < 2 ? a.d : a.m;
    const int p = std::min(r, c), np = (p + kNsbQ - 1) / kNsbQ;
    // Q + Q^T is symmetric: only tiles on or above the diagonal are computed (tile t of np (np + 1) / 2,
    // row-major over the upper triangle), and an off-diagonal tile also writes its mirror block
    int ti = 0;
    while (t >= np - ti) t -= np - ti++;  // uniform: row ti of the upper triangle, column ti + t
    const int i0 = ti * kNsbQ, j0 = (ti + t) * kNsbQ;
    const int64_t dm = (int64_t)a.d * a.m;
    const T* G = a.Gs + (int64_t)s * 3 * dm + mat * dm;
    const T* X = a.X + (int64_t)s * 3 * dm + mat * dm;
    T* Q = a.Q + ((int64_t)s * 3 + mat) * p * p;
    auto out = [&](auto& tl) {
        tl.for_each([&](const float (&v)[2], int row, int col) {
            if (i0 + row < p && j0 + col < p) {
                const T x = Elt<T>::st(v[0] + v[1]);
                Q[(int64_t)(i0 + row) * p + j0 + col] = x;
                if (i0 != j0) Q[(int64_t)(j0 + col) * p + i0 + row] = x;
            }
        });
    };
    if (r <= c) {  // Q = G X^T over the columns: rows of G and X are k-contiguous
        TW tl;
        const Opnd<T> A[2] = {{G + (int64_t)i0 * c, c, p - i0, c}, {X + (int64_t)i0 * c, c, p - i0, c}};
        const Opnd<T> B[2] = {{X + (int64_t)j0 * c, c, p - j0, c}, {G + (int64_t)j0 * c, c, p - j0, c}};
        tl.template run<PMD>(A, B, c, smem);
        out(tl);
    } else {       // Q = G^T X over the rows: columns of G and X, k-strided
        TT tl;
        const Opnd<T> A[2] = {{G + i0, c, p - i0, r}, {X + i0, c, p - i0, r}};
        const Opnd<T> B[2] = {{X + j0, c, p - j0, r}, {G + j0, c, p - j0, r}};
        tl.template run<PMD>(A, B, r, smem);
        out(tl);
    }
}

// FULL: every tile lies inside its matrix (d and m multiples of 128); the tiles then take one LDS
// stage and four workgroups share a CU, so that one workgroup's pipeline fill and epilogue overlap
// the others' contractions (the forward's Newton-Schulz step does the same)
template <typename T, bool FULL>
__global__ __launch_bounds__(kThreads, FULL ? 4 : 2) void k_nsb_step(NsbArgs<T> a) {
    using TW = Tile<T, kNsbRows, kNsbCols, 2, 2, 1, 1, 1, false, true, false, 4, FULL ? 1 : 2>;   // B k-strided
    using TT = Tile<T, kNsbRows, kNsbCols, 2, 2, 1, 1, 1, false, false, false, 4, FULL ? 1 : 2>;  // B symmetric rows
    constexpr int LDSB = std::max(TW::LDS, TT::LDS);
    __shared__ __attribute__((aligned(16))) char smem[LDSB];
    const int per = a.nmat * a.tiles;
    const int lb = xcd_block(gridDim.x);
    const int s = lb / per;
    int t = lb % per;
    const int mat = a.mat0 + t / a.tiles;
    t %= a.tiles;
    const int r = mat < 2 ? a.m : a.d, c = mat < 2 ? a.d : a.m;
    const int p = std::min(r, c);
    const int nct = (c + kNsbCols - 1) / kNsbCols;
    const int r0 = (t / nct) * kNsbRows, c0 = (t % nct) * kNsbCols;
    if (r0 >= r) return;  // uniform: tiles covers the larger of the two orientations
    const int64_t dm = (int64_t)a.d * a.m, mo = (int64_t)s * 3 * dm + mat * dm;
    const float* G = a.G + mo;
    const T* Gs = a.Gs + mo;
    const T* X = a.X + mo;
    const T* P = a.P + ((int64_t)s * 3 + mat) * p * p;
    const T* Q = a.Q + ((int64_t)s * 3 + mat) * p * p;
    float* O = a.Gout + mo;
    T* Os = a.Gsout + mo;
    auto out = [&](auto& tl) {
        tl.for_each([&](const float (&v)[1], int row, int col) {
            if (FULL || (r0 + row < r && c0 + col < c)) {
                const int64_t e = (int64_t)(r0 + row) * c + c0 + col;
                const float x = 1.5f * G[e] - 0.5f * v[0];
                O[e] = x;
                if constexpr (sizeof(T) == 2) Os[e] = Elt<T>::st(x);
            }
        });
    };
    if (r <= c) {  // (Q + Q^T) X + P G: B is X or G read k-strided
        TW tl;
        const Opnd<T> A0[1] = {{Q + (int64_t)r0 * p, p, r - r0, p}};
        const Opnd<T> B0[1] = {{X + c0, c, c - c0, r}};
        const Opnd<T> A1[1] = {{P + (int64_t)r0 * p, p, r - r0, p}};
        const Opnd<T> B1[1] = {{Gs + c0, c, c - c0, r}};
        tl.template run<PM1>(A0, B0, r, smem);
        if (FULL) lds_barrier();  // one LDS stage: every wave is done with the first product's last stage
        tl.template run<PM1>(A1, B1, r, smem, true);
        out(tl);
    } else {       // G P + X (Q + Q^T): P and Q + Q^T are symmetric, so their rows serve as B
        TT tl;
        const Opnd<T> A0[1] = {{Gs + (int64_t)r0 * c, c, r - r0, c}};
        const Opnd<T> B0[1] = {{P + (int64_t)c0 * p, p, c - c0, p}};
        const Opnd<T> A1[1] = {{X + (int64_t)r0 * c, c, r - r0, c}};
        const Opnd<T> B1[1] = {{Q + (int64_t)c0 * p, p, c - c0, p}};
        tl.template run<PM1>(A0, B0, c, smem);
        if (FULL) lds_barrier();  // one LDS stage: every wave is done with the first product's last stage
        tl.template run<PM1>(A1, B1, c, smem, true);
        out(tl);
    }
}

// X_0 = U / (|U| + 1e-7) as the steps' operand (bf16: hi plane to X, lo plane to Xlo), and with
// Gs the operand copy of the fp32 gradient G, for the learned matrices; pu holds U's partial sums
template <typename T>
__global__ __launch_bounds__(kThreads) void k_nsb_x0(const float* U, const float* pu, T* X, T* Xlo, const float* G,
                                                     T* Gs, int64_t dm, int mat0, int nmat, int nblk) {
    const int per = nmat * nblk;
    const int s = blockIdx.x / per, t = blockIdx.x % per;
    const int mat = mat0 + t / nblk, blk = t % nblk;
    float su = 0.f;
    for (int i = threadIdx.x & 63; i < nblk; i += 64) su += pu[((int64_t)s * 3 + mat) * nblk + i];
    const float inv = 1.0f / (sqrtf(wave_sum(su)) + 1e-7f);
    const int64_t mo = (int64_t)s * 3 * dm + mat * dm;
    for (int64_t e = (int64_t)blk * kNsbElems + threadIdx.x; e < std::min<int64_t>((int64_t)(blk + 1) * kNsbElems, dm);
         e += kThreads) {
        const float x = U[mo + e] * inv;
        const T h = Elt<T>::st(x);
        X[mo + e] = h;
        if constexpr (sizeof(T) == 2) {
            Xlo[mo + e] = f2bf(x - bf2f(h));
            Gs[mo + e] = f2bf(G[mo + e]);
        }
    }
}

// partial sums of <G, U> per block of 4096 elements of each learned matrix
__global__ __launch_bounds__(kThreads) void k_nsb_dot(const float* G, const float* U, float* part, int64_t dm,
                                                      int mat0, int nmat, int nblk) {
    __shared__ float red[4];
    const int per = nmat * nblk;
    const int s = blockIdx.x / per, t = blockIdx.x % per;
    const int mat = mat0 + t / nblk, blk = t % nblk;
    const int64_t mo = (int64_t)s * 3 * dm + mat * dm;
    float x = 0.f;
    for (int64_t e = (int64_t)blk * kNsbElems + threadIdx.x; e < std::min<int64_t>((int64_t)(blk + 1) * kNsbElems, dm);
         e += kThreads)
        x += G[mo + e] * U[mo + e];
    x = wave_sum(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) part[((int64_t)s * 3 + mat) * nblk + blk] = red[0] + red[1] + red[2] + red[3];
}

// dU = G / (n + eps) - <G, U> U / ((n + eps)^2 n) (n = |U|, the second term absent at n = 0), then the
// momentum: dMi = dM + dU, Gamma = dMi, dM <- beta dMi (dM null: Gamma = dU)
struct NsbFinalArgs {
    const float* G; const float* U; const float* pu; const float* pgu;  // partial sums of U^2 and <G, U>
    float* Gamma; float* dM; float beta;
    int64_t dm; int mat0, nmat, nblk;
};

__global__ __launch_bounds__(kThreads) void k_nsb_final(NsbFinalArgs a) {
    const int per = a.nmat * a.nblk;
    const int s = blockIdx.x / per, t = blockIdx.x % per;
    const int mat = a.mat0 + t / a.nblk, blk = t % a.nblk;
    const int64_t pb = ((int64_t)s * 3 + mat) * a.nblk;
    float su = 0.f, sgu = 0.f;
    for (int i = threadIdx.x & 63; i < a.nblk; i += 64) {
        su += a.pu[pb + i];
        sgu += a.pgu[pb + i];
    }
    const float n = sqrtf(wave_sum(su)), gu = wave_sum(sgu);
    const float inv = 1.0f / (n + 1e-7f);
    const float k2 = n > 0.f ? gu * inv * inv / n : 0.f;
    const int64_t mo = (int64_t)s * 3 * a.dm + mat * a.dm;
    for (int64_t e = (int64_t)blk * kNsbElems + threadIdx.x; e < std::min<int64_t>((int64_t)(blk + 1) * kNsbElems, a.dm);
         e += kThreads) {
        float du = a.G[mo + e] * inv - k2 * a.U[mo + e];
        if (a.dM) {
            du += a.dM[mo + e];
            a.dM[mo + e] = a.beta * du;
        }
        a.Gamma[mo + e] = du;
    }
}

// ---------------------------------------------------------------------------------------------
// small kernels: dW <- dW_out (or zero) and dM <- 0; zero rows of the token gradients of chunks
// that do not update; dW0 of each weight block from dW and the pending parts (fixed order)
__global__ __launch_bounds__(kThreads) void k_fb_init(float* dW, const float* dWo, float* dM, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(dW)[i] = dWo ? reinterpret_cast<const float4*>(dWo)[i] : z;
    if (dM) reinterpret_cast<float4*>(dM)[i] = z;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_fb_zero_rows(T* dk, T* dv, float* deta, int64_t N, int64_t lo, int len,
                                                           int d, int nscan) {
    const int64_t per = (int64_t)len * (d / 4);
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= per * nscan) return;
    const int64_t s = g / per, e = g % per;
    const int64_t row = s * N + lo + e / (d / 4);
    const int64_t off = row * d + (e % (d / 4)) * 4;
    Pack4<T>::store(dk + off, 0.f, 0.f, 0.f, 0.f);
    Pack4<T>::store(dv + off, 0.f, 0.f, 0.f, 0.f);
    if (e % (d / 4) == 0) deta[row] = 0.f;
}

struct FbFinalArgs {
    const float* dW; const float* part; int nparts; int64_t part_stride;
    float* dW0;
    int nw, nb, H, per_head;
    int64_t dm3;
};

__global__ __launch_bounds__(kThreads) void k_fb_final(FbFinalArgs a) {
    const int64_t per = a.dm3 / 4;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= per * a.nw) return;
    const int hw = (int)(g / per);
    const int64_t e = (g % per) * 4;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < a.nb; ++b) {
        const int64_t s = a.per_head ? (int64_t)b * a.H + hw : hw;
        f32x4_t x = *reinterpret_cast<const f32x4_t*>(a.dW + s * a.dm3 + e);
        for (int p = 0; p < a.nparts; ++p) x += *reinterpret_cast<const f32x4_t*>(a.part + p * a.part_stride + s * a.dm3 + e);
        acc += x;
    }
    *reinterpret_cast<f32x4_t*>(a.dW0 + (int64_t)hw * a.dm3 + e) = acc;
}

// ---------------------------------------------------------------------------------------------
// host driver

// The versions of the weights and what reads them, from the descriptor alone: update i is a step
// of chunk step_chunk[i] (its step_it[i]-th inner step); version v (0 .. T) is read by the queries
// of the token range [qlo[v], qhi[v]) (empty when qlo == qhi): the chunks that read one version are
// consecutive.
struct FbPlan {
    std::vector<int> step_chunk, step_it;
    std::vector<int64_t> qlo, qhi;
    int T = 0, nin = 1;
    int64_t qcap = 0;
};

static FbPlan fb_plan(const ttt_desc& D) {
    FbPlan P;
    P.nin = std::max(1, D.inner_steps);
    const int64_t nc = D.N > 0 ? cdiv(D.N, D.chunk) : 0;
    const bool first = D.mask == TTT_MASK_APPLY_THEN_UPDATE || D.mask == TTT_MASK_STRIDED;
    std::vector<int64_t> lo(1, -1), hi(1, -1);
    auto read = [&](int v, int64_t a, int64_t b) {
        if (lo[v] < 0) lo[v] = a;
        hi[v] = b;  // contiguous: each chunk that reads v follows the previous one
    };
    for (int64_t j = 0; j < nc; ++j) {
        const int64_t a = j * D.chunk, b = std::min<int64_t>(a + D.chunk, D.N);
        const bool upd = D.mask != TTT_MASK_STRIDED || D.update_chunks[j];
        if (first) read(P.T, a, b);
        if (upd)
            for (int it = 0; it < P.nin; ++it) {
                P.step_chunk.push_back((int)j);
                P.step_it.push_back(it);
                ++P.T;
                lo.push_back(-1);
                hi.push_back(-1);
            }
        if (!first) read(P.T, a, b);
    }
    P.qlo.resize(P.T + 1);
    P.qhi.resize(P.T + 1);
    for (int v = 0; v <= P.T; ++v) {
        P.qlo[v] = lo[v] < 0 ? 0 : lo[v];
        P.qhi[v] = lo[v] < 0 ? 0 : hi[v];
        P.qcap = std::max(P.qcap, P.qhi[v] - P.qlo[v]);
    }
    return P;
}

// Token parts of the weight-gradient launch: the count in 1 .. 8 whose launch (tiles x parts
// workgroups, two per CU on 256 CUs) leaves the least idle share in its last round, every part at
// least 1024 positions long; ties go to fewer parts.
static int fb_parts(int64_t tiles, int64_t total) {
    int best = 1;
    double best_eff = 0.0;
    for (int p = 1; p <= 8; ++p) {
        if (p > 1 && total / p < 1024) break;
        const int64_t n = tiles * p, rounds = cdiv(n, 512);
        const double eff = (double)n / (double)(rounds * 512);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = p;
        }
    }
    return best;
}

// The record of a forward (the weights before every update and after the last, fp32; with the norm
// every update's row norms; with Muon every update's U), as offsets into one buffer
struct FRecord {
    size_t hist, nrm, urec, total;
};

static FRecord record_layout(const ttt_desc& D, const FbPlan& P) {
    FRecord R{};
    const int64_t S = (int64_t)D.B * D.H, d = D.d_h, m = D.m_h, dm = d * m;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    R.hist = take((size_t)(P.T + 1) * S * 3 * dm * 4);
    if (D.rule == TTT_UPD_GD_L2 || D.rule == TTT_UPD_MUON_L2) R.nrm = take((size_t)P.T * S * (2 * m + d) * 4);
    if (D.rule == TTT_UPD_MUON || D.rule == TTT_UPD_MUON_L2) R.urec = take((size_t)P.T * S * 3 * dm * 4);
    R.total = off;
    return R;
}

struct FLayout {
    size_t fwd, rec, dW, dM, G, op, acp, qa, qh, pk, pv, pe, acck, accv, epart, part, total;
    size_t nsx, nsxl, gs[2], nsp, nsq, gb, pu, pgu;  // Muon: iterates (and lo plane), G's operand copies,
                                                      // Grams, Q + Q^T, G's pair, partial sums
    int nparts, nK;
    int64_t bcap, qcap;
};

// own_record: the workspace holds the forward's workspace and the record (else the caller's record)
static FLayout make_flayout(const ttt_desc& D, const FbPlan& P, bool own_record) {
    FLayout L{};
    const int64_t S = (int64_t)D.B * D.H, d = D.d_h, m = D.m_h, dm = d * m;
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    L.bcap = D.N < D.chunk ? D.N : D.chunk;
    L.qcap = P.qcap;
    L.nK = (int)(cdiv(L.bcap, kFbRows) * cdiv(m, kFbCols));
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    if (own_record) {
        L.fwd = take(ttt_history_ws_bytes(D));
        L.rec = take(record_layout(D, P).total);
    }
    L.dW = take((size_t)S * 3 * dm * 4);
    if (D.momentum != 0.0f) L.dM = take((size_t)S * 3 * dm * 4);
    L.G = take((size_t)S * 3 * dm * 4);
    L.op = take((size_t)S * 6 * dm * es);
    if (P.T > 0) {
        if (es == 4) L.acp = take((size_t)S * L.nK * 3 * FbTQ<float>::ELEMS * FbTQ<float>::NT * 4);
        L.pk = take((size_t)S * L.bcap * 4 * m * es);
        L.pv = take((size_t)S * L.bcap * 2 * m * es);
        L.pe = take((size_t)S * L.bcap * m * es);
        if (P.nin > 1) {
            L.acck = take((size_t)S * L.bcap * d * 4);
            L.accv = take((size_t)S * L.bcap * d * 4);
        }
        L.epart = take((size_t)cdiv(d, kFxCols) * S * L.bcap * 4);
    }
    if (L.qcap > 0) {
        L.qa = take((size_t)S * L.qcap * 2 * m * es);
        L.qh = take((size_t)S * L.qcap * m * es);
    }
    const int64_t tiles = S * 2 * cdiv(m, kFwTile) * cdiv(d, kFwTile);
    L.nparts = fb_parts(tiles, (P.T > 0 ? L.bcap : 0) + L.qcap);
    L.part = take((size_t)L.nparts * S * 3 * dm * 4);
    if (D.rule == TTT_UPD_MUON || D.rule == TTT_UPD_MUON_L2) {
        const int64_t p = std::min(d, m), nblk = cdiv(dm, kNsbElems);
        L.nsx = take((size_t)std::max(D.ns_iters, 1) * S * 3 * dm * es);
        if (es == 2) {
            L.nsxl = take((size_t)S * 3 * dm * es);
            L.gs[0] = take((size_t)S * 3 * dm * es);
            L.gs[1] = take((size_t)S * 3 * dm * es);
        }
        L.nsp = take((size_t)std::max(D.ns_iters, 1) * S * 3 * p * p * es);
        L.nsq = take((size_t)S * 3 * p * p * es);
        L.gb = take((size_t)S * 3 * dm * 4);
        L.pu = take((size_t)S * 3 * nblk * 4);
        L.pgu = take((size_t)S * 3 * nblk * 4);
    }
    L.total = off;
    return L;
}

ttt_status validate_full_bwd(const ttt_desc* D) {
    if (D->chunk_rates || (D->parallel_form && !D->last_layer_only))
        return fail(TTT_ERR_UNSUPPORTED,
                    "the backward of the recurrence covers every rule (with or without momentum) with per-token rates");
    const int64_t S = (int64_t)D->B * D->H, d = D->d_h, m = D->m_h;
    const int64_t bmax = D->N < D->chunk ? D->N : D->chunk;
    const int64_t lim = 1LL << 31;
    // every update keeps a copy of the weights: the count is bounded before anything is planned
    if ((D->N > 0 ? cdiv(D->N, D->chunk) : 0) * std::max(1, D->inner_steps) > kFbMaxUpdates)
        return fail(TTT_ERR_UNSUPPORTED, "the backward records at most %d updates (chunks x inner steps)", kFbMaxUpdates);
    // launch sizes (the query range may span every chunk)
    if (S * (cdiv(bmax, kFbRows) + cdiv(D->N, kFbRows)) * cdiv(m, kFbCols) >= lim ||
        S * (2 * cdiv(bmax, kFxRows) + cdiv(D->N, kFxRows)) * cdiv(d, kFxCols) >= lim ||
        S * 8 * 2 * cdiv(m, kFwTile) * cdiv(d, kFwTile) >= lim || S * (2 * m + d) >= lim ||
        S * 3 * d * m / 4 >= lim * kThreads || 4 * m * (bmax + D->N) >= lim)
        return fail(TTT_ERR_UNSUPPORTED, "B*H, N, d_h, m_h too large for one launch");
    return TTT_OK;
}

size_t full_bwd_ws_bytes(const ttt_desc& D, bool own_record) {
    const FbPlan P = fb_plan(D);
    return make_flayout(D, P, own_record).total;
}

template <typename T>
ttt_status run_full_backward(const ttt_desc& D, const T* q, const T* k, const T* v, const float* eta, const float* W0,
                             const T* dO, const float* dWo, T* dq, T* dk, T* dv, float* deta, float* dW0, char* ws,
                             hipStream_t st, char* record) {
    const FbPlan P = fb_plan(D);
    const FLayout L = make_flayout(D, P, record == nullptr);
    const FRecord R = record_layout(D, P);
    const int S = D.B * D.H, d = D.d_h, m = D.m_h;
    const int64_t dm = (int64_t)d * m, dm3 = 3 * dm;
    const int64_t hs = (int64_t)S * dm3;  // one version of every scan's weights
    const bool norm = D.rule == TTT_UPD_GD_L2 || D.rule == TTT_UPD_MUON_L2, mom = D.momentum != 0.0f;
    const bool muon = D.rule == TTT_UPD_MUON || D.rule == TTT_UPD_MUON_L2;
    const int mat0 = D.last_layer_only ? 2 : 0, nmat = D.last_layer_only ? 1 : 3;
    const int64_t pp = std::min(d, m);
    const float sign = D.ascent ? -1.0f : 1.0f;
    char* rec = record ? record : ws + L.rec;
    float* hist = (float*)(rec + R.hist);
    float* nrm = norm ? (float*)(rec + R.nrm) : nullptr;
    float* dW = (float*)(ws + L.dW);
    float* dM = mom ? (float*)(ws + L.dM) : nullptr;
    float* G = (float*)(ws + L.G);
    T* op = (T*)(ws + L.op);
    float* part = (float*)(ws + L.part);
    ttt_status rc;
    // the forward's record, unless the caller brings it
    float* urec = muon ? (float*)(rec + R.urec) : nullptr;
    if (!record && (rc = ttt_run_history<T>(D, q, k, v, eta, W0, (T*)nullptr, nullptr, hist, nrm, urec, ws + L.fwd,
                                            st)) != TTT_OK)
        return rc;
    {
        ProfScope ps(PK_FB_MISC, st);
        hipLaunchKernelGGL(k_fb_init, dim3((unsigned)cdiv(hs / 4, kThreads)), dim3(kThreads), 0, st, dW, dWo, dM,
                           hs / 4);
    }
    if ((rc = check_launch("k_fb_init", st)) != TTT_OK) return rc;
    // Muon at update ver: G holds the gradient of Newton-Schulz's output; it becomes Gamma
    auto muon_backward = [&](int ver) -> ttt_status {
        const float* U = urec + (int64_t)ver * hs;
        T* X = (T*)(ws + L.nsx);
        T* Xlo = sizeof(T) == 2 ? (T*)(ws + L.nsxl) : nullptr;
        T* P = (T*)(ws + L.nsp);
        T* Q = (T*)(ws + L.nsq);
        float* pu = (float*)(ws + L.pu);
        float* pgu = (float*)(ws + L.pgu);
        const int nblk = (int)cdiv(dm, kNsbElems);
        const unsigned eg = (unsigned)((int64_t)S * nmat * nblk);
        ttt_status r;
        // |U| (as partial sums), X_0 and the gradient's operand copy, then the forward's steps again
        {
            ProfScope ps(PK_FB_NSB, st);
            hipLaunchKernelGGL(k_nsb_dot, dim3(eg), dim3(kThreads), 0, st, U, U, pu, dm, mat0, nmat, nblk);
        }
        if ((r = check_launch("k_nsb_dot", st)) != TTT_OK) return r;
        T* gs[2] = {sizeof(T) == 2 ? (T*)(ws + L.gs[0]) : (T*)G, sizeof(T) == 2 ? (T*)(ws + L.gs[1]) : (T*)(ws + L.gb)};
        {
            ProfScope ps(PK_FB_NSB, st);
            hipLaunchKernelGGL(k_nsb_x0<T>, dim3(eg), dim3(kThreads), 0, st, U, (const float*)pu, X, Xlo, (const float*)G,
                               gs[0], dm, mat0, nmat, nblk);
        }
        if ((r = check_launch("k_nsb_x0", st)) != TTT_OK) return r;
        if ((r = ns_steps<T>(D, X, Xlo, P, st)) != TTT_OK) return r;
        float* Gc = G;
        float* Gn = (float*)(ws + L.gb);
        const int np = (int)cdiv(pp, kNsbQ);
        const int stt = (int)std::max(cdiv(m, kNsbRows) * cdiv(d, kNsbCols), cdiv(d, kNsbRows) * cdiv(m, kNsbCols));
        int cur = 0;
        for (int it = D.ns_iters - 1; it >= 0; --it) {
            NsbArgs<T> na{Gc, gs[cur], Gn, gs[cur ^ 1], X + (int64_t)it * hs, P + (int64_t)it * S * 3 * pp * pp, Q, d, m,
                          mat0, nmat, np * (np + 1) / 2};
            {
                ProfScope ps(PK_FB_NSB, st);
                hipLaunchKernelGGL(k_nsb_q<T>, dim3((unsigned)((int64_t)S * nmat * na.tiles)), dim3(kThreads), 0, st,
                                   na);
            }
            if ((r = check_launch("k_nsb_q", st)) != TTT_OK) return r;
            na.tiles = stt;
            {
                ProfScope ps(PK_FB_NSB, st);
                const dim3 grid((unsigned)((int64_t)S * nmat * stt));
                if (d % 128 == 0 && m % 128 == 0) hipLaunchKernelGGL((k_nsb_step<T, true>), grid, dim3(kThreads), 0, st, na);
                else hipLaunchKernelGGL((k_nsb_step<T, false>), grid, dim3(kThreads), 0, st, na);
            }
            if ((r = check_launch("k_nsb_step", st)) != TTT_OK) return r;
            std::swap(Gc, Gn);
            cur ^= 1;
        }
        {
            ProfScope ps(PK_FB_NSB, st);
            hipLaunchKernelGGL(k_nsb_dot, dim3(eg), dim3(kThreads), 0, st, (const float*)Gc, U, pgu, dm, mat0, nmat,
                               nblk);
        }
        if ((r = check_launch("k_nsb_dot", st)) != TTT_OK) return r;
        NsbFinalArgs fa{Gc, U, pu, pgu, G, dM, D.momentum, dm, mat0, nmat, nblk};
        {
            ProfScope ps(PK_FB_NSB, st);
            hipLaunchKernelGGL(k_nsb_final, dim3(eg), dim3(kThreads), 0, st, fa);
        }
        return check_launch("k_nsb_final", st);
    };
    const int ntm = (int)cdiv(m, kFwTile), ntd = (int)cdiv(d, kFwTile);
    int pending = 0;  // partial buffers holding sums the next prep (or the last step) adds
    for (int ver = P.T; ver >= 0; --ver) {
        const bool step = ver < P.T;
        const int ju = step ? P.step_chunk[ver] : -1, it = step ? P.step_it[ver] : 0;
        if (step) {
            FbPrepArgs pa{dW, part, pending, hs, norm ? hist + (int64_t)(ver + 1) * hs : nullptr,
                          norm ? nrm + (int64_t)ver * S * (2 * m + d) : nullptr, dM, D.momentum, G, d, m, S,
                          muon ? 1 : 0, D.last_layer_only ? 2 * m : 0};
            {
                ProfScope ps(PK_FB_PREP, st);
                hipLaunchKernelGGL(k_fb_prep, dim3((unsigned)cdiv((int64_t)S * (2 * m + d), kThreads / 64)),
                                   dim3(kThreads), 0, st, pa);
            }
            if ((rc = check_launch("k_fb_prep", st)) != TTT_OK) return rc;
            pending = 0;
            if (muon && (rc = muon_backward(ver)) != TTT_OK) return rc;
        }
        const int64_t a0 = P.qlo[ver];
        const int la = (int)(P.qhi[ver] - P.qlo[ver]);
        const int64_t u0 = step ? (int64_t)ju * D.chunk : 0;
        const int lu = step ? (int)(std::min<int64_t>(u0 + D.chunk, D.N) - u0) : 0;
        if (!la && !lu) continue;
        {
            FbOpsArgs<T> oa{step ? G : nullptr, hist + (int64_t)ver * hs, op, d, m, S, (int)cdiv(dm, kThreads),
                            2 * (d / 32) * (m / 32)};
            ProfScope ps(PK_FB_OPS, st);
            hipLaunchKernelGGL(k_fb_ops<T>, dim3((unsigned)((int64_t)S * (oa.ncopy + oa.ntr))), dim3(kThreads), 0, st,
                               oa);
        }
        if ((rc = check_launch("k_fb_ops", st)) != TTT_OK) return rc;
        const int nct = (int)cdiv(m, kFbCols);
        FbUpArgs<T> ua{q, k, v, dO, eta, op, L.acp ? (float*)(ws + L.acp) : nullptr,
                       L.qa ? (T*)(ws + L.qa) : nullptr, L.qh ? (T*)(ws + L.qh) : nullptr,
                       L.pk ? (T*)(ws + L.pk) : nullptr, L.pv ? (T*)(ws + L.pv) : nullptr,
                       L.pe ? (T*)(ws + L.pe) : nullptr, D.N, L.qcap, L.bcap, d, m, a0, la, u0, lu,
                       lu ? (int)(cdiv(lu, kFbRows) * nct) : 0, la ? (int)(cdiv(la, kFbRows) * nct) : 0, nct, sign};
        {
            ProfScope ps(PK_FB_UP, st);
            hipLaunchKernelGGL(k_fb_up<T>, dim3((unsigned)((int64_t)S * (ua.nK + ua.nQ))), dim3(64 * kFbWaves), 0, st,
                               ua);
        }
        if ((rc = check_launch("k_fb_up", st)) != TTT_OK) return rc;
        const int nin = P.nin;
        const int kmode = nin == 1 ? 0 : it == nin - 1 ? 1 : it == 0 ? 3 : 2;
        FbDxArgs<T> xa{ua.pk, ua.pv, ua.qa, op, v, eta, dk, dv, dq,
                       L.acck ? (float*)(ws + L.acck) : nullptr, L.accv ? (float*)(ws + L.accv) : nullptr,
                       L.epart ? (float*)(ws + L.epart) : nullptr, D.N, L.qcap, L.bcap, d, m, S, a0, la, u0, lu,
                       lu ? (int)cdiv(lu, kFxRows) : 0, la ? (int)cdiv(la, kFxRows) : 0, (int)cdiv(d, kFxCols),
                       kmode, sign};
        {
            ProfScope ps(PK_FB_DX, st);
            hipLaunchKernelGGL(k_fb_dx<T>, dim3((unsigned)((int64_t)S * (2 * xa.ntu + xa.nta) * xa.ntd)),
                               dim3(kThreads), 0, st, xa);
        }
        if ((rc = check_launch("k_fb_dx", st)) != TTT_OK) return rc;
        if (lu) {
            {
                ProfScope ps(PK_FB_MISC, st);
                hipLaunchKernelGGL(k_fb_deta, dim3((unsigned)cdiv((int64_t)S * lu, kThreads)), dim3(kThreads), 0, st,
                                   (const float*)xa.epart, deta, D.N, u0, lu, L.bcap, S, xa.ntd, sign,
                                   it == nin - 1 ? 0 : 1);
            }
            if ((rc = check_launch("k_fb_deta", st)) != TTT_OK) return rc;
        }
        const int total = lu + la;
        const int lp = (int)(cdiv(cdiv(total, L.nparts), 64) * 64);
        FbDwArgs<T> wa{ua.pk, ua.pe, ua.qa, ua.qh, k, v, q, dO, part, D.N, L.qcap, L.bcap, hs, d, m, a0, la, u0, lu,
                       L.nparts, lp, ntm, ntd};
        for (int job = 0; job < 2; ++job) {
            {
                ProfScope ps(PK_FB_DW, st);
                const dim3 grid((unsigned)((int64_t)S * L.nparts * ntm * ntd));
                if (job == 0) hipLaunchKernelGGL((k_fb_dw<T, 0>), grid, dim3(kThreads), 0, st, wa);
                else hipLaunchKernelGGL((k_fb_dw<T, 1>), grid, dim3(kThreads), 0, st, wa);
            }
            if ((rc = check_launch("k_fb_dw", st)) != TTT_OK) return rc;
        }
        pending = L.nparts;
    }
    // token gradients of chunks that do not update
    if (D.mask == TTT_MASK_STRIDED)
        for (int64_t j = 0; j < cdiv(D.N, D.chunk); ++j) {
            if (D.update_chunks[j]) continue;
            const int64_t lo = j * D.chunk;
            const int len = (int)(std::min<int64_t>(lo + D.chunk, D.N) - lo);
            const int64_t n = (int64_t)S * len * (d / 4);
            {
                ProfScope ps(PK_FB_MISC, st);
                hipLaunchKernelGGL(k_fb_zero_rows<T>, dim3((unsigned)cdiv(n, kThreads)), dim3(kThreads), 0, st, dk, dv,
                                   deta, D.N, lo, len, d, S);
            }
            if ((rc = check_launch("k_fb_zero_rows", st)) != TTT_OK) return rc;
        }
    if (dW0) {
        const int nw = D.w0_per_batch ? S : D.H;
        FbFinalArgs fa{dW, part, pending, hs, dW0, nw, D.w0_per_batch ? 1 : D.B, D.H, D.w0_per_batch ? 0 : 1, dm3};
        {
            ProfScope ps(PK_FB_MISC, st);
            hipLaunchKernelGGL(k_fb_final, dim3((unsigned)cdiv((int64_t)nw * dm3 / 4, kThreads)), dim3(kThreads), 0,
                               st, fa);
        }
        if ((rc = check_launch("k_fb_final", st)) != TTT_OK) return rc;
    }
    return TTT_OK;
}

template ttt_status run_full_backward<uint16_t>(const ttt_desc&, const uint16_t*, const uint16_t*, const uint16_t*,
                                                const float*, const float*, const uint16_t*, const float*, uint16_t*,
                                                uint16_t*, uint16_t*, float*, float*, char*, hipStream_t, char*);
template ttt_status run_full_backward<float>(const ttt_desc&, const float*, const float*, const float*, const float*,
                                             const float*, const float*, const float*, float*, float*, float*, float*,
                                             float*, char*, hipStream_t, char*);

size_t full_bwd_record_bytes(const ttt_desc& D) { return record_layout(D, fb_plan(D)).total; }

template <typename T>
ttt_status run_forward_record(const ttt_desc& D, const T* q, const T* k, const T* v, const float* eta, const float* W0,
                              T* o, float* W_out, char* record, char* ws, hipStream_t st) {
    const FbPlan P = fb_plan(D);
    const FRecord R = record_layout(D, P);
    const bool norm = D.rule == TTT_UPD_GD_L2 || D.rule == TTT_UPD_MUON_L2;
    const bool muon = D.rule == TTT_UPD_MUON || D.rule == TTT_UPD_MUON_L2;
    return ttt_run_history<T>(D, q, k, v, eta, W0, o, W_out, (float*)(record + R.hist),
                              norm ? (float*)(record + R.nrm) : nullptr, muon ? (float*)(record + R.urec) : nullptr, ws,
                              st);
}
template ttt_status run_forward_record<uint16_t>(const ttt_desc&, const uint16_t*, const uint16_t*, const uint16_t*,
                                                 const float*, const float*, uint16_t*, float*, char*, char*,
                                                 hipStream_t);
template ttt_status run_forward_record<float>(const ttt_desc&, const float*, const float*, const float*, const float*,
                                              const float*, float*, float*, char*, char*, hipStream_t);

}  // namespace ttt
