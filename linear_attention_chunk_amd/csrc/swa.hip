// LaCT's sliding-window attention on gfx950: causal softmax attention over a window of w tokens
// with a per-head, per-channel scale and shift on Q and K, sharing Q, K, V with the fast-weight
// branch (PaperTrace "5.2.1 LaCT and TTT-E2E", section 1.1, the window-attention paragraphs, and the
// remark after Eq. (10): a window as wide as the chunk covers the chunk that the fast weights see
// only from the next chunk on).  Token t attends to the tokens s with t - w < s <= t; the scores are
// q'_t . k'_s / sqrt(d) with q' = q * gamma_q + beta_q and k' = k * gamma_k + beta_k per channel.
//
// Two launches per call:
//   qprep  q'' = (q * gamma_q + beta_q) * gamma_k per channel, into the workspace (io dtype).  The
//          scores then are q'' . k plus q' . beta_k, and the second term is one number per query
//          (the same for every key), which softmax removes: the key shift never changes the result,
//          so k is used as it is.
//   attend one workgroup per 128 queries of one (batch, head), walking the 128-key blocks that meet
//          its window.  Per block: S = q'' k^T on MFMA (tile engine, contraction over d), the window
//          mask and 1/sqrt(d), an online softmax in fp32 (running row maximum and sum, the output
//          accumulators rescaled when the maximum grows), P rounded to the io dtype straight into
//          the LDS stage of the P v product, and O += P v with v through the transposing stager.
//          The outputs of all d columns stay in MFMA accumulators for the whole walk; at the end
//          they are divided by the row sums.
#include <algorithm>
#include <math.h>

#include "host_common.hpp"
#include "tile.hpp"

namespace ttt {

constexpr int kSwaRows = 128;    // queries per workgroup
constexpr int kSwaKeys = 64;     // keys per block of the walk
constexpr int kSwaWaves = 8;
constexpr int kSwaMaxD = 384;

template <typename T> struct SwaArgs {
    const T* q2;                 // q'' [S][N][d]
    const T* k; const T* v; T* o;
    int64_t N; int d, window, nqb, ncb;  // query blocks, output-column blocks per scan
    float inv_sqrt_d;
};

// One workgroup per 128 queries of one scan and DV output columns (heads wider than DV take several
// workgroups, each computing the scores again), eight waves as 4 x 2: in the score tile (128 queries x
// 64 keys) and in the output tile (128 x DV) wave (wm, wn) owns the same 32 queries, with keys or
// output columns split in two halves, so a lane's 16 row statistics serve its own output rows; the
// two waves that share a row exchange their partial maxima and sums through LDS.
template <typename T, int DV>
__global__ __launch_bounds__(64 * kSwaWaves, 1) void k_swa(SwaArgs<T> a) {
    using TS = Tile<T, kSwaRows, kSwaKeys, 2, 4, 1, 1, 1, false, false, false, kSwaWaves>;
    using TD = Tile<T, kSwaRows, DV, 2, 4, 1, 1, 1, false, true, false, kSwaWaves, 1>;
    static_assert(TS::FM == 1 && TD::FM == 1 && TS::WGN == 2 && TD::WGN == 2, "waves share query rows");
    constexpr int NSTG = kSwaKeys / TD::KSTEP;  // P v stages per key block
    static_assert(kSwaKeys % TD::KSTEP == 0 && TS::WN % TD::KSTEP == 0 || TD::KSTEP % TS::WN == 0, "key stages");
    constexpr int LDST = std::max(TS::LDS, TD::STAGE);
    __shared__ __attribute__((aligned(16))) char smem[LDST + 2 * 2 * kSwaRows * 4];
    float* xmax = reinterpret_cast<float*>(smem + LDST);  // [2 key halves][128 rows]
    float* xsum = xmax + 2 * kSwaRows;

    const int lb = xcd_block(gridDim.x);
    const int cb = lb % a.ncb, scan = lb / a.ncb / a.nqb, qb = lb / a.ncb % a.nqb;
    const int c0 = cb * DV;  // this workgroup's output columns [c0, c0 + DV)
    const int64_t q0 = (int64_t)qb * kSwaRows;
    const int nq = (int)std::min<int64_t>(kSwaRows, a.N - q0);
    const int64_t base = (int64_t)scan * a.N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / 2, wn = wave % 2, g = lane >> 5;
    // this lane's 16 rows (the same in the score and output tiles)
    auto row_of = [&](int r) { return wm * 32 + 8 * (r >> 2) + 4 * g + (r & 3); };

    float m[16], l[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) { m[r] = -INFINITY; l[r] = 0.f; }
    TD td;
    td.zero();

    // key blocks that meet the window of some query of this block
    const int64_t kfirst = std::max<int64_t>(0, q0 - a.window + 1), klast = q0 + nq - 1;
    for (int64_t k0 = (kfirst / kSwaKeys) * kSwaKeys; k0 <= klast; k0 += kSwaKeys) {
        const int nk = (int)std::min<int64_t>(kSwaKeys, a.N - k0);
        // S = q'' k^T over d
        const Opnd<T> A[1] = {{a.q2 + (base + q0) * a.d, a.d, nq, a.d}};
        const Opnd<T> B[1] = {{a.k + (base + k0) * a.d, a.d, nk, a.d}};
        TS ts;
        ts.template run<PM1>(A, B, a.d, smem);
        // window mask and 1/sqrt(d); this half's row maxima, reduced over the 32 lanes of a row group
        // key - query offsets in 32 bits: key j*32 + c of this half against query row_of(r); a key
        // counts when 0 <= query - key < window and it lies before N
        const int dq = (int)(q0 - k0), kend = nk;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qr = dq + row_of(r);  // query index relative to k0
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < TS::FN; ++j) {
                const int kr = wn * TS::WN + j * 32 + (lane & 31);
                const bool ok = kr <= qr && qr - kr < a.window && kr < kend;
                const float sv = ok ? ts.acc[0][0][j][r] * a.inv_sqrt_d : -INFINITY;
                ts.acc[0][0][j][r] = sv;
                mx = fmaxf(mx, sv);
            }
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            if ((lane & 31) == r) xmax[wn * kSwaRows + row_of(r)] = mx;
        }
        lds_barrier();  // both halves' maxima are in; every wave is done with the score tile's stages
        // new maxima; rescale the output rows and the sums by exp(m_old - m_new); P = exp(S - m)
        // rounded to the io dtype (0 where masked), kept in the score accumulators, and this half's
        // row sums of the rounded weights (the ones the product uses)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float mn = fmaxf(m[r], fmaxf(xmax[row_of(r)], xmax[kSwaRows + row_of(r)]));
            // a row that has seen no key yet keeps -inf: nothing to rescale, and its P stays 0
            const float alpha = mn == -INFINITY ? 1.f : __expf(m[r] - mn);
            m[r] = mn;
            l[r] *= alpha;
#pragma unroll
            for (int j = 0; j < TD::FN; ++j) td.acc[0][0][j][r] *= alpha;
            float sm = 0.f;
#pragma unroll
            for (int j = 0; j < TS::FN; ++j) {
                const float sv = ts.acc[0][0][j][r];
                const float p = Elt<T>::ld(Elt<T>::st(sv == -INFINITY ? 0.f : __expf(sv - mn)));
                ts.acc[0][0][j][r] = p;
                sm += p;
            }
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) sm += __shfl_xor(sm, o, 64);
            if ((lane & 31) == r) xsum[wn * kSwaRows + row_of(r)] = sm;
        }
        // O += P v, one key stage at a time through one LDS stage: P of the stage's keys into its A
        // region, v of those keys into its B region (stages with no key left are skipped)
#pragma unroll
        for (int st = 0; st < NSTG; ++st) {
            const int kv = st * TD::KSTEP;
            if (kv >= nk) break;  // uniform over the workgroup
#pragma unroll
            for (int j = 0; j < TS::FN; ++j) {
                const int col = wn * TS::WN + j * 32 + (lane & 31);
                if (col / TD::KSTEP == st)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        *reinterpret_cast<T*>(smem + row_of(r) * TD::PITCH + (col % TD::KSTEP) * (int)sizeof(T)) =
                            Elt<T>::st(ts.acc[0][0][j][r]);
            }
            const Opnd<T> V = {a.v + (base + k0 + kv) * a.d + c0, a.d, a.d - c0, std::min(TD::KSTEP, nk - kv)};
            typename TD::SB gv;
            if (a.d - c0 >= DV && nk - kv >= TD::KSTEP) {
                gv.template load<true>(V, 0);
                gv.template store<true>(smem + TD::A_BYTES);
            } else {
                gv.template load<false>(V, 0);
                gv.template store<false>(smem + TD::A_BYTES);
            }
            lds_barrier();
            td.template compute<PM1>(smem);
            lds_barrier();  // every wave is done with the stage before it is refilled
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) l[r] += xsum[row_of(r)] + xsum[kSwaRows + row_of(r)];
    }
    // O = acc / l, rows below nq and columns below d
    T* O = a.o + (base + q0) * a.d + c0;
#pragma unroll
    for (int j = 0; j < TD::FN; ++j) {
        const int col = RowMap<T, DV, 2, true>::row_of(wn * TD::WN + j * 32 + (lane & 31));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = row_of(r);
            if (row < nq && c0 + col < a.d) O[(uint32_t)row * (uint32_t)a.d + (uint32_t)col] = Elt<T>::st(td.acc[0][0][j][r] / l[r]);
        }
    }
}

// bf16 heads whose d is a multiple of 64: a walk with the queries resident in registers.  One
// workgroup of 4 waves (one per SIMD, one workgroup per CU) takes 128 queries of one scan; wave w owns
// queries 32w .. 32w+31 as two groups of 16 and keeps their q'' over all of d as 16 x 16 x 32 MFMA
// fragments for the whole walk.  Per block of 32 keys:
//   - the block's k rows are staged in LDS as they are, and its v block as prepared by k_swa_vprep
//     (d-major, keys in the order below), in two alternating LDS buffers, so one workgroup barrier
//     per block suffices;
//   - each wave forms the transposed scores k q''^T of its 32 queries (keys on the accumulator
//     rows), so a lane holds 8 keys of one query: the window mask (only on blocks at the window's
//     edges), the query's maximum over the 4 lanes that hold it (lane swaps across rows and halves),
//     and the online-softmax step, against a reference maximum that moves only when exceeded by more
//     than kSwqTau (so the output rows are rarely rescaled; the row sums are kept per lane and
//     reduced once at the end);
//   - the lane's 8 weights, rounded to bf16, are its part of the B operand of O^T += v^T P^T.  That
//     product contracts over the keys in the order the lane holds them: keys 4g .. 4g+3 and
//     16+4g .. 16+4g+3 for lane group g, the order in which the prepared v block stores them, so a
//     v fragment is one 16-byte LDS read and P never leaves the registers;
//   - O^T's accumulators put each lane on its own query and 4 consecutive output columns of d.
// q'' is formed from q and the per-channel parameters as the fragments are loaded (fp32, rounded to
// bf16 once).  The next block's k and v are loaded into registers while the current block is
// computed; the MFMA accumulators are kept in VGPRs (build flag), since the softmax works on them
// with VALU code.
constexpr int kSwqQ = 128, kSwqK = 32;
constexpr float kSwqTau = 8.f;  // how far (in e-folds) a block's maximum may exceed the reference
constexpr float kLog2e = 1.44269504088896341f;

// two floats to a packed bf16 pair, round to nearest even (one instruction on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, b2));
}
// max / sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the 4 lanes that hold one query): swaps of
// 16-lane rows and of 32-lane halves
__device__ __forceinline__ float max4rows(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4rows(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The v blocks of every scan for the walk: block kb of scan s is d rows (columns of v) of 32 keys,
// 64 bytes a row, the keys in the order 0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31 (so the 16
// bytes at 16 g hold keys 4g .. 4g+3 and 16+4g .. 16+4g+3); keys at or beyond N are zero.  One thread
// takes 8 columns of one block: 32 loads of 16 bytes (one per key), 32 stores of 16 bytes.
struct VPrepArgs {
    const uint16_t* v; uint16_t* vp;
    int64_t N, nkb, nthreads; int d;
};

__global__ __launch_bounds__(kThreads) void k_swa_vprep(VPrepArgs a) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= a.nthreads) return;
    const int ncg = a.d / 8;
    const int cg = (int)(t % ncg);
    const int64_t blk = t / ncg, scan = blk / a.nkb, kb = blk % a.nkb;
    const int64_t k0 = kb * kSwqK;
    const uint16_t* src = a.v + (scan * a.N + k0) * a.d + cg * 8;
    u32x4_t r[kSwqK];
#pragma unroll
    for (int k = 0; k < kSwqK; ++k) {
        const bool in = k0 + k < a.N;  // rows past N read row k0 (in range) and are zeroed
        r[k] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)(in ? k : 0) * a.d);
        if (!in) r[k] = u32x4_t{0u, 0u, 0u, 0u};
    }
    uint16_t* dst = a.vp + (blk * a.d + cg * 8) * kSwqK;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        // element c of key k: half (c & 1) of word c >> 1
        auto el = [&](int k) -> uint32_t { return (r[k][c >> 1] >> (16 * (c & 1))) & 0xFFFFu; };
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const u32x4_t w = {el(4 * g) | (el(4 * g + 1) << 16), el(4 * g + 2) | (el(4 * g + 3) << 16),
                               el(16 + 4 * g) | (el(16 + 4 * g + 1) << 16), el(16 + 4 * g + 2) | (el(16 + 4 * g + 3) << 16)};
            *reinterpret_cast<u32x4_t*>(dst + c * kSwqK + 8 * g) = w;
        }
    }
}

struct QresArgs {
    const uint16_t* q; const uint16_t* k; const uint16_t* vp; uint16_t* o;
    const float* qs; const float* qb; const float* ks;  // [H][d] or null
    int64_t N; int H, window, nqb;
    float inv_sqrt_d;
};

template <int D>
__global__ __launch_bounds__(256, 1) void k_swa_qres(QresArgs a) {
    using T = uint16_t;
    constexpr int KP = 2 * D + 16;             // bytes per staged k row
    constexpr int VP = 2 * kSwqK + 16;         // bytes per staged v row (one column of v)
    constexpr int NQF = D / 32, NOB = D / 16;  // q'' fragments per query group, 16-column output blocks
    constexpr int KPER = kSwqK * D / 8 / 256, VPR = D / 8;
    constexpr int VPER = D * 4 / 256;          // 16-byte vectors of the v block per thread
    static_assert(kSwqK * D / 8 % 256 == 0 && D * 4 % 256 == 0, "whole rounds");
    constexpr int K_BYTES = kSwqK * KP, V_BYTES = D * VP, BUF = K_BYTES + V_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

    const int lb = xcd_block(gridDim.x);
    const int scan = lb / a.nqb, qb = lb % a.nqb;
    const int64_t q0 = (int64_t)qb * kSwqQ;
    const int nq = (int)std::min<int64_t>(kSwqQ, a.N - q0);
    const int64_t base = (int64_t)scan * a.N;
    const int64_t nkb = (a.N + kSwqK - 1) / kSwqK;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    // the lane's query in group g is 32 wave + 16 g + lr; element i of its 16 x 16 score block j
    // is key 16 j + 4 lg + i of the block

    // B fragments: query 32 wave + 16 g + lr, d = 32 s + 8 lg .. + 7 of q'' = (q * q_scale + q_shift)
    // * k_scale, formed in fp32 and rounded to bf16 once
    u32x4_t qf[2][NQF];
    {
        const int h = scan % a.H;
        const float* qs = a.qs ? a.qs + h * D + lg * 8 : nullptr;
        const float* qbs = a.qb ? a.qb + h * D + lg * 8 : nullptr;
        const float* ks = a.ks ? a.ks + h * D + lg * 8 : nullptr;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int row = 32 * wave + 16 * g + lr;
            const T* src = a.q + (base + q0 + (row < nq ? row : 0)) * D + lg * 8;
#pragma unroll
            for (int s = 0; s < NQF; ++s) {
                const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(src + s * 32);
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = __uint_as_float(e & 1 ? raw[e >> 1] & 0xFFFF0000u : raw[e >> 1] << 16);
                if (qs)
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] *= qs[s * 32 + e];
                if (qbs)
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] += qbs[s * 32 + e];
                if (ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] *= ks[s * 32 + e];
                qf[g][s] = row < nq ? u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                              pack_bf16x2(y[6], y[7])}
                                    : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    }
    // key blocks that meet the window of some query of this block
    const int64_t kfirst = std::max<int64_t>(0, q0 - a.window + 1), klast = q0 + nq - 1;
    const int64_t kstart = (kfirst / kSwqK) * kSwqK;
    const int nblk = (int)((klast - kstart) / kSwqK) + 1;
    const float sc = a.inv_sqrt_d * kLog2e;  // base-2 units
    const float tau = kSwqTau / a.inv_sqrt_d;  // the threshold in raw score units

    u32x4_t kr[KPER], vr[VPER];
    uint32_t kok = 0;
    auto load_kv = [&](int64_t k0) {
        const int nk = (int)std::min<int64_t>(kSwqK, a.N - k0);
        kok = 0;
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int v = threadIdx.x + i * 256, row = v / VPR, c = v % VPR;
            const bool in = row < nk;
            kr[i] = *reinterpret_cast<const u32x4_t*>(a.k + (base + k0 + (in ? row : 0)) * D + c * 8);
            kok |= (uint32_t)in << i;
        }
        const T* vb = a.vp + (scan * nkb + k0 / kSwqK) * D * kSwqK;
#pragma unroll
        for (int i = 0; i < VPER; ++i) vr[i] = *reinterpret_cast<const u32x4_t*>(vb + (threadIdx.x + i * 256) * 8);
    };

    float m[2], lp[2];   // per query: reference maximum (raw score units) and this lane's row-sum part
    f32x4_t o[2][NOB];   // O^T: element i of block jd is column 16 jd + 4 lg + i of the lane's query
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        m[g] = -INFINITY;
        lp[g] = 0.f;
#pragma unroll
        for (int j = 0; j < NOB; ++j) o[g][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    load_kv(kstart);
    for (int b = 0; b < nblk; ++b) {
        const int64_t k0 = kstart + (int64_t)b * kSwqK;
        const int nk = (int)std::min<int64_t>(kSwqK, a.N - k0);
        char* Ks = smem + (b & 1) * BUF;
        char* Vs = Ks + K_BYTES;
        // this buffer was last read two blocks ago, before every wave passed the previous barrier
#pragma unroll
        for (int i = 0; i < KPER; ++i) {
            const int v = threadIdx.x + i * 256, row = v / VPR, c = v % VPR;
            *reinterpret_cast<u32x4_t*>(Ks + row * KP + c * 16) = ((kok >> i) & 1u) ? kr[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < VPER; ++i) {
            const int v = threadIdx.x + i * 256;
            *reinterpret_cast<u32x4_t*>(Vs + (v >> 2) * VP + (v & 3) * 16) = vr[i];
        }
        if (b + 1 < nblk) load_kv(k0 + kSwqK);
        lds_barrier();  // the block is staged
        // transposed scores: A = the block's k rows, B = the queries' q''
        f32x4_t sacc[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 2; ++g) sacc[j][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < NQF; ++s)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(Ks + (j * 16 + lr) * KP + s * 64 + lg * 16);
                Elt<T>::mma(sacc[j][0], kf, qf[0][s]);
                Elt<T>::mma(sacc[j][1], kf, qf[1][s]);
            }
        __builtin_amdgcn_s_setprio(0);
        // a block inside every query's window (and before N) needs no mask; the test is uniform
        const bool inside = k0 + kSwqK - 1 <= q0 && q0 + nq - 1 - k0 < a.window && nk == kSwqK;
        if (!inside) {
            const int dq = (int)(q0 - k0);
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int qr = dq + 32 * wave + 16 * g + lr;  // the lane's query, relative to k0
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kc = 16 * j + 4 * lg + i;
                        if (!(kc <= qr && qr - kc < a.window && kc < nk)) sacc[j][g][i] = -INFINITY;
                    }
            }
        }
        float alpha[2];
        bool resc = false;
        u32x4_t pk[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            float mx = fmaxf(fmaxf(fmaxf(sacc[0][g][0], sacc[0][g][1]), fmaxf(sacc[0][g][2], sacc[0][g][3])),
                             fmaxf(fmaxf(sacc[1][g][0], sacc[1][g][1]), fmaxf(sacc[1][g][2], sacc[1][g][3])));
            mx = max4rows(mx);
            // a query that has seen no key yet (reference -inf) has nothing to rescale; one with no key
            // in this block keeps its reference, and its weights stay 0
            const float mref = m[g];
            const float mn = mref == -INFINITY || mx > mref + tau ? mx : mref;
            alpha[g] = mref == -INFINITY || mn == mref ? 1.f : __builtin_amdgcn_exp2f((mref - mn) * sc);
            resc = resc || alpha[g] != 1.f;
            m[g] = mn;
            // p = 2^((s - m) sc); masked scores are -inf and give 0 (a reference still at -inf means
            // every score of the query is -inf so far: subtracting 0 keeps them -inf)
            const float off = mn == -INFINITY ? 0.f : -mn * sc;
            float pw[8];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[4 * j + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][g][i], sc, off));
            float ps = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t w2 = pack_bf16x2(pw[2 * x], pw[2 * x + 1]);
                pk[g][x] = w2;
                ps += __uint_as_float(w2 << 16) + __uint_as_float(w2 & 0xFFFF0000u);  // the rounded weights
            }
            lp[g] = lp[g] * alpha[g] + ps;
        }
        if (__any(resc)) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int j = 0; j < NOB; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[g][j][i] *= alpha[g];
        }
        // O^T += v^T P^T
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int jd = 0; jd < NOB; ++jd) {
            const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(Vs + (16 * jd + lr) * VP + 16 * lg);
            Elt<T>::mma(o[0][jd], vf, pk[0]);
            Elt<T>::mma(o[1][jd], vf, pk[1]);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    // O = acc / (row sum) for the lane's query if below nq: 4 consecutive columns per store
    T* O = a.o + (base + q0) * D;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const float inv = 1.f / sum4rows(lp[g]);
        const int row = 32 * wave + 16 * g + lr;
        if (row < nq) {
#pragma unroll
            for (int jd = 0; jd < NOB; ++jd)
                Pack4<T>::store(O + (uint32_t)row * (uint32_t)D + (uint32_t)(16 * jd + 4 * lg), o[g][jd][0] * inv,
                                o[g][jd][1] * inv, o[g][jd][2] * inv, o[g][jd][3] * inv);
        }
    }
}

// q'' = (q * gamma_q + beta_q) * gamma_k per channel, four elements per thread; the parameters are
// per head [H][d] (null: scale 1, shift 0)
template <typename T> struct QPrepArgs {
    const T* q; T* q2; const float* qs; const float* qb; const float* ks;
    int64_t n4; int d, H; int64_t N;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_swa_qprep(QPrepArgs<T> a) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= a.n4) return;
    const int64_t e = 4 * i;
    const int c = (int)(e % a.d);
    const int h = (int)((e / a.d / a.N) % a.H);
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float y = Elt<T>::ld(a.q[e + u]);
        if (a.qs) y *= a.qs[h * a.d + c + u];
        if (a.qb) y += a.qb[h * a.d + c + u];
        if (a.ks) y *= a.ks[h * a.d + c + u];
        x[u] = y;
    }
    Pack4<T>::store(a.q2 + e, x[0], x[1], x[2], x[3]);
}

static ttt_status validate_swa(const swa_desc* D) {
    if (!D) return fail(TTT_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (D->B < 0 || D->H < 0 || D->N < 0) return fail(TTT_ERR_INVALID_ARGUMENT, "B, H, N must be >= 0");
    if (D->d < 32 || D->d > kSwaMaxD || D->d % 32)
        return fail(TTT_ERR_INVALID_ARGUMENT, "d=%d must be a multiple of 32 in [32, %d]", D->d, kSwaMaxD);
    if (D->window < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "window must be >= 1");
    if (D->io_dtype != TTT_F32 && D->io_dtype != TTT_BF16) return fail(TTT_ERR_INVALID_ARGUMENT, "bad io_dtype");
    const int64_t S = (int64_t)D->B * D->H;
    if (S > (1 << 20) || S * cdiv(D->N, kSwaRows) * cdiv(D->d, 128) >= (1LL << 31))
        return fail(TTT_ERR_INVALID_ARGUMENT, "B*H*N too large for one launch");
    return TTT_OK;
}

// bf16 heads on the query-resident walk (d a multiple of 64 other than 320)
static bool swa_qres(const swa_desc& D) { return D.io_dtype == TTT_BF16 && D.d % 64 == 0 && D.d != 320; }

static size_t swa_ws_bytes(const swa_desc& D) {
    if (swa_qres(D)) return (size_t)D.B * D.H * cdiv(D.N, kSwqK) * kSwqK * D.d * 2;  // prepared v blocks
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    return (size_t)D.B * D.H * D.N * D.d * es;  // q''
}

template <typename T, int DV>
static ttt_status launch_swa(const SwaArgs<T>& a, int64_t grid, hipStream_t st) {
    {
        ProfScope ps(PK_SWA, st);
        hipLaunchKernelGGL((k_swa<T, DV>), dim3((unsigned)grid), dim3(64 * kSwaWaves), 0, st, a);
    }
    return check_launch("k_swa", st);
}

template <typename T>
static ttt_status run_swa(const swa_desc& D, const T* q, const T* k, const T* v, const float* qs, const float* qb,
                          const float* ks, T* o, char* ws, hipStream_t st) {
    const int64_t S = (int64_t)D.B * D.H;
    ttt_status rc;
    if constexpr (sizeof(T) == 2) {
        if (swa_qres(D)) {  // queries resident in registers, v prepared in blocks of 32 keys
            T* vp = (T*)ws;
            VPrepArgs va{v, vp, D.N, cdiv(D.N, kSwqK), 0, D.d};
            va.nthreads = S * va.nkb * (D.d / 8);
            {
                ProfScope ps(PK_SWA_VPREP, st);
                hipLaunchKernelGGL(k_swa_vprep, dim3((unsigned)cdiv(va.nthreads, kThreads)), dim3(kThreads), 0, st, va);
            }
            if ((rc = check_launch("k_swa_vprep", st)) != TTT_OK) return rc;
            QresArgs a{q, k, vp, o, qs, qb, ks, D.N, D.H, D.window, (int)cdiv(D.N, kSwqQ), 1.0f / sqrtf((float)D.d)};
            const unsigned grid = (unsigned)(S * a.nqb);
            {
                ProfScope ps(PK_SWA, st);
                switch (D.d) {
                    case 64: hipLaunchKernelGGL(k_swa_qres<64>, dim3(grid), dim3(256), 0, st, a); break;
                    case 128: hipLaunchKernelGGL(k_swa_qres<128>, dim3(grid), dim3(256), 0, st, a); break;
                    case 192: hipLaunchKernelGGL(k_swa_qres<192>, dim3(grid), dim3(256), 0, st, a); break;
                    case 256: hipLaunchKernelGGL(k_swa_qres<256>, dim3(grid), dim3(256), 0, st, a); break;
                    default: hipLaunchKernelGGL(k_swa_qres<384>, dim3(grid), dim3(256), 0, st, a); break;
                }
            }
            return check_launch("k_swa_qres", st);
        }
    }
    T* q2 = (T*)ws;
    QPrepArgs<T> pa{q, q2, qs, qb, ks, S * D.N * D.d / 4, D.d, D.H, D.N};
    {
        ProfScope ps(PK_SWA_PREP, st);
        hipLaunchKernelGGL(k_swa_qprep<T>, dim3((unsigned)cdiv(pa.n4, kThreads)), dim3(kThreads), 0, st, pa);
    }
    if ((rc = check_launch("k_swa_qprep", st)) != TTT_OK) return rc;
    SwaArgs<T> a{q2, k, v, o, D.N, D.d, D.window, (int)cdiv(D.N, kSwaRows), 1, 1.0f / sqrtf((float)D.d)};
    // output columns per workgroup: as many as fit the registers beside the scores (bf16: 256, or
    // 192 in two workgroups for wider heads; fp32: 128)
    if constexpr (sizeof(T) == 2) {
        if (D.d <= 128) return launch_swa<T, 128>(a, S * a.nqb, st);
        if (D.d <= 256) return launch_swa<T, 256>(a, S * a.nqb, st);
        a.ncb = (int)cdiv(D.d, 192);
        return launch_swa<T, 192>(a, S * a.nqb * a.ncb, st);
    } else {
        a.ncb = (int)cdiv(D.d, 128);
        return launch_swa<T, 128>(a, S * a.nqb * a.ncb, st);
    }
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status swa_workspace_bytes(const swa_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_swa(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = swa_ws_bytes(*desc);
    return TTT_OK;
}

extern "C" ttt_status swa_forward(const swa_desc* desc, const void* q, const void* k, const void* v,
                                  const float* q_scale, const float* q_shift, const float* k_scale,
                                  const float* k_shift, void* o, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    clear_error();
    ttt_status rc = validate_swa(desc);
    if (rc != TTT_OK) return rc;
    const swa_desc& D = *desc;
    const int64_t S = (int64_t)D.B * D.H;
    if (S == 0 || D.N == 0) return TTT_OK;
    if (!q || !k || !v || !o) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v and o are required");
    const void* p16[] = {q, k, v, o};
    for (const void* p : p16)
        if (!aligned(p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, o must be 16-byte aligned");
    const float* par[] = {q_scale, q_shift, k_scale, k_shift};
    for (const float* p : par)
        if (p && !aligned(p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "scale and shift vectors must be 16-byte aligned");
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const size_t ib = (size_t)S * D.N * D.d * es, pb = (size_t)D.H * D.d * 4;
    if (overlaps(o, ib, q, ib) || overlaps(o, ib, k, ib) || overlaps(o, ib, v, ib))
        return fail(TTT_ERR_INVALID_ARGUMENT, "o overlaps an input");
    const size_t need = swa_ws_bytes(D);
    if (!workspace || workspace_bytes < need)
        return fail(TTT_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 256)) return fail(TTT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (overlaps(workspace, need, o, ib) || overlaps(workspace, need, q, ib) || overlaps(workspace, need, k, ib) ||
        overlaps(workspace, need, v, ib))
        return fail(TTT_ERR_INVALID_ARGUMENT, "workspace overlaps an input or the output");
    {  // every buffer the call touches lies in a device allocation that holds all of it (k_shift is not read)
        const struct { const void* p; size_t n; const char* name; } bufs[] = {
            {q, ib, "q"}, {k, ib, "k"}, {v, ib, "v"}, {o, ib, "o"}, {q_scale, pb, "q_scale"}, {q_shift, pb, "q_shift"},
            {k_scale, pb, "k_scale"}, {workspace, need, "workspace"}};
        for (const auto& b : bufs)
            if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    }
    hipStream_t st = (hipStream_t)stream;
    if (D.io_dtype == TTT_BF16)
        return run_swa<uint16_t>(D, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, q_scale, q_shift, k_scale,
                                 (uint16_t*)o, (char*)workspace, st);
    return run_swa<float>(D, (const float*)q, (const float*)k, (const float*)v, q_scale, q_shift, k_scale, (float*)o,
                          (char*)workspace, st);
}
