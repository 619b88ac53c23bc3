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

static size_t swa_ws_bytes(const swa_desc& D) {
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
    T* q2 = (T*)ws;
    QPrepArgs<T> pa{q, q2, qs, qb, ks, S * D.N * D.d / 4, D.d, D.H, D.N};
    {
        ProfScope ps(PK_SWA_PREP, st);
        hipLaunchKernelGGL(k_swa_qprep<T>, dim3((unsigned)cdiv(pa.n4, kThreads)), dim3(kThreads), 0, st, pa);
    }
    ttt_status rc = check_launch("k_swa_qprep", st);
    if (rc != TTT_OK) return rc;
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
