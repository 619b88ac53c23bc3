// Backward of the TTT-KVB layer whose inner loop trains W2 alone by GD (last layer only, with or
// without momentum and the L2 norm): the outer-loop gradients that training through the parallel form needs ("TTT with KV
// Binding Is Secretly Linear Attention", Thm. 5.2-5.3, Sec. 6.1-6.2 and Fig. 4).  With W1 and W3
// frozen the layer is chunked linear attention with queries phi(q), keys phi(k), values v and state
// W2, phi(x) = SiLU(W1 x) o (W3 x) (PaperTrace "5.2.1 LaCT and TTT-E2E", Eq. (3)), so its gradients
// are those of linear attention followed by the chain rule through phi:
//   w13t   W1^T | W3^T as [d][2m] contraction operands (and W1 | W3 in bf16 for phi)
//   phi    a = x W1^T, c = x W3^T on MFMA for q and k; the epilogue writes phi = SiLU(a) c and,
//          side by side in rows of 2m, the factors u = c SiLU'(a) and w = SiLU(a)
//   linear the chunked linear-attention backward over (phi(q), phi(k), v) with state W2 -> dv,
//          deta, dW2; its dq and dk (the gradients g of phi(q), phi(k)) never leave the product
//          kernel's epilogue, which turns each u | w row into dA = g u | dC = g w in place
//   dx     dq, dk = [dA | dC] [W1; W3] on MFMA (contraction over 2m)
//   dw13   dW1 | dW3 = [dA | dC]^T x over the tokens of q and k (and the batch, for per-head
//          weights), split over token ranges into partial buffers
//   dwsum  the partials, dW_out's W1 | W3 and the scans' dW2 summed into dW0 (fixed order)
#include <algorithm>

#include "host_common.hpp"
#include "phi.hpp"
#include "tile.hpp"

namespace ttt {

// W1^T | W3^T of every weight block as [d][2m] in the io type: row j holds W1[0..m-1][j], then
// W3[0..m-1][j] (W1 and W3 are the first 2m rows of the block, each d floats long).  32 x 32 tiles
// pass through LDS; a thread loads 4 consecutive columns of one row and stores 4 of one column.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_w13t_cvt(const float* W0, int64_t w_stride, T* out, int d, int m) {
    __shared__ float tile[32][33];
    const int ni = 2 * m / 32, nj = d / 32;
    const int hw = blockIdx.x / (ni * nj), t = blockIdx.x % (ni * nj);
    const int i0 = (t / nj) * 32, j0 = (t % nj) * 32;
    {
        const int i = threadIdx.x / 8, j = (threadIdx.x % 8) * 4;
        const float4 w = *reinterpret_cast<const float4*>(W0 + hw * w_stride + (int64_t)(i0 + i) * d + j0 + j);
        tile[i][j] = w.x;
        tile[i][j + 1] = w.y;
        tile[i][j + 2] = w.z;
        tile[i][j + 3] = w.w;
    }
    __syncthreads();
    const int j = threadIdx.x / 8, i = (threadIdx.x % 8) * 4;
    Pack4<T>::store(out + ((int64_t)hw * d + j0 + j) * 2 * m + i0 + i, tile[i][j], tile[i + 1][j], tile[i + 2][j],
                    tile[i + 3][j]);
}

// dx = [dA | dC] [W1; W3] for the q and k sides: tiles of 256 tokens x 128 columns of d, the
// contraction over 2m hidden units with both operands k-contiguous ([N][2m] and [d][2m]).
template <typename T> struct DxArgs {
    const T* dac[2]; T* dx[2];  // [S][N][2m] -> [S][N][d]
    const T* Wt;                // [nw][d][2m]
    int w_heads;                // weight block of scan s: s % w_heads, or s when 0
    int64_t N; int d, m, nscan, ntt, ntd;
};

constexpr int kDxRows = 256, kDxCols = 128;

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_phi_dx(DxArgs<T> a) {
    using TO = Tile<T, kDxRows, kDxCols, 2, 2, 1, 1, 1, false, false, false, 4, 1>;
    __shared__ __attribute__((aligned(16))) char smem[TO::LDS];
    const int per = a.ntt * a.ntd;
    const int lb = xcd_block(gridDim.x);
    const int u = lb / per, t = lb % per;
    const int which = u / a.nscan, s = u % a.nscan;
    const int hw = a.w_heads ? s % a.w_heads : s;
    const int r0 = (t / a.ntd) * kDxRows, c0 = (t % a.ntd) * kDxCols;
    const int rows = (int)(a.N - r0), m2 = 2 * a.m;
    const Opnd<T> A[1] = {{a.dac[which] + ((int64_t)s * a.N + r0) * m2, m2, rows, m2}};
    const Opnd<T> B[1] = {{a.Wt + ((int64_t)hw * a.d + c0) * m2, m2, a.d - c0, m2}};
    TO tl;
    tl.template run<PM1>(A, B, m2, smem);
    T* O = a.dx[which] + ((int64_t)s * a.N + r0) * a.d + c0;
    auto epi = [&](auto check) {
        tl.for_each([&](const float (&v)[1], int row, int col) {
            if (!decltype(check)::value || (row < rows && c0 + col < a.d))
                O[(uint32_t)row * (uint32_t)a.d + (uint32_t)col] = Elt<T>::st(v[0]);
        });
    };
    if (kDxRows <= rows && c0 + kDxCols <= a.d) epi(std::false_type{});
    else epi(std::true_type{});
}

// dW1 | dW3 (rows r0.. and m + r0.. of the [2m][d] block) = [dA | dC]^T x, contracting over the
// tokens: both operands are token-major and go through the transposing stager; dA and dC share the
// x operand.  The contraction of weight block hw runs over the concatenation, batch element by
// batch element (per-head weights) and side by side (q, then k), of N tokens each; part p takes
// positions [p lp, (p + 1) lp) of it and writes partial buffer p.
template <typename T> struct DwArgs {
    const T* dac[2]; const T* x[2];  // [S][N][2m], [S][N][d]
    float* part;                     // partial p of block hw at part + (p * nw + hw) * 2 d m
    int nw, nb, H, per_head;         // weight blocks; scans per block (B when per head, else 1)
    int64_t N, lp; int d, m, ntr, ntc, nparts;
};

constexpr int kDwRows = 128, kDwCols = 128;

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_dw13(DwArgs<T> a) {
    using TW = Tile<T, kDwRows, kDwCols, 2, 2, 2, 1, 2, true, true, false, 4, 1>;
    static_assert(TW::RV_LDS <= TW::LDS, "row bands fit the tile's LDS");
    __shared__ __attribute__((aligned(16))) char smem[TW::LDS];
    const int per = a.ntr * a.ntc;
    const int lb = xcd_block(gridDim.x);
    const int u = lb / per, t = lb % per;
    const int hw = u / a.nparts, p = u % a.nparts;
    const int r0 = (t / a.ntc) * kDwRows, c0 = (t % a.ntc) * kDwCols;
    const int m2 = 2 * a.m;
    const int64_t total = (int64_t)a.nb * 2 * a.N;
    const int64_t lo = (int64_t)p * a.lp, hi = std::min(lo + a.lp, total);
    TW tl;
    tl.zero();
    // One masking variant per workgroup (a loop over both would keep both register sets live): a
    // tile whose rows and columns are all in range, over whole stages, never needs masking.
    auto segments = [&](auto full) {
        for (int64_t pos = lo; pos < hi;) {
            const int64_t seg = pos / a.N, t0 = pos % a.N;
            const int kl = (int)std::min<int64_t>(a.N - t0, hi - pos);
            const int b = (int)(seg / 2), side = (int)(seg % 2);
            const int64_t s = a.per_head ? (int64_t)b * a.H + hw : hw;
            const T* G = a.dac[side] + (s * a.N + t0) * m2;
            const T* X = a.x[side] + (s * a.N + t0) * a.d;
            const Opnd<T> A[2] = {{G + r0, m2, a.m - r0, kl}, {G + a.m + r0, m2, a.m - r0, kl}};
            const Opnd<T> B[1] = {{X + c0, a.d, a.d - c0, kl}};
            if (pos > lo) lds_barrier();  // every wave is done with the previous segment's last stage
            tl.template run_<PMG, decltype(full)::value>(A, B, kl, smem, true);
            pos += kl;
        }
    };
    if (r0 + TW::BM <= a.m && c0 + TW::BN <= a.d && a.N % TW::KSTEP == 0 && a.lp % TW::KSTEP == 0)
        segments(std::true_type{});
    else
        segments(std::false_type{});
    // 32-bit offsets from the tile corner
    float* G1 = a.part + ((int64_t)p * a.nw + hw) * m2 * a.d + (int64_t)r0 * a.d + c0;
    float* G3 = G1 + (int64_t)a.m * a.d;
    if (r0 + TW::BM <= a.m && c0 + TW::BN <= a.d) {
        // full tiles: both operands' staging permutes rows and columns, so rows are gathered in LDS
        // and leave as whole 512-byte row segments
        tl.rows_via_lds(smem, [&](int, int q, int row, int col, const float4& v) {
            *reinterpret_cast<float4*>((q ? G3 : G1) + (uint32_t)row * (uint32_t)a.d + (uint32_t)col) = v;
        });
    } else {
        tl.for_each([&](const float (&v)[2], int row, int col) {
            if (r0 + row < a.m && c0 + col < a.d) {
                const uint32_t off = (uint32_t)row * (uint32_t)a.d + (uint32_t)col;
                G1[off] = v[0];
                G3[off] = v[1];
            }
        });
    }
}

// dW0 of weight block hw, 4 consecutive elements per thread, summed in a fixed order:
//   W1 | W3 part: the partial buffers in order, then dW_out's W1 | W3 of the block's scans;
//   W2 part: the block's scans' dW2 (which already hold dW_out's W2).
struct DwSumArgs {
    const float* part; int nparts;  // [nparts][nw][2dm], or null
    const float* dW2;               // [S][dm]
    const float* dWo;               // [S][3dm], or null
    float* dW0;                     // [nw][3dm]
    int nw, nb, H, per_head;
    int64_t dm;
};

__global__ __launch_bounds__(kThreads) void k_dw_sum(DwSumArgs a) {
    const int64_t per = 3 * a.dm / 4;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= per * a.nw) return;
    const int hw = (int)(g / per);
    const int64_t e = (g % per) * 4;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto scan = [&](int b) -> int64_t { return a.per_head ? (int64_t)b * a.H + hw : hw; };
    if (e < 2 * a.dm) {
        if (a.part)
            for (int p = 0; p < a.nparts; ++p)
                acc += *reinterpret_cast<const f32x4_t*>(a.part + ((int64_t)p * a.nw + hw) * 2 * a.dm + e);
        if (a.dWo)
            for (int b = 0; b < a.nb; ++b) acc += *reinterpret_cast<const f32x4_t*>(a.dWo + scan(b) * 3 * a.dm + e);
    } else {
        for (int b = 0; b < a.nb; ++b)
            acc += *reinterpret_cast<const f32x4_t*>(a.dW2 + scan(b) * a.dm + (e - 2 * a.dm));
    }
    *reinterpret_cast<f32x4_t*>(a.dW0 + (int64_t)hw * 3 * a.dm + e) = acc;
}

// ---------------------------------------------------------------------------------------------
// host driver

// Token parts of the weight-gradient contraction: the count in 1 .. 16 whose launch (tiles x parts
// workgroups, two per CU on 256 CUs) leaves the least idle share in its last round, keeping every
// part at least 1024 positions long; ties go to fewer parts.  Depends on the descriptor only.
static int dw_parts(int64_t tiles, int64_t total) {
    int best = 1;
    double best_eff = 0.0;
    for (int p = 1; p <= 16; ++p) {
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

struct BLayout {
    size_t w13, w13t, ph[2], dac[2], dw2, part, lin, total;
    int nparts;
    int64_t lp;
};

static linattn_desc lin_desc_of(const ttt_desc& D) {
    return linattn_desc{D.B, D.H, D.N, D.m_h, D.d_h, D.chunk, D.io_dtype, D.mask, D.update_chunks};
}

static BLayout make_blayout(const ttt_desc& D, bool want_dw) {
    BLayout L{};
    const int64_t S = (int64_t)D.B * D.H, d = D.d_h, m = D.m_h, dm = d * m;
    const int64_t nw = D.w0_per_batch ? S : D.H;
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    if (D.N > 0) {
        if (es == 2) L.w13 = take((size_t)nw * 2 * dm * es);
        L.w13t = take((size_t)nw * 2 * dm * es);
        for (int i = 0; i < 2; ++i) L.ph[i] = take((size_t)S * D.N * m * es);
        for (int i = 0; i < 2; ++i) L.dac[i] = take((size_t)S * D.N * 2 * m * es);  // u | w, then dA | dC
    }
    if (want_dw) {
        L.dw2 = take((size_t)S * dm * 4);
        if (D.N > 0) {
            const int64_t nb = D.w0_per_batch ? 1 : D.B, total = nb * 2 * D.N;
            const int64_t tiles = nw * cdiv(m, kDwRows) * cdiv(d, kDwCols);
            L.nparts = dw_parts(tiles, total);
            L.lp = cdiv(cdiv(total, L.nparts), 64) * 64;
            L.part = take((size_t)L.nparts * nw * 2 * dm * 4);
        }
    }
    L.lin = take(lin_chunked_bwd_ws_bytes(lin_desc_of(D), D.rule == TTT_UPD_GD_L2, D.inner_steps > 1 ? D.inner_steps : 1));
    L.total = off;
    return L;
}

// whether the backward runs as the reverse of the recurrence (all weights learning, or Muon) rather
// than through linear attention over phi (W2 alone, GD or GD + L2)
static bool uses_full(const ttt_desc& D) {
    return !D.last_layer_only || D.rule == TTT_UPD_MUON || D.rule == TTT_UPD_MUON_L2;
}

static ttt_status validate_bwd(const ttt_desc* D) {
    ttt_status rc = validate_ttt_desc(D);
    if (rc != TTT_OK) return rc;
    // all three weights learning, or Muon: the reverse of the recurrence
    if (!D->last_layer_only || D->rule == TTT_UPD_MUON || D->rule == TTT_UPD_MUON_L2) return validate_full_bwd(D);
    if ((D->rule != TTT_UPD_GD && D->rule != TTT_UPD_GD_L2) || D->chunk_rates)
        return fail(TTT_ERR_UNSUPPORTED,
                    "the backward covers the layer whose inner loop trains W2 alone by GD (with or without momentum "
                    "and the L2 norm): last_layer_only = 1, rule TTT_UPD_GD or TTT_UPD_GD_L2, per-token rates");
    const int64_t S = (int64_t)D->B * D->H, nc = D->N > 0 ? cdiv(D->N, D->chunk) : 0;
    if (D->mask == TTT_MASK_STRIDED && nc > 32 * 32)
        return fail(TTT_ERR_UNSUPPORTED, "the backward with MASK_STRIDED supports at most 1024 chunks");
    const linattn_desc LD = lin_desc_of(*D);
    // the linear-attention checks over (phi(q), phi(k), v): d_k = m_h, d_v = d_h
    const ttt_status lr = validate_lin_desc_bwd(&LD);
    if (lr != TTT_OK) return lr;
    const int64_t lim = 1LL << 31, nw = D->w0_per_batch ? S : D->H;
    if (2 * S * cdiv(D->N, kPhiRows) * cdiv(D->m_h, kPhiCols) >= lim ||
        2 * S * cdiv(D->N, kDxRows) * cdiv(D->d_h, kDxCols) >= lim ||
        16 * nw * cdiv(D->m_h, kDwRows) * cdiv(D->d_h, kDwCols) >= lim || nw * 2 * D->m_h / 32 * (D->d_h / 32) >= lim ||
        S * 3 * (int64_t)D->d_h * D->m_h / 4 >= lim * kThreads)
        return fail(TTT_ERR_UNSUPPORTED, "B*H, N, d_h, m_h too large for one launch");
    return TTT_OK;
}

template <typename T>
static ttt_status run_backward(const ttt_desc& D, const BLayout& L, const T* q, const T* k, const T* v,
                               const float* eta, const float* W0, const T* dO, const float* dWo, T* dq, T* dk, T* dv,
                               float* deta, float* dW0, char* ws, hipStream_t st) {
    const int64_t S = (int64_t)D.B * D.H, d = D.d_h, m = D.m_h, dm = d * m;
    const int64_t nw = D.w0_per_batch ? S : D.H;
    const int w_heads = D.w0_per_batch ? 0 : D.H;
    ttt_status rc;
    T* ph[2] = {(T*)(ws + L.ph[0]), (T*)(ws + L.ph[1])};
    T* dac[2] = {(T*)(ws + L.dac[0]), (T*)(ws + L.dac[1])};
    T* Wt = (T*)(ws + L.w13t);
    float* dW2 = dW0 ? (float*)(ws + L.dw2) : nullptr;
    if (D.N > 0) {
        // 1. W1 | W3 and W1^T | W3^T as contraction operands
        const T* W13;
        int64_t w13_stride;
        if constexpr (sizeof(T) == 2) {
            T* w = (T*)(ws + L.w13);
            const int64_t per4 = 2 * dm / 4, n4 = nw * per4;
            {
                ProfScope ps(PK_W13, st);
                hipLaunchKernelGGL(k_w13_cvt<T>, dim3((unsigned)cdiv(n4, kThreads)), dim3(kThreads), 0, st, W0, 3 * dm,
                                   w, n4, per4);
            }
            if ((rc = check_launch("k_w13_cvt", st)) != TTT_OK) return rc;
            W13 = w;
            w13_stride = 2 * dm;
        } else {
            W13 = reinterpret_cast<const T*>(W0);
            w13_stride = 3 * dm;
        }
        {
            ProfScope ps(PK_W13T, st);
            hipLaunchKernelGGL(k_w13t_cvt<T>, dim3((unsigned)(nw * (2 * m / 32) * (d / 32))), dim3(kThreads), 0, st,
                               W0, 3 * dm, Wt, (int)d, (int)m);
        }
        if ((rc = check_launch("k_w13t_cvt", st)) != TTT_OK) return rc;
        // 2. the features of every query and key, and the factors u | w of their backward
        PhiArgs<T> pa{{q, k}, {ph[0], ph[1]}, {dac[0], dac[1]}, W13, w13_stride, w_heads, D.N, (int)d, (int)m,
                      (int)S, (int)cdiv(D.N, kPhiRows), (int)cdiv(m, kPhiCols)};
        {
            ProfScope ps(PK_PHI, st);
            hipLaunchKernelGGL((k_phi<T, true>), dim3((unsigned)(2 * S * pa.ntt * pa.nct)), dim3(64 * kPhiWaves), 0,
                               st, pa);
        }
        if ((rc = check_launch("k_phi", st)) != TTT_OK) return rc;
    }
    // 3. the linear-attention backward with state W2 (the W2 block of each weight block)
    const linattn_desc LD = lin_desc_of(D);
    uint32_t flags[32] = {};
    if (D.mask == TTT_MASK_STRIDED)
        for (int64_t j = 0; j < cdiv(D.N, D.chunk); ++j)
            if (D.update_chunks[j]) flags[j >> 5] |= 1u << (j & 31);
    LinBwdIO io;
    io.S0 = W0 + 2 * dm;
    io.s0_stride = 3 * dm;
    io.s0_heads = w_heads;
    io.dS_out = dWo ? dWo + 2 * dm : nullptr;
    io.dso_stride = 3 * dm;
    io.dS0 = dW2;
    io.ds0_stride = dm;
    io.dsign = D.ascent ? -1.0f : 1.0f;
    io.reps = D.inner_steps > 1 ? D.inner_steps : 1;
    if (D.momentum != 0.0f) {  // M <- beta M + g, W2 <- W2 - M: the running term is m = -M, from zero
        io.mom = 1;
        io.beta = D.momentum;
    }
    io.norm = D.rule == TTT_UPD_GD_L2;  // W2's rows L2-normalized after every step
    if (D.N > 0) {  // the gradients of phi(q), phi(k) turn u | w into dA | dC
        io.gate[0] = dac[0];
        io.gate[1] = dac[1];
    }
    if ((rc = lin_chunked_bwd<T>(LD, flags, ph[0], ph[1], v, eta, dO, io, nullptr, nullptr, dv, deta, ws + L.lin,
                                 st)) != TTT_OK)
        return rc;
    if (D.N > 0) {
        // 4. dq, dk
        DxArgs<T> xa{{dac[0], dac[1]}, {dq, dk}, Wt, w_heads, D.N, (int)d, (int)m, (int)S,
                     (int)cdiv(D.N, kDxRows), (int)cdiv(d, kDxCols)};
        {
            ProfScope ps(PK_PHI_DX, st);
            hipLaunchKernelGGL(k_phi_dx<T>, dim3((unsigned)(2 * S * xa.ntt * xa.ntd)), dim3(kThreads), 0, st, xa);
        }
        if ((rc = check_launch("k_phi_dx", st)) != TTT_OK) return rc;
        // 5. dW1 | dW3 partials
        if (dW0) {
            DwArgs<T> wa{{dac[0], dac[1]}, {q, k}, (float*)(ws + L.part), (int)nw, D.w0_per_batch ? 1 : D.B, D.H,
                         D.w0_per_batch ? 0 : 1, D.N, L.lp, (int)d, (int)m, (int)cdiv(m, kDwRows),
                         (int)cdiv(d, kDwCols), L.nparts};
            {
                ProfScope ps(PK_DW13, st);
                hipLaunchKernelGGL(k_dw13<T>, dim3((unsigned)(nw * L.nparts * wa.ntr * wa.ntc)), dim3(kThreads), 0,
                                   st, wa);
            }
            if ((rc = check_launch("k_dw13", st)) != TTT_OK) return rc;
        }
    }
    // 6. dW0
    if (dW0) {
        DwSumArgs sa{D.N > 0 ? (const float*)(ws + L.part) : nullptr, L.nparts, dW2, dWo, dW0, (int)nw,
                     D.w0_per_batch ? 1 : D.B, D.H, D.w0_per_batch ? 0 : 1, dm};
        {
            ProfScope ps(PK_DW_SUM, st);
            hipLaunchKernelGGL(k_dw_sum, dim3((unsigned)cdiv(nw * 3 * dm / 4, kThreads)), dim3(kThreads), 0, st, sa);
        }
        if ((rc = check_launch("k_dw_sum", st)) != TTT_OK) return rc;
    }
    return TTT_OK;
}

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_backward_workspace_bytes(const ttt_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_bwd(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = uses_full(*desc) ? full_bwd_ws_bytes(*desc) : make_blayout(*desc, true).total;
    return TTT_OK;
}

namespace {
// The argument checks of the backward entry points: required and aligned pointers, no output over
// an input or another output, a workspace of `need` bytes, and every buffer inside a HIP allocation.
// W0 or the record (rec, rec_bytes) is the weights' source.
ttt_status check_bwd_args(const ttt_desc& D, const void* q, const void* k, const void* v, const float* eta,
                          const float* W0, const void* rec, size_t rec_bytes, const void* dO, const float* dW_out,
                          void* dq, void* dk, void* dv, float* deta, float* dW0, void* workspace,
                          size_t workspace_bytes, size_t need) {
    const int64_t S = (int64_t)D.B * D.H;
    const bool t = D.N > 0;
    if (!W0 && !rec) return fail(TTT_ERR_INVALID_ARGUMENT, rec_bytes ? "record is NULL" : "W0 is NULL");
    if (t && (!q || !k || !v || !eta || !dO || !dq || !dk || !dv || !deta))
        return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, eta, dO, dq, dk, dv and deta are required");
    const void* p16[] = {q, k, v, dO, dq, dk, dv, W0, dW_out, dW0};
    for (const void* p : p16)
        if (p && !aligned(p, 16))
            return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, dO, dq, dk, dv, W0, dW_out, dW0 must be 16-byte aligned");
    if (rec && !aligned(rec, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "record must be 256-byte aligned");
    const void* p4[] = {eta, deta};
    for (const void* p : p4)
        if (p && !aligned(p, 4)) return fail(TTT_ERR_INVALID_ARGUMENT, "eta and deta must be 4-byte aligned");
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const int64_t dm3 = 3 * (int64_t)D.d_h * D.m_h;
    const size_t xb = t ? (size_t)S * D.N * D.d_h * es : 0, eb = t ? (size_t)S * D.N * 4 : 0;
    const size_t wb = (size_t)(D.w0_per_batch ? S : D.H) * dm3 * 4, wob = (size_t)S * dm3 * 4;
    const struct { const void* p; size_t n; const char* name; } ins[] = {
        {q, xb, "q"}, {k, xb, "k"}, {v, xb, "v"}, {eta, eb, "eta"}, {W0, wb, "W0"}, {rec, rec_bytes, "record"},
        {dO, xb, "dO"}, {dW_out, wob, "dW_out"}};
    const struct { const void* p; size_t n; const char* name; } outs[] = {
        {dq, xb, "dq"}, {dk, xb, "dk"}, {dv, xb, "dv"}, {deta, eb, "deta"}, {dW0, wb, "dW0"}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const auto& in : ins)
            if (overlaps(outs[i].p, outs[i].n, in.p, in.n))
                return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps the input %s", outs[i].name, in.name);
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    if (need && (!workspace || workspace_bytes < need))
        return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (need && !aligned(workspace, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    ttt_status rc;
    for (const auto& b : ins)
        if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    for (const auto& b : outs)
        if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    return check_buffer(workspace, need, "workspace");
}
}  // namespace

extern "C" ttt_status ttt_backward(const ttt_desc* desc, const void* q, const void* k, const void* v, const float* eta,
                                   const float* W0, const void* dO, const float* dW_out, void* dq, void* dk, void* dv,
                                   float* deta, float* dW0, void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    ttt_status rc = validate_bwd(desc);
    if (rc != TTT_OK) return rc;
    const ttt_desc& D = *desc;
    if ((int64_t)D.B * D.H == 0) return TTT_OK;
    const bool full = uses_full(D);
    const BLayout L = full ? BLayout{} : make_blayout(D, dW0 != nullptr);
    const size_t need = full ? full_bwd_ws_bytes(D) : L.total;
    if ((rc = check_bwd_args(D, q, k, v, eta, W0, nullptr, 0, dO, dW_out, dq, dk, dv, deta, dW0, workspace,
                             workspace_bytes, need)) != TTT_OK)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    if (full) {
        if (D.io_dtype == TTT_BF16)
            return run_full_backward<uint16_t>(D, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta, W0,
                                               (const uint16_t*)dO, dW_out, (uint16_t*)dq, (uint16_t*)dk,
                                               (uint16_t*)dv, deta, dW0, (char*)workspace, st);
        return run_full_backward<float>(D, (const float*)q, (const float*)k, (const float*)v, eta, W0,
                                        (const float*)dO, dW_out, (float*)dq, (float*)dk, (float*)dv, deta, dW0,
                                        (char*)workspace, st);
    }
    if (D.io_dtype == TTT_BF16)
        return run_backward<uint16_t>(D, L, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta, W0,
                                      (const uint16_t*)dO, dW_out, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, deta,
                                      dW0, (char*)workspace, st);
    return run_backward<float>(D, L, (const float*)q, (const float*)k, (const float*)v, eta, W0, (const float*)dO,
                               dW_out, (float*)dq, (float*)dk, (float*)dv, deta, dW0, (char*)workspace, st);
}

// The training pair: the forward that keeps a record, and the backward that reads it.
// The pair always walks the recurrence back, the layer whose inner loop trains W2 alone by GD
// included (ttt_backward takes that one through linear attention instead, as its parallel form does)
static ttt_status validate_record(const ttt_desc* desc) {
    ttt_status rc = validate_ttt_desc(desc);
    if (rc != TTT_OK) return rc;
    return validate_full_bwd(desc);
}

extern "C" ttt_status ttt_record_bytes(const ttt_desc* desc, size_t* record_bytes, size_t* workspace_bytes) {
    clear_error();
    ttt_status rc = validate_record(desc);
    if (rc != TTT_OK) return rc;
    if (!record_bytes || !workspace_bytes)
        return fail(TTT_ERR_INVALID_ARGUMENT, "record_bytes and workspace_bytes are required");
    *record_bytes = full_bwd_record_bytes(*desc);
    *workspace_bytes = ttt_history_ws_bytes(*desc);
    return TTT_OK;
}

extern "C" ttt_status ttt_forward_record(const ttt_desc* desc, const void* q, const void* k, const void* v,
                                         const float* eta, const float* W0, void* o, float* W_out, void* record,
                                         size_t record_bytes, void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    ttt_status rc = validate_record(desc);
    if (rc != TTT_OK) return rc;
    const ttt_desc& D = *desc;
    const int64_t S = (int64_t)D.B * D.H;
    if (S == 0) return TTT_OK;
    const bool t = D.N > 0;
    if (!W0 || !record) return fail(TTT_ERR_INVALID_ARGUMENT, "W0 and record are required");
    if (t && (!q || !k || !v || !eta || !o)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, eta and o are required");
    const void* p16[] = {q, k, v, o, W0, W_out};
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, o, W0, W_out must be 16-byte aligned");
    if (eta && !aligned(eta, 4)) return fail(TTT_ERR_INVALID_ARGUMENT, "eta must be 4-byte aligned");
    if (!aligned(record, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "record must be 256-byte aligned");
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const int64_t dm3 = 3 * (int64_t)D.d_h * D.m_h;
    const size_t xb = t ? (size_t)S * D.N * D.d_h * es : 0, eb = t ? (size_t)S * D.N * 4 : 0;
    const size_t wb = (size_t)(D.w0_per_batch ? S : D.H) * dm3 * 4, wob = (size_t)S * dm3 * 4;
    const size_t rb = full_bwd_record_bytes(D), need = ttt_history_ws_bytes(D);
    if (record_bytes < rb) return fail(TTT_ERR_WORKSPACE, "record of %zu bytes needed, %zu given", rb, record_bytes);
    if (need && (!workspace || workspace_bytes < need))
        return fail(TTT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    if (need && !aligned(workspace, 256)) return fail(TTT_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    const struct { const void* p; size_t n; const char* name; } ins[] = {
        {q, xb, "q"}, {k, xb, "k"}, {v, xb, "v"}, {eta, eb, "eta"}, {W0, wb, "W0"}};
    const struct { const void* p; size_t n; const char* name; } outs[] = {
        {o, xb, "o"}, {W_out, wob, "W_out"}, {record, rb, "record"}, {workspace, need, "workspace"}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const auto& in : ins)
            if (overlaps(outs[i].p, outs[i].n, in.p, in.n))
                return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps the input %s", outs[i].name, in.name);
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(TTT_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    for (const auto& b : ins)
        if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    for (const auto& b : outs)
        if ((rc = check_buffer(b.p, b.n, b.name)) != TTT_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (D.io_dtype == TTT_BF16)
        return run_forward_record<uint16_t>(D, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta, W0,
                                            (uint16_t*)o, W_out, (char*)record, (char*)workspace, st);
    return run_forward_record<float>(D, (const float*)q, (const float*)k, (const float*)v, eta, W0, (float*)o, W_out,
                                     (char*)record, (char*)workspace, st);
}

extern "C" ttt_status ttt_backward_record_workspace_bytes(const ttt_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_record(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = full_bwd_ws_bytes(*desc, false);
    return TTT_OK;
}

extern "C" ttt_status ttt_backward_record(const ttt_desc* desc, const void* q, const void* k, const void* v,
                                          const float* eta, const void* record, size_t record_bytes, const void* dO,
                                          const float* dW_out, void* dq, void* dk, void* dv, float* deta, float* dW0,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    ttt_status rc = validate_record(desc);
    if (rc != TTT_OK) return rc;
    const ttt_desc& D = *desc;
    if ((int64_t)D.B * D.H == 0) return TTT_OK;
    const size_t rb = full_bwd_record_bytes(D);
    if (!record) return fail(TTT_ERR_INVALID_ARGUMENT, "record is NULL");
    if (record_bytes < rb) return fail(TTT_ERR_WORKSPACE, "record of %zu bytes needed, %zu given", rb, record_bytes);
    if ((rc = check_bwd_args(D, q, k, v, eta, nullptr, record, rb, dO, dW_out, dq, dk, dv, deta, dW0, workspace,
                             workspace_bytes, full_bwd_ws_bytes(D, false))) != TTT_OK)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    // the record is read only; the backward's own buffers are all in the workspace
    char* rec = const_cast<char*>(reinterpret_cast<const char*>(record));
    if (D.io_dtype == TTT_BF16)
        return run_full_backward<uint16_t>(D, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta, nullptr,
                                           (const uint16_t*)dO, dW_out, (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv,
                                           deta, dW0, (char*)workspace, st, rec);
    return run_full_backward<float>(D, (const float*)q, (const float*)k, (const float*)v, eta, nullptr,
                                    (const float*)dO, dW_out, (float*)dq, (float*)dk, (float*)dv, deta, dW0,
                                    (char*)workspace, st, rec);
}
