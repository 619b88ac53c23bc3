// The large-chunk TTT-KVB layer on gfx950: SwiGLU fast weight f_W(x) = W2 [SiLU(W1 x) o (W3 x)]
// (PaperTrace "5.2.1 LaCT and TTT-E2E", Eq. (3)), dot-product loss (Eq. (4)), one gradient step per
// chunk (Eq. (2)) followed by W - U, L2-Normalize(W - U) (Eq. (5)) or Muon (Eq. (6)), in the
// update/apply order of the notes' section 1.1 and Eq. (10).
//
// Every (batch, head) scan is independent; all scans advance one chunk per step in lock-step, and a
// step is a short sequence of grid-wide launches on one stream:
//   up    [Q_a; K_u] x [W1; W3]^T and V_u x W2 on MFMA, with the SwiGLU forward and backward in
//         the epilogue -> Hq = SiLU(Aq) o Cq, HkE = -eta o Hk, DA, DC (token-major, io dtype)
//   down  O_a = Hq W2^T (queries of the apply chunk) and the chunk gradients
//         G1 = DA^T K, G3 = DC^T K, G2 = V^T HkE (contractions over the chunk's tokens)
//   [muon] momentum + Frobenius partial sums, scale, ns_iters x (Gram, polynomial step)
//   update W <- [norm](W - U) row-wise, fp32 master copy plus io-dtype shadows for the MFMAs
// The fp32 fast weights live in a ping-pong pair in the workspace; the shadows (W1, W3, W2, W2^T)
// are what the next chunk's MFMAs read.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "host_common.hpp"
#include "phi.hpp"
#include "tile.hpp"

namespace ttt {

constexpr int kUpWaves = 8;     // up-kernel workgroups: 8 waves, one workgroup per CU
constexpr int kUpQRows = 256;   // token rows per query tile
constexpr int kUpKRows = 192;   // token rows per key tile
constexpr int kUpCols = 128;    // hidden units per up-kernel tile
constexpr int kORows = 256;     // token rows per output tile
constexpr int kPanelShift = 6;  // intermediates are stored in panels of 64 hidden units
constexpr int kPanel = 1 << kPanelShift;

// Chunk intermediates of one scan.  Hq (read by the output GEMM, which contracts over hidden
// units) is token-major in panels: hidden unit h of token t is element (h / 64) * pan + t * 64 +
// h % 64, with pan = 64 x (chunk capacity), so a query tile writes one contiguous block.  HkE, DA
// and DC (read by the gradient GEMMs, which contract over tokens) are hidden-major in blocks of
// kHB hidden units x kTB tokens: element ((h / kHB) * ntb + t / kTB) * kHB * kTB + (h % kHB) * kTB +
// t % kTB, with ntb token blocks per chunk capacity.  A gradient tile's k-step (128 or 256 hidden
// units x 64 tokens) is then one contiguous 16 or 32 KB piece, where rows a chunk apart would
// each open their own DRAM page, and a key tile writes contiguous 16 KB pieces.
constexpr int kHB = 256, kTB = 64, kTBShift = 6, kBlk = kHB * kTB;
template <typename T> struct StepArgs {
    const T* q; const T* k; const T* v; const float* eta; T* o;
    int64_t N; int d, m;
    T* Hq; T* HkE; T* DA; T* DC; int64_t inter_stride;  // per-scan intermediates
    int64_t pan;                                          // Hq panel stride (elements)
    int ntb;                                              // HkE / DA / DC token blocks per chunk
    const T* sh; int64_t sh_stride;                       // shadows [W1 | W3 | W2 | W2^T]
    float* G; int64_t g_stride;                           // [G1 | G3 | G2] fp32
    int64_t a0; int la;                                   // apply chunk: first token, length
    int64_t u0; int lu;                                   // update chunk
    int nQ, nK;                                           // up-kernel workgroups per scan
    int nG13, nG2, nO;                                    // down-kernel tiles per scan
    float eta_sign;                                       // -1: gradient ascent
    int ksplit, kpart;                                    // gradient tiles: token parts, tokens per part
    int64_t gpart_stride;                                 // elements between partial-G buffers
};

template <typename T> __device__ __forceinline__ int64_t panel_off(const StepArgs<T>& a, int t, int h) {
    return (int64_t)(h >> kPanelShift) * a.pan + (int64_t)t * kPanel + (h & (kPanel - 1));
}

// ---------------------------------------------------------------------------------------------
// up: SwiGLU forward of the queries, forward + backward of the keys.  Workgroups of 8 waves (two
// per SIMD, one workgroup per CU): each wave keeps the accumulator blocking of a 4-wave tile while
// the workgroup tile doubles, which halves the operand bytes loaded per MFMA.  Key tiles are
// computed transposed (hidden units x tokens): each lane then holds consecutive tokens of one
// hidden unit, so the hidden-major HkE, DA, DC leave as contiguous runs, and eta is one value per
// lane column.
template <typename T>
__global__ __launch_bounds__(64 * kUpWaves, 1) void k_up(StepArgs<T> a) {
    // query wave: 64 tokens x 64 hidden x {A, C}; key wave: 32 hidden x 96 tokens x {A, C, DH}
    using TQ = Tile<T, kUpQRows, kUpCols, 2, 4, 1, 2, 2, false, false, false, kUpWaves>;
    // key tiles run two passes over d, each with two 64-wide LDS stages: W1, W3 x K, then W2^T x V
    using TK1 = Tile<T, kUpCols, kUpKRows, 2, 4, 2, 1, 2, false, false, false, kUpWaves>;
    using TK2 = Tile<T, kUpCols, kUpKRows, 2, 4, 1, 1, 1, false, false, false, kUpWaves>;
    constexpr int LDSB = std::max(TQ::LDS, std::max(TK1::LDS, TK2::LDS));
    __shared__ __attribute__((aligned(16))) char smem[LDSB];

    const int per = a.nQ + a.nK;
    const int lb = xcd_block(gridDim.x);
    const int s = lb / per, t = lb % per;
    const int64_t dm = (int64_t)a.d * a.m;
    const T* sh = a.sh + s * a.sh_stride;
    const T* W1s = sh;
    const T* W3s = sh + dm;
    const T* W2Ts = sh + 3 * dm;
    const int64_t ioff = s * a.inter_stride;

    if (t < a.nQ) {
        const int nct = (a.m + kUpCols - 1) / kUpCols;
        const int r0 = (t / nct) * kUpQRows, c0 = (t % nct) * kUpCols;
        const T* Q = a.q + ((int64_t)s * a.N + a.a0 + r0) * a.d;
        const Opnd<T> A[1] = {{Q, a.d, a.la - r0, a.d}};
        const Opnd<T> B[2] = {{W1s + (int64_t)c0 * a.d, a.d, a.m - c0, a.d},
                              {W3s + (int64_t)c0 * a.d, a.d, a.m - c0, a.d}};
        TQ tl;
        tl.template run<PMQ>(A, B, a.d, smem);
        // the tile's hidden units span whole panels: element (row, col) is (col / 64) * pan +
        // row * 64 + col % 64 from the tile corner
        static_assert(kUpCols % kPanel == 0, "a query tile must cover whole panels");
        T* Hq = a.Hq + ioff + panel_off(a, r0, c0);
        auto epi = [&](auto check) {
            tl.for_each([&](const float (&v)[2], int row, int col) {
                if (!decltype(check)::value || (r0 + row < a.la && c0 + col < a.m))
                    Hq[(col >> kPanelShift) * a.pan + (uint32_t)row * kPanel + (uint32_t)(col & (kPanel - 1))] =
                        Elt<T>::st(v[0] * sigmoidf_(v[0]) * v[1]);
            });
        };
        if (r0 + kUpQRows <= a.la && c0 + kUpCols <= a.m) epi(std::false_type{});
        else epi(std::true_type{});
    } else {
        const int nct = (a.m + kUpCols - 1) / kUpCols;
        const int tt = t - a.nQ;
        const int r0 = (tt / nct) * kUpKRows, c0 = (tt % nct) * kUpCols;
        const int64_t tok = (int64_t)s * a.N + a.u0 + r0;
        const Opnd<T> A1[2] = {{W1s + (int64_t)c0 * a.d, a.d, a.m - c0, a.d},
                               {W3s + (int64_t)c0 * a.d, a.d, a.m - c0, a.d}};
        const Opnd<T> B1[1] = {{a.k + tok * a.d, a.d, a.lu - r0, a.d}};
        const Opnd<T> A2[1] = {{W2Ts + (int64_t)c0 * a.d, a.d, a.m - c0, a.d}};
        const Opnd<T> B2[1] = {{a.v + tok * a.d, a.d, a.lu - r0, a.d}};
        TK1 tl;  // (K W1^T, K W3^T) transposed
        TK2 tp;  // (V W2) transposed
        // the second pass's first stage is loaded before the first pass starts, so its latency
        // does not open the second pass
        typename TK2::Regs g2;
        const bool f2 = TK2::full(A2, B2, a.d) && a.d > 0;
        if (f2) TK2::template issue<true>(g2, A2, B2, 0);
        tl.template run<PMG>(A1, B1, a.d, smem);
        if (f2) tp.template run_issued<PM1, true>(g2, A2, B2, a.d, smem);
        else tp.template run<PM1>(A2, B2, a.d, smem);
        const float* eta = a.eta ? a.eta + tok : nullptr;  // null: every token weighs 1
        // the tile's hidden units lie in one block (c0 % kHB is 0 or 128) and its tokens start a
        // token block (r0 % kTB == 0)
        static_assert(kHB % kUpCols == 0 && kUpKRows % kTB == 0, "key tiles must align with the blocks");
        const int64_t boff = ioff + ((int64_t)(c0 / kHB) * a.ntb + r0 / kTB) * kBlk + (int64_t)(c0 % kHB) * kTB;
        T* HkE = a.HkE + boff;
        T* DA = a.DA + boff;
        T* DC = a.DC + boff;
        // SwiGLU backward at one (token, hidden unit): x = (K W1^T), c = (K W3^T), p = (V W2) there
        auto bwd = [](float x, float c, float p, float e, float& hk, float& da, float& dc) {
            const float sg = sigmoidf_(x), xs = x * sg;
            const float dh = -e * p;  // dLoss/dH = -eta (V W2)
            hk = -e * xs * c;         // -eta o SiLU(A) o C
            da = dh * c * (sg + xs * (1.f - sg));
            dc = dh * xs;
        };
        // tile row = hidden unit c0 + row, tile column = token r0 + col
        // both tiles have the same wave layout: accumulator element idx of one is at the same
        // (row, col) as in the other
        auto epi = [&](auto check) {
            TK1::for_each_pos([&](int idx, int row, int col) {
                const int i = idx / (TK1::FN * 16), j = (idx / 16) % TK1::FN, r = idx % 16;
                if (!decltype(check)::value || (r0 + col < a.lu && c0 + row < a.m)) {
                    float hk, da, dc;
                    bwd(tl.acc[0][i][j][r], tl.acc[1][i][j][r], tp.acc[0][i][j][r], a.eta_sign * (eta ? eta[col] : 1.0f), hk, da, dc);
                    const uint32_t off = (uint32_t)(col >> kTBShift) * kBlk + (uint32_t)row * kTB + (uint32_t)(col & (kTB - 1));
                    HkE[off] = Elt<T>::st(hk);
                    DA[off] = Elt<T>::st(da);
                    DC[off] = Elt<T>::st(dc);
                }
            });
        };
        if (r0 + kUpKRows <= a.lu && c0 + kUpCols <= a.m) epi(std::false_type{});
        else epi(std::true_type{});
    }
}

// ---------------------------------------------------------------------------------------------
// down: chunk gradients (contractions over tokens) and the apply chunk's outputs
template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_down(StepArgs<T> a) {
    // 64-wide k-steps (whole 128-byte lines per row) in a single LDS stage, two workgroups per CU
    using TG13 = Tile<T, 128, 128, 2, 2, 2, 1, 2, false, true, false, 4, 1>;  // G1 and G3 share the K operand
    using TG2 = Tile<T, 128, 256, 2, 2, 1, 1, 1, true, false, false, 4, 1>;
    using TO = Tile<T, kORows, 128, 2, 2, 1, 1, 1, false, false, false, 4, 1>;
    constexpr int L1 = TG13::LDS > TG2::LDS ? TG13::LDS : TG2::LDS;
    constexpr int LDSB = L1 > TO::LDS ? L1 : TO::LDS;
    __shared__ __attribute__((aligned(16))) char smem[LDSB];

    // Each XCD (blocks b with the same b % 8) takes a contiguous group of scans, so tiles that share
    // operands share an L2; within its group it runs the longest tiles first (the G1/G3 tiles of all
    // its scans, then G2, then the outputs), so that short output tiles fill the end of the launch.
    const int per = a.nG13 + a.nG2 + a.nO;
    const int S = gridDim.x / per;
    int s, t;
    if (S % 8 == 0) {
        const int sp = S / 8, x = blockIdx.x % 8;
        int i = blockIdx.x / 8;
        if (i < sp * a.nG13) {  // last scan first: the up kernel wrote its DA, DC last
            s = sp - 1 - i / a.nG13; t = i % a.nG13;
        } else if ((i -= sp * a.nG13) < sp * a.nG2) {
            s = sp - 1 - i / a.nG2; t = a.nG13 + i % a.nG2;
        } else {
            i -= sp * a.nG2;
            s = i / a.nO; t = a.nG13 + a.nG2 + i % a.nO;
        }
        s += x * sp;
    } else {
        const int lb = xcd_block(gridDim.x);
        s = lb / per;
        t = lb % per;
    }
    const int64_t dm = (int64_t)a.d * a.m;
    const int ndt = (a.d + 127) / 128, nmt2 = (a.m + 255) / 256;
    const int64_t ioff = s * a.inter_stride;
    // With few scans the gradient tiles are split over the chunk's tokens: part p takes tokens
    // [p kpart, (p + 1) kpart) and writes partial-G buffer p; a reduction sums the parts.
    if (t < a.nG13) {  // G1 = DA^T K and G3 = DC^T K: rows c of m, cols e of d
        const int per13 = a.nG13 / a.ksplit, part = t / per13;
        t %= per13;
        const int k0 = part * a.kpart, kl = min(a.kpart, a.lu - k0);
        const int r0 = (t / ndt) * 128, c0 = (t % ndt) * 128;
        const T* K = a.k + ((int64_t)s * a.N + a.u0 + k0) * a.d;
        // rows r0 .. r0 + 127 lie in one hidden block; k (tokens) runs through its token blocks
        const int64_t hoff = ioff + ((int64_t)(r0 / kHB) * a.ntb + (k0 >> kTBShift)) * kBlk + (int64_t)(r0 % kHB) * kTB;
        const Opnd<T> A[2] = {{a.DA + hoff, kTB, a.m - r0, kl, kTBShift, kBlk},
                              {a.DC + hoff, kTB, a.m - r0, kl, kTBShift, kBlk}};
        const Opnd<T> B[1] = {{K + c0, a.d, a.d - c0, kl}};
        TG13 tl;
        tl.template run<PMG>(A, B, kl, smem);
        // stores go through 32-bit offsets from the tile corner
        float* G1 = a.G + part * a.gpart_stride + s * a.g_stride + (int64_t)r0 * a.d + c0;
        float* G3 = G1 + dm;
        if (r0 + TG13::BM <= a.m && c0 + TG13::BN <= a.d) {
            // full tiles: the K operand's staging permutes the columns, so rows are gathered in LDS
            // and leave as whole 512-byte row segments
            static_assert(TG13::RV_LDS <= LDSB, "row bands fit the tile's LDS");
            tl.rows_via_lds(smem, [&](int, int p, int row, int col, const float4& v) {
                *reinterpret_cast<float4*>((p ? G3 : G1) + (uint32_t)row * (uint32_t)a.d + (uint32_t)col) = v;
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
        return;
    }
    t -= a.nG13;
    if (t < a.nG2) {  // G2 = V^T HkE: rows e of d, cols c of m
        const int per2 = a.nG2 / a.ksplit, part = t / per2;
        t %= per2;
        const int k0 = part * a.kpart, kl = min(a.kpart, a.lu - k0);
        const int r0 = (t / nmt2) * 128, c0 = (t % nmt2) * 256;
        const T* V = a.v + ((int64_t)s * a.N + a.u0 + k0) * a.d;
        const Opnd<T> A[1] = {{V + r0, a.d, a.d - r0, kl}};
        static_assert(TG2::BN == kHB, "a G2 tile covers one hidden block");
        const Opnd<T> B[1] = {{a.HkE + ioff + ((int64_t)(c0 / kHB) * a.ntb + (k0 >> kTBShift)) * kBlk, kTB, a.m - c0, kl,
                               kTBShift, kBlk}};
        TG2 tl;
        tl.template run<PM1>(A, B, kl, smem);
        float* G2 = a.G + part * a.gpart_stride + s * a.g_stride + 2 * dm + (int64_t)r0 * a.m + c0;
        auto epi = [&](auto check) {
            tl.for_each([&](const float (&v)[1], int row, int col) {
                if (!decltype(check)::value || (r0 + row < a.d && c0 + col < a.m))
                    G2[(uint32_t)row * (uint32_t)a.m + (uint32_t)col] = v[0];
            });
        };
        if (r0 + TG2::BM <= a.d && c0 + TG2::BN <= a.m) epi(std::false_type{});
        else epi(std::true_type{});
        return;
    }
    t -= a.nG2;
    {  // O = Hq W2^T: rows t of the apply chunk, cols e of d
        const int r0 = (t / ndt) * kORows, c0 = (t % ndt) * 128;
        const T* W2s = a.sh + s * a.sh_stride + 2 * dm;
        const Opnd<T> A[1] = {{a.Hq + ioff + panel_off(a, r0, 0), kPanel, a.la - r0, a.m, kPanelShift, a.pan}};
        const Opnd<T> B[1] = {{W2s + (int64_t)c0 * a.m, a.m, a.d - c0, a.m}};
        TO tl;
        tl.template run<PM1>(A, B, a.m, smem);
        T* O = a.o + ((int64_t)s * a.N + a.a0 + r0) * a.d + c0;
        auto epi = [&](auto check) {
            tl.for_each([&](const float (&v)[1], int row, int col) {
                if (!decltype(check)::value || (r0 + row < a.la && c0 + col < a.d))
                    O[(uint32_t)row * (uint32_t)a.d + (uint32_t)col] = Elt<T>::st(v[0]);
            });
        };
        if (r0 + TO::BM <= a.la && c0 + TO::BN <= a.d) epi(std::false_type{});
        else epi(std::true_type{});
    }
}

// ---------------------------------------------------------------------------------------------
// update: W <- [L2-Normalize](W - U) for blocks of 16 rows; writes the fp32 master copy (unless dst
// is null: the initial copy of W0 when an update follows, which then reads W0 itself) and (unless
// shadows == 0: the last update, when nothing applies after it) the io-dtype shadows W1, W3, W2 and
// W2^T.  With U == nullptr and norm == 0 it copies (initial W0).
template <typename T> struct UpdArgs {
    const float* src; int64_t src_stride; int src_per_head; int H;
    const float* U; int64_t u_stride;
    float* dst; int64_t dst_stride;
    T* sh; int64_t sh_stride;
    int d, m, norm, last_only, shadows;
    const float* u_scale;                 // per-chunk rates [scan][nchunk]: W - u_scale[s nchunk + jchunk] U,
    int nchunk, jchunk;                   // or null: W - U
    float* nrm; int64_t nrm_stride;       // with norm: each normalized row's |W - U| (rows W1, W3, W2), or null
};

constexpr int kUpdRows = 16;
constexpr int kMaxDim = 2048;

template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
    typedef uint32_t raw __attribute__((ext_vector_type(2)));
    __device__ static void store(uint16_t* p, float4 v) {
        *reinterpret_cast<raw*>(p) = raw{(uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16),
                                         (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16)};
    }
};
template <> struct Vec4<float> {
    __device__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};

// One pass per row: the row of W - U is held in registers (NV float4 per lane, NV = ceil(row / 256)).
// Every load of a row is issued before any is used: a lane past the row's end reads the row's first
// vector and drops the value, so no load waits behind a per-lane branch.  W2's rows are also written
// to LDS so that W2^T can be stored 16 consecutive elements at a time.
template <int NV, typename T>
__device__ __forceinline__ void update_rows(const float* src, const float* U, float us, float* dst, T* shm, T* tileT,
                                            int row0, int L, bool norm, bool to_lds, bool shadows, float* nrm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int L4 = L / 4;
#pragma unroll
    for (int rr = 0; rr < kUpdRows / 4; ++rr) {
        const int row = wave * (kUpdRows / 4) + rr;
        const int64_t ro = (int64_t)(row0 + row) * L;
        const float4* s4 = reinterpret_cast<const float4*>(src + ro);
        float4 x[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] = s4[min(lane + 64 * i, L4 - 1)];
        if (U) {
            const float4* u4 = reinterpret_cast<const float4*>(U + ro);
            float4 uv[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) uv[i] = u4[min(lane + 64 * i, L4 - 1)];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                x[i].x -= us * uv[i].x; x[i].y -= us * uv[i].y; x[i].z -= us * uv[i].z; x[i].w -= us * uv[i].w;
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (lane + 64 * i < L4) ss += x[i].x * x[i].x + x[i].y * x[i].y + x[i].z * x[i].z + x[i].w * x[i].w;
        float sc = 1.0f;
        if (norm) {
            const float n = sqrtf(wave_sum(ss));
            sc = 1.0f / fmaxf(n, 1e-6f);
            if (nrm && lane == 0) nrm[row0 + row] = n;
        }
        float4* d4 = dst ? reinterpret_cast<float4*>(dst + ro) : nullptr;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c4 = lane + 64 * i;
            if (c4 < L4) {
                const float4 w = make_float4(x[i].x * sc, x[i].y * sc, x[i].z * sc, x[i].w * sc);
                if (d4) d4[c4] = w;
                if (shadows) {
                    Vec4<T>::store(shm + ro + 4 * c4, w);
                    if (to_lds) Vec4<T>::store(tileT + row * L + 4 * c4, w);
                }
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_update(UpdArgs<T> a) {
    extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
    T* tileT = reinterpret_cast<T*>(dyn_lds);  // [kUpdRows][m], used by W2 blocks
    const int per = (2 * a.m + a.d) / kUpdRows;
    const int s = blockIdx.x / per, rb = blockIdx.x % per;
    const int64_t dm = (int64_t)a.d * a.m;
    int mat, row0, L;
    if (rb < a.m / kUpdRows) { mat = 0; row0 = rb * kUpdRows; L = a.d; }
    else if (rb < 2 * a.m / kUpdRows) { mat = 1; row0 = rb * kUpdRows - a.m; L = a.d; }
    else { mat = 2; row0 = rb * kUpdRows - 2 * a.m; L = a.m; }
    const bool frozen = a.last_only && mat != 2;
    const int64_t moff = mat * dm;
    const int hs = a.src_per_head ? (s % a.H) : s;
    const float* src = a.src + hs * a.src_stride + moff;
    const float* U = (a.U && !frozen) ? a.U + s * a.u_stride + moff : nullptr;
    const bool norm = a.norm && !frozen;
    float* dst = a.dst ? a.dst + s * a.dst_stride + moff : nullptr;
    T* shm = a.sh + s * a.sh_stride + moff;
    static_assert(kMaxDim <= 8 * 256, "update rows hold at most 8 float4 per lane");
    const float us = a.u_scale ? a.u_scale[(int64_t)s * a.nchunk + a.jchunk] : 1.0f;
    float* nrm = (a.nrm && norm) ? a.nrm + s * a.nrm_stride + (mat == 0 ? 0 : mat == 1 ? a.m : 2 * a.m) : nullptr;
    switch ((L / 4 + 63) / 64) {  // uniform per workgroup
        case 1: update_rows<1>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        case 2: update_rows<2>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        case 3: update_rows<3>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        case 4: update_rows<4>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        case 5: update_rows<5>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        case 6: update_rows<6>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        case 7: update_rows<7>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
        default: update_rows<8>(src, U, us, dst, shm, tileT, row0, L, norm, mat == 2, a.shadows, nrm); break;
    }
    if (mat == 2 && a.shadows) {  // W2^T [m][d]: column c of this 16-row block is 16 consecutive elements
        __syncthreads();
        T* w2t = a.sh + s * a.sh_stride + 3 * dm;
        for (int c = threadIdx.x; c < L; c += kThreads) {
            constexpr int NQ = kUpdRows * (int)sizeof(T) / 16;
            union { T e[kUpdRows]; u32x4_t q[NQ]; } vals;
#pragma unroll
            for (int j = 0; j < kUpdRows; ++j) vals.e[j] = tileT[j * L + c];
            u32x4_t* out = reinterpret_cast<u32x4_t*>(w2t + (int64_t)c * a.d + row0);
#pragma unroll
            for (int q = 0; q < NQ; ++q) out[q] = vals.q[q];
        }
    }
}

template <typename T>
static ttt_status launch_update(const UpdArgs<T>& u, int grid, hipStream_t st) {
    const size_t lds = (size_t)kUpdRows * u.m * sizeof(T);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_update<T>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(TTT_ERR_DEVICE, "k_update LDS attribute: %s", hipGetErrorString(e));
    }
    {
        ProfScope ps(PK_UPDATE, st);
        hipLaunchKernelGGL(k_update<T>, dim3(grid), dim3(kThreads), lds, st, u);
    }
    return check_launch("k_update", st);
}

// ---------------------------------------------------------------------------------------------
// Muon.  prep: U = G, or M <- beta M + G and U = M; per-block partial sums of U^2.  Newton-Schulz
// starts from X_0 = U / (||U||_F + 1e-7) and takes cubic steps X <- 1.5 X - 0.5 (X X^T) X, each as
// a Gram kernel and a step kernel on the side with the smaller Gram matrix.  The first step folds
// the scaling in: with s = 1 / (||U||_F + 1e-7), its Gram kernel writes s^2 U U^T (or s^2 U^T U) and
// its step kernel s (1.5 U - 0.5 Gram U), which is the step from X_0.
// The iterate lives in two planes in bf16 mode: hi = bf16(x) is the contraction operand and
// lo = bf16(x - hi) carries the next 8 bits, so x = hi + lo keeps about 16 bits for 4 bytes per
// element (an fp32 plane beside a bf16 copy would take 6).  prep writes U this way; the last step
// writes x in fp32, which the row update reads.  fp32 mode keeps one fp32 plane, and its first
// step reads U in place.
constexpr int kPrepElems = 4096;
static_assert(kPrepElems % kThreads == 0, "prep blocks take whole rounds of the workgroup");

template <typename T> struct PrepArgs {
    const float* G; int64_t g_stride;
    int parts; int64_t gpart_stride;      // partial-G buffers summed in buffer order (as k_gsum does)
    float* Gsum;                          // the sum written back over G's first buffer, or null
    float* M; int64_t m_stride; float beta;
    float* part; int nblk;
    T* Xhi; T* Xlo; int64_t x_stride;     // bf16 mode, Newton-Schulz: U as hi + lo planes; else null
    int64_t dm; int mat0, nmat;
    int mbase;                            // matrix index of a scan's first stored matrix (offsets are
                                          // (mat - mbase) d m): 0 for [W1 | W3 | W2], 2 for W2 alone
    const float* beta_chunk;              // per-chunk momentum factors [scan][nchunk] (beta_chunk[s nchunk +
    int nchunk, jchunk;                   // jchunk] replaces beta), or null
    float* Urec; int64_t urec_stride;     // U as fp32 (the backward's record), or null
};

__device__ __forceinline__ float block_sum(float x, float* red) {
    x = wave_sum(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = x;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_muon_prep(PrepArgs<T> a) {
    __shared__ float red[4];
    const int per = a.nmat * a.nblk;
    const int s = blockIdx.x / per, t = blockIdx.x % per;
    const int mat = a.mat0 + t / a.nblk, blk = t % a.nblk;
    const int64_t mo = (int64_t)(mat - a.mbase) * a.dm;
    const float* G = a.G + s * a.g_stride + mo;
    float* Gs = a.Gsum ? a.Gsum + s * a.g_stride + mo : nullptr;
    float* M = a.M ? a.M + s * a.m_stride + mo : nullptr;
    T* Xh = a.Xhi ? a.Xhi + s * a.x_stride + mo : nullptr;
    T* Xl = a.Xhi ? a.Xlo + s * a.x_stride + mo : nullptr;
    float* Ur = a.Urec ? a.Urec + s * a.urec_stride + mo : nullptr;
    float ss = 0.f;
    const float beta = a.beta_chunk ? a.beta_chunk[(int64_t)s * a.nchunk + a.jchunk] : a.beta;
    const int64_t e0 = (int64_t)blk * kPrepElems;
    // all loads first (an index past the matrix reads its last element and is not used), then the
    // arithmetic and stores, so the loads are in flight together
    constexpr int NI = kPrepElems / kThreads;
    float g[NI], mv[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) g[j] = G[min(e0 + threadIdx.x + j * kThreads, a.dm - 1)];
    for (int p = 1; p < a.parts; ++p) {
        float gp[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) gp[j] = G[p * a.gpart_stride + min(e0 + threadIdx.x + j * kThreads, a.dm - 1)];
#pragma unroll
        for (int j = 0; j < NI; ++j) g[j] += gp[j];
    }
    if (M) {
#pragma unroll
        for (int j = 0; j < NI; ++j) mv[j] = M[min(e0 + threadIdx.x + j * kThreads, a.dm - 1)];
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int64_t e = e0 + threadIdx.x + j * kThreads;
        if (e < a.dm) {
            float u = g[j];
            if (Gs) Gs[e] = u;
            if (M) {
                u = beta * mv[j] + u;
                M[e] = u;
            }
            if (Ur) Ur[e] = u;
            if constexpr (sizeof(T) == 2) {
                if (Xh) {
                    const uint16_t h = f2bf(u);
                    Xh[e] = h;
                    Xl[e] = f2bf(u - bf2f(h));
                }
            }
            ss += u * u;
        }
    }
    const float tot = block_sum(ss, red);
    if (threadIdx.x == 0) a.part[((int64_t)s * 3 + mat) * a.nblk + blk] = tot;
}

template <typename T> struct NSArgs {
    const float* U; int64_t u_stride;     // k_ns_init only: U
    const float* part; int nblk;          // partial sums of U^2 on the first step (and k_ns_init), else null
    const T* Xin; T* Xout;                // hi planes (ping-pong), stride x_stride
    T* Xlo;                               // bf16 mode: lo plane, updated in place; fp32 mode: null
    float* Xf;                            // fp32 result (last step in bf16 mode, k_ns_init), else null
    int64_t x_stride;
    T* Gram; int64_t gram_stride;         // 3 x p*p
    int d, m, mat0, nmat, tiles;          // tiles per matrix
    int mbase;                            // as in PrepArgs: offsets are (mat - mbase) d m, (mat - mbase) p^2
};

// s = 1 / (||U||_F + 1e-7) from nblk partial sums; every lane of every wave gets the same value
__device__ __forceinline__ float ns_scale(const float* part, int nblk) {
    float t = 0.f;
    for (int i = threadIdx.x & 63; i < nblk; i += 64) t += part[i];
    return 1.0f / (sqrtf(wave_sum(t)) + 1e-7f);
}

// Zero Newton-Schulz steps: X = U / (||U||_F + 1e-7) in fp32.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_ns_init(NSArgs<T> a) {
    const int64_t dm = (int64_t)a.d * a.m;
    const int per = a.nmat * a.nblk;
    const int s = blockIdx.x / per, t = blockIdx.x % per;
    const int mat = a.mat0 + t / a.nblk, blk = t % a.nblk;
    const float inv = ns_scale(a.part + ((int64_t)s * 3 + mat) * a.nblk, a.nblk);
    const float* U = a.U + s * a.u_stride + (mat - a.mbase) * dm;
    float* Xf = a.Xf + s * a.x_stride + (mat - a.mbase) * dm;
    const int64_t e0 = (int64_t)blk * kPrepElems;
    constexpr int NI = kPrepElems / kThreads;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int64_t e = e0 + threadIdx.x + j * kThreads;
        if (e < dm) Xf[e] = U[e] * inv;
    }
}

// Gram tiles of TS x TS: one 64-wide LDS stage (18 KB at TS = 64)
template <typename T, bool KS, int TS> using NSTile = Tile<T, TS, TS, 2, 2, 1, 1, 1, KS, KS, false, 4, 1>;
// step tiles: two LDS stages, or (FULL: every tile in range) one stage at four workgroups per CU
template <typename T, bool FULL> using NSStepTall = Tile<T, 128, 64, 2, 2, 1, 1, 1, false, false, false, 4, FULL ? 1 : 2>;
template <typename T, bool FULL> using NSStepWide = Tile<T, 128, 64, 2, 2, 1, 1, 1, false, true, false, 4, FULL ? 1 : 2>;
constexpr int kNSStepRows = 128, kNSStepCols = 64;

// The Gram matrix is symmetric: only its tiles on or above the diagonal are computed (tile t of
// np (np + 1) / 2, row-major over the upper triangle), and an off-diagonal tile also writes its
// mirror block, transposed through LDS so that those stores are whole rows as well.  The launch
// takes TS = 64 (launch_ns_gram).
template <typename T, int TS>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 3 : 2) void k_ns_gram(NSArgs<T> a) {
    constexpr int kTP = TS + 16 / (int)sizeof(T);  // transposed-tile pitch (elements)
    constexpr int LDSB = std::max(NSTile<T, false, TS>::LDS, TS * kTP * (int)sizeof(T));
    __shared__ __attribute__((aligned(16))) char smem[LDSB];
    const int64_t dm = (int64_t)a.d * a.m;
    const int per = a.nmat * a.tiles;
    const int lb = xcd_block(gridDim.x);
    const int s = lb / per;
    int t = lb % per;
    const int mat = a.mat0 + t / a.tiles;
    t %= a.tiles;
    const int r = mat < 2 ? a.m : a.d, c = mat < 2 ? a.d : a.m;
    const int p = r < c ? r : c;
    const int np = (p + TS - 1) / TS;
    int ti = 0;
    while (t >= np - ti) t -= np - ti++;  // uniform: row ti of the upper triangle, column ti + t
    const int i0 = ti * TS, j0 = (ti + t) * TS;
    const T* X = a.Xin + s * a.x_stride + (mat - a.mbase) * dm;
    T* Gm = a.Gram + s * a.gram_stride + (int64_t)(mat - a.mbase) * p * p;
    T* tT = reinterpret_cast<T*>(smem);
    auto epi = [&](auto& tl) {
        float sc2 = 1.0f;
        if (a.part) {
            const float sc = ns_scale(a.part + ((int64_t)s * 3 + mat) * a.nblk, a.nblk);
            sc2 = sc * sc;
        }
        tl.for_each([&](const float (&v)[1], int row, int col) {
            if (i0 + row < p && j0 + col < p) Gm[(uint32_t)(i0 + row) * (uint32_t)p + (uint32_t)(j0 + col)] = Elt<T>::st(v[0] * sc2);
        });
        if (i0 == j0) return;
        lds_barrier();  // every wave is done with the LDS stage
        tl.for_each([&](const float (&v)[1], int row, int col) { tT[col * kTP + row] = Elt<T>::st(v[0] * sc2); });
        __syncthreads();
        // mirror block: Gram row j0 + cc, columns i0 .. i0 + TS - 1, from LDS row cc
        constexpr int VEC = 16 / (int)sizeof(T), VPR = TS / VEC;
        for (int u = threadIdx.x; u < TS * VPR; u += kThreads) {
            const int cc = u / VPR, x = (u % VPR) * VEC;
            if (j0 + cc < p && i0 + x < p)
                *reinterpret_cast<u32x4_t*>(Gm + (uint32_t)(j0 + cc) * (uint32_t)p + (uint32_t)(i0 + x)) =
                    *reinterpret_cast<const u32x4_t*>(tT + cc * kTP + x);
        }
    };
    // a diagonal tile's two operands are the same rows of X, staged once
    if (r > c) {  // Gram = X^T X (c x c), contracted over the r rows
        NSTile<T, true, TS> tl;
        const Opnd<T> A[1] = {{X + i0, c, c - i0, r}};
        const Opnd<T> B[1] = {{X + j0, c, c - j0, r}};
        if (i0 == j0) tl.template run_sym<PM1>(A, r, smem);
        else tl.template run<PM1>(A, B, r, smem);
        epi(tl);
    } else {      // Gram = X X^T (r x r), contracted over the c columns
        NSTile<T, false, TS> tl;
        const Opnd<T> A[1] = {{X + (int64_t)i0 * c, c, r - i0, c}};
        const Opnd<T> B[1] = {{X + (int64_t)j0 * c, c, r - j0, c}};
        if (i0 == j0) tl.template run_sym<PM1>(A, c, smem);
        else tl.template run<PM1>(A, B, c, smem);
        epi(tl);
    }
}

// Four consecutive iterate values at one position: hi and lo planes (bf16) or the fp32 plane.
template <typename T> struct NSQuad;
template <> struct NSQuad<uint16_t> {
    typedef uint32_t raw __attribute__((ext_vector_type(2)));
    raw h, l;
    __device__ void load(const uint16_t* hi, const uint16_t* lo, uint32_t e) {
        h = *reinterpret_cast<const raw*>(hi + e);
        l = *reinterpret_cast<const raw*>(lo + e);
    }
    __device__ static float lo16(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static float hi16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    __device__ float4 value() const {
        return make_float4(lo16(h.x) + lo16(l.x), hi16(h.x) + hi16(l.x), lo16(h.y) + lo16(l.y), hi16(h.y) + hi16(l.y));
    }
    __device__ static void store(uint16_t* hi, uint16_t* lo, uint32_t e, float4 x) {
        const uint16_t h0 = f2bf(x.x), h1 = f2bf(x.y), h2 = f2bf(x.z), h3 = f2bf(x.w);
        *reinterpret_cast<raw*>(hi + e) = raw{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
        Pack4<uint16_t>::store(lo + e, x.x - bf2f(h0), x.y - bf2f(h1), x.z - bf2f(h2), x.w - bf2f(h3));
    }
};
template <> struct NSQuad<float> {
    float4 h;
    __device__ void load(const float* hi, const float*, uint32_t e) { h = *reinterpret_cast<const float4*>(hi + e); }
    __device__ float4 value() const { return h; }
    __device__ static void store(float* hi, float*, uint32_t e, float4 x) { *reinterpret_cast<float4*>(hi + e) = x; }
};

// X <- s (1.5 X - 0.5 P) with P = X Gram (tall) or Gram X (wide), s = 1 except on the first step.
// The iterate values this thread updates are loaded before the contraction, so their latency hides
// behind it.  Each position belongs to one tile, so the lo plane is read and rewritten in place;
// the hi plane is read by every tile's contraction and is written to the other buffer.
// FULL: every tile of the launch lies inside its matrix (d and m multiples of 128); the tiles then
// take one LDS stage, read the iterate in the epilogue, and four workgroups share a CU, so that one
// workgroup's pipeline fill and epilogue overlap the others' contractions.
template <typename T, bool FULL>
__global__ __launch_bounds__(kThreads, FULL ? 4 : 2) void k_ns_step(NSArgs<T> a) {
    constexpr bool kLo = sizeof(T) == 2;
    __shared__ __attribute__((aligned(16))) char smem[NSStepTall<T, FULL>::LDS];
    const int64_t dm = (int64_t)a.d * a.m;
    const int per = a.nmat * a.tiles;
    const int lb = xcd_block(gridDim.x);
    const int s = lb / per;
    int t = lb % per;
    const int mat = a.mat0 + t / a.tiles;
    t %= a.tiles;
    const int r = mat < 2 ? a.m : a.d, c = mat < 2 ? a.d : a.m;
    const int p = r < c ? r : c;
    const int nct = (c + kNSStepCols - 1) / kNSStepCols;
    const int r0 = (t / nct) * kNSStepRows, c0 = (t % nct) * kNSStepCols;
    if (r0 >= r) return;  // a.tiles covers the larger of the tall and wide tilings
    const int64_t base = (int64_t)s * a.x_stride + (int64_t)(mat - a.mbase) * dm;
    const T* X = a.Xin + base;
    const T* Gm = a.Gram + s * a.gram_stride + (int64_t)(mat - a.mbase) * p * p;
    // this tile's own positions, as 32-bit offsets from its corner
    const int64_t corner = base + (int64_t)r0 * c + c0;
    const T* Xh = a.Xin + corner;
    T* Xl = kLo ? a.Xlo + corner : nullptr;
    T* Xo = a.Xout + corner;
    float* Xf = a.Xf ? a.Xf + corner : nullptr;
    auto scale = [&]() {
        return a.part ? ns_scale(a.part + ((int64_t)s * 3 + mat) * a.nblk, a.nblk) : 1.0f;
    };
    auto body = [&](auto& tl, const auto& A, const auto& B, int K) {
        using TT = typename std::remove_reference<decltype(tl)>::type;
        if (FULL || (r0 + TT::BM <= r && c0 + TT::BN <= c)) {
            // full tiles: rows gathered in LDS, the iterate read and written four elements at a time
            // (FULL: the iterate is read in the epilogue, which the other workgroups on the CU hide;
            // else it is loaded before the contraction)
            static_assert(TT::RV_LDS <= (int)sizeof(smem), "row bands fit the tile's LDS");
            NSQuad<T> xv[FULL ? 1 : TT::RV_N];
            if constexpr (!FULL)
                TT::rows_via_lds_pos([&](int idx, int, int row, int col) {
                    xv[idx].load(Xh, Xl, (uint32_t)row * (uint32_t)c + (uint32_t)col);
                });
            tl.template run<PM1>(A, B, K, smem);
            const float sc = scale();
            tl.rows_via_lds(smem, [&](int idx, int, int row, int col, const float4& v) {
                NSQuad<T> xq;
                if constexpr (FULL) xq.load(Xh, Xl, (uint32_t)row * (uint32_t)c + (uint32_t)col);
                else xq = xv[idx];
                const float4 x = xq.value();
                const float4 xn = make_float4(sc * (1.5f * x.x - 0.5f * v.x), sc * (1.5f * x.y - 0.5f * v.y),
                                              sc * (1.5f * x.z - 0.5f * v.z), sc * (1.5f * x.w - 0.5f * v.w));
                const uint32_t e = (uint32_t)row * (uint32_t)c + (uint32_t)col;
                if (Xf) *reinterpret_cast<float4*>(Xf + e) = xn;
                else NSQuad<T>::store(Xo, Xl, e, xn);
            });
        } else if constexpr (!FULL) {
            // partial tiles, element by element; a position outside the matrix reads the corner and
            // is not stored
            float xv[TT::ELEMS];
            TT::for_each_pos([&](int idx, int row, int col) {
                const bool in = r0 + row < r && c0 + col < c;
                const uint32_t e = in ? (uint32_t)row * (uint32_t)c + (uint32_t)col : 0u;
                if constexpr (kLo) xv[idx] = bf2f(Xh[e]) + bf2f(Xl[e]);
                else xv[idx] = Xh[e];
            });
            tl.template run<PM1>(A, B, K, smem);
            const float sc = scale();
            int idx = 0;
            tl.for_each([&](const float (&v)[1], int row, int col) {
                const float xn = sc * (1.5f * xv[idx++] - 0.5f * v[0]);
                if (r0 + row < r && c0 + col < c) {
                    const uint32_t e = (uint32_t)row * (uint32_t)c + (uint32_t)col;
                    if (Xf) {
                        Xf[e] = xn;
                    } else {
                        const T h = Elt<T>::st(xn);
                        Xo[e] = h;
                        if constexpr (kLo) Xl[e] = f2bf(xn - bf2f(h));
                    }
                }
            });
        }
    };
    if (r > c) {  // P = X Gram; Gram is symmetric, so its rows serve as the B operand
        NSStepTall<T, FULL> tl;
        const Opnd<T> A[1] = {{X + (int64_t)r0 * c, c, r - r0, c}};
        const Opnd<T> B[1] = {{Gm + (int64_t)c0 * p, p, c - c0, p}};
        body(tl, A, B, c);
    } else {      // P = Gram X; B[j][i] = X[i][j] is read k-strided
        NSStepWide<T, FULL> tl;
        const Opnd<T> A[1] = {{Gm + (int64_t)r0 * p, p, r - r0, p}};
        const Opnd<T> B[1] = {{X + c0, c, c - c0, r}};
        body(tl, A, B, r);
    }
}

// The Gram matrices of nmats matrices (sets na.tiles).  64 x 64 tiles: 64 VGPRs and 18 KB of LDS, so
// up to eight workgroups share a CU and hide each other's pipeline fill and epilogue; 128 x 128 tiles
// carry twice the MFMA work per operand byte but fit only three per CU, and were slower even at the
// LaCT LM shape (2.92 against 2.73 ms per call).
template <typename T>
static void launch_ns_gram(NSArgs<T> na, int64_t nmats, hipStream_t st) {
    constexpr int TS = 64;
    const int np = (int)cdiv(std::min(na.d, na.m), TS);
    na.tiles = np * (np + 1) / 2;
    hipLaunchKernelGGL((k_ns_gram<T, TS>), dim3((unsigned)(nmats * na.tiles)), dim3(kThreads), 0, st, na);
}

// The step over grid tiles, with the full-tile workgroups when every tile lies inside its matrix
template <typename T>
static void launch_ns_step(const NSArgs<T>& na, unsigned grid, hipStream_t st) {
    if (na.d % 128 == 0 && na.m % 128 == 0)
        hipLaunchKernelGGL((k_ns_step<T, true>), dim3(grid), dim3(kThreads), 0, st, na);
    else
        hipLaunchKernelGGL((k_ns_step<T, false>), dim3(grid), dim3(kThreads), 0, st, na);
}

// ---------------------------------------------------------------------------------------------
// Parallel static-kernel form (last layer only, plain GD).  With W1 and W3 frozen, the features
// phi(x) = SiLU(W1 x) * (W3 x) stay fixed along the sequence, a chunk's W2 gradient is
// -sum_i eta_i v_i phi(k_i)^T, and W2 follows chunked linear attention with queries phi(q), keys
// phi(k), values v and state W2 ("TTT with KV Binding Is Secretly Linear Attention", Thm. 5.2 and
// 5.3, Sec. 6.1, Table 2 Variant 2).  One launch computes the features of every token; the
// chunk-parallel linear-attention kernels do the rest, with the recurrence's momentum, inner steps
// and ascent folded into their state scan.

// ---------------------------------------------------------------------------------------------
// host driver

// Zeroes n4 float4 (a kernel rather than hipMemsetAsync, so that a caller may capture the call
// into a HIP graph)
__global__ __launch_bounds__(kThreads) void k_zero(float4* p, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Sum of the partial-G buffers into the first: n float4 per buffer, parts buffers gstride apart,
// added in buffer order (deterministic).
__global__ __launch_bounds__(kThreads) void k_gsum(float* G, int64_t n4, int parts, int64_t gstride) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    float4* g = reinterpret_cast<float4*>(G) + i;
    float4 acc = *g;
    for (int p = 1; p < parts; ++p) {
        const float4 x = *reinterpret_cast<const float4*>(G + p * gstride + 4 * i);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    *g = acc;
}

// Token parts for the gradient tiles of a step over lu tokens: the largest power of two up to 8
// that keeps the launch at most 512 gradient workgroups (two per CU on 256 CUs) and every part at
// least 512 tokens, which also keeps every part non-empty.  Depends on the descriptor only.
// gradient tiles per scan and step: G1/G3 (unless only W2 learns) and G2
static int grad_tiles(const ttt_desc& D) {
    const int64_t d = D.d_h, m = D.m_h;
    return (int)((D.last_layer_only ? 0 : cdiv(m, 128) * cdiv(d, 128)) + cdiv(d, 128) * cdiv(m, 256));
}

static int grad_split(int64_t S, int gtiles, int64_t lu) {
    int p = 1;
    while (p < 8 && S * gtiles * (2 * p) <= 512 && lu >= 512 * (2 * p)) p *= 2;
    return p;
}

struct Layout {
    size_t wf[2], sh[2], hq, hke, da, dc, g, xf, xb[2], xlo, gram, part, mom, total;
    int64_t wf_stride, sh_stride, inter_stride, g_stride, x_stride, gram_stride;
    int nblk, gparts;
};

static Layout make_layout(const ttt_desc& D, bool muon, bool own_m) {
    Layout L{};
    const int64_t S = (int64_t)D.B * D.H, d = D.d_h, m = D.m_h, dm = d * m;
    const int64_t bmax = D.N < D.chunk ? D.N : D.chunk;
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const int64_t p = d < m ? d : m;
    L.wf_stride = 3 * dm;
    L.sh_stride = 4 * dm;
    L.inter_stride = std::max<int64_t>(bmax * cdiv(m, kPanel) * kPanel, cdiv(m, kHB) * kBlk * cdiv(bmax, kTB));  // see StepArgs
    L.g_stride = 3 * dm;
    L.x_stride = 3 * dm;
    L.gram_stride = 3 * p * p;
    L.nblk = (int)cdiv(dm, kPrepElems);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    L.wf[0] = take(S * L.wf_stride * 4);
    L.wf[1] = take(S * L.wf_stride * 4);
    L.sh[0] = take(S * L.sh_stride * es);
    L.sh[1] = take(S * L.sh_stride * es);
    L.hq = take(S * L.inter_stride * es);
    L.hke = take(S * L.inter_stride * es);
    L.da = take(S * L.inter_stride * es);
    L.dc = take(S * L.inter_stride * es);
    L.gparts = grad_split(S, grad_tiles(D), bmax);  // partial-G buffers for the longest chunk
    L.g = take(S * L.g_stride * 4 * L.gparts);
    L.part = take(S * 3 * (size_t)L.nblk * 4);
    if (muon) {
        L.xf = take(S * L.x_stride * 4);
        L.xb[0] = take(S * L.x_stride * es);
        L.xb[1] = take(S * L.x_stride * es);
        if (es == 2) L.xlo = take(S * L.x_stride * es);
        L.gram = take(S * L.gram_stride * es);
    }
    if (own_m) L.mom = take(S * 3 * dm * 4);
    L.total = off;
    return L;
}

// Workspace of the parallel form: W1 | W3 in bf16 (bf16 io only), phi(q), phi(k), and the
// linear-attention chunk states; with Muon also the Newton-Schulz buffers of every (scan, chunk)
// matrix (Frobenius partial sums, iterate planes, fp32 result, Gram matrices).
struct PLayout {
    size_t w13, phq, phk, lin, part, xb[2], xlo, xf, gram, total;
    int64_t nc;
    int nblk;
};

static PLayout make_playout(const ttt_desc& D) {
    PLayout L{};
    const int64_t S = (int64_t)D.B * D.H, dm = (int64_t)D.d_h * D.m_h;
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    L.nc = D.N > 0 ? cdiv(D.N, D.chunk) : 0;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    if (es == 2) L.w13 = take((size_t)(D.w0_per_batch ? S : D.H) * 2 * dm * es);
    L.phq = take((size_t)S * D.N * D.m_h * es);
    L.phk = take((size_t)S * D.N * D.m_h * es);
    L.lin = take(lin_chunked_ws_bytes(S, L.nc, D.m_h, D.d_h, es));
    L.nblk = (int)cdiv(dm, kPrepElems);
    if (D.rule == TTT_UPD_MUON) {
        const int64_t nmx = S * L.nc, p = std::min(D.d_h, D.m_h);
        L.part = take((size_t)nmx * 3 * L.nblk * 4);
        L.xb[0] = take((size_t)nmx * dm * es);
        L.xb[1] = take((size_t)nmx * dm * es);
        if (es == 2) L.xlo = take((size_t)nmx * dm * es);
        L.xf = take((size_t)nmx * dm * 4);
        L.gram = take((size_t)nmx * p * p * es);
    }
    L.total = off;
    return L;
}

// Momentum over the chunks of the parallel form with Muon (last layer only: a chunk's W2 gradient
// g_c = -sum eta v phi(k)^T depends on the frozen phi and on v alone, never on W2, so every chunk's
// g_c is known up front).  One thread owns 4 consecutive elements of one scan's W2 and walks the
// chunks in order: for an updating chunk m <- beta m + g_c, and m replaces dS_c (dS_c = -g_c for
// descent, +g_c for ascent); a chunk that does not update leaves m as it is and its slot is zeroed.
// m starts from M0 (the W2 block of the caller's momentum) or zero, and leaves in Mout.
struct ParMomArgs {
    float* dS; const float* M0; float* Mout; int64_t m_stride;
    int64_t dm; int nc, nscan, mode; float beta, gsign;  // g_c = gsign * dS_c
    uint32_t flags[32];
};

__global__ __launch_bounds__(kThreads) void k_par_momentum(ParMomArgs a) {
    const int64_t per = a.dm / 4;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g >= per * a.nscan) return;
    const int64_t scan = g / per, e = (g % per) * 4;
    f32x4_t m = {0.f, 0.f, 0.f, 0.f};
    if (a.M0)
#pragma unroll
        for (int u = 0; u < 4; ++u) m[u] = a.M0[scan * a.m_stride + e + u];
    for (int c = 0; c < a.nc; ++c) {
        f32x4_t* p = reinterpret_cast<f32x4_t*>(a.dS + (scan * a.nc + c) * a.dm + e);
        if (a.mode != TTT_MASK_STRIDED || ((a.flags[c >> 5] >> (c & 31)) & 1u)) {
            m = a.beta * m + a.gsign * *p;
            *p = m;
        } else {
            *p = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (a.Mout)
#pragma unroll
        for (int u = 0; u < 4; ++u) a.Mout[scan * a.m_stride + e + u] = m[u];
}

// The parallel form's step between the chunk updates and the state scan, with Muon: the momentum
// over chunks (k_par_momentum), then Newton-Schulz on every (scan, chunk) momentum matrix at once
// with the recurrence's kernels (each such matrix is a d x m W2 block).  The scan then subtracts
// U_c = Muon(M_c) from W2 chunk by chunk.
template <typename T> struct ParMuon {
    const ttt_desc* D;
    const PLayout* L;
    char* ws;
    float* M_inout;
    uint32_t flags[32];
};

template <typename T>
static ttt_status par_muon_between(void* ctx, float* dS, const float** src, hipStream_t st) {
    const ParMuon<T>& c = *static_cast<const ParMuon<T>*>(ctx);
    const ttt_desc& D = *c.D;
    const PLayout& L = *c.L;
    const int64_t S = (int64_t)D.B * D.H, nmx = S * L.nc, d = D.d_h, m = D.m_h, dm = d * m;
    ttt_status rc;
    {  // 1. momentum over chunks, in place
        ParMomArgs ma{};
        ma.dS = dS;
        if (D.momentum != 0.0f && c.M_inout) {
            ma.M0 = c.M_inout + 2 * dm;
            ma.Mout = c.M_inout + 2 * dm;
            ma.m_stride = 3 * dm;
        }
        ma.dm = dm;
        ma.nc = (int)L.nc;
        ma.nscan = (int)S;
        ma.mode = D.mask;
        ma.beta = D.momentum;
        ma.gsign = D.ascent ? 1.0f : -1.0f;
        for (int w = 0; w < 32; ++w) ma.flags[w] = c.flags[w];
        {
            ProfScope ps(PK_PAR_MOM, st);
            hipLaunchKernelGGL(k_par_momentum, dim3((unsigned)cdiv(S * dm / 4, kThreads)), dim3(kThreads), 0, st, ma);
        }
        if ((rc = check_launch("k_par_momentum", st)) != TTT_OK) return rc;
    }
    float* part = (float*)(c.ws + L.part);
    T* Xb[2] = {(T*)(c.ws + L.xb[0]), (T*)(c.ws + L.xb[1])};
    T* Xlo = sizeof(T) == 2 ? (T*)(c.ws + L.xlo) : nullptr;
    float* Xf = (float*)(c.ws + L.xf);
    const bool split = sizeof(T) == 2 && D.ns_iters > 0;
    {  // 2. Frobenius partial sums of each matrix (and, in bf16 mode, its hi + lo planes)
        PrepArgs<T> pa{dS, dm, 1, 0, nullptr, nullptr, 0, 0.0f, part, L.nblk, split ? Xb[1] : nullptr,
                       split ? Xlo : nullptr, dm, dm, 2, 1, 2};
        {
            ProfScope ps(PK_MUON_PREP, st);
            hipLaunchKernelGGL(k_muon_prep<T>, dim3((unsigned)(nmx * L.nblk)), dim3(kThreads), 0, st, pa);
        }
        if ((rc = check_launch("k_muon_prep", st)) != TTT_OK) return rc;
    }
    if (D.ns_iters == 0) {  // 3. U_c = M_c / (||M_c||_F + 1e-7)
        NSArgs<T> na{dS, dm, part, L.nblk, nullptr, nullptr, nullptr, Xf, dm, nullptr, 0, (int)d, (int)m, 2, 1, 0, 2};
        {
            ProfScope ps(PK_NS_INIT, st);
            hipLaunchKernelGGL(k_ns_init<T>, dim3((unsigned)(nmx * L.nblk)), dim3(kThreads), 0, st, na);
        }
        if ((rc = check_launch("k_ns_init", st)) != TTT_OK) return rc;
        *src = Xf;
        return TTT_OK;
    }
    // 3. ns_iters Newton-Schulz steps on every matrix (as in the recurrence: the first step folds
    // the Frobenius scaling in; bf16 mode ends in fp32 in Xf, fp32 mode reads M_c in place first)
    const T* first = sizeof(T) == 2 ? Xb[1] : reinterpret_cast<const T*>(dS);
    const int64_t p = std::min(d, m);
    NSArgs<T> na{nullptr, 0, nullptr, L.nblk, first, Xb[0], Xlo, nullptr, dm, (T*)(c.ws + L.gram), p * p, (int)d,
                 (int)m, 2, 1, 0, 2};
    const int stt = (int)std::max(cdiv(m, kNSStepRows) * cdiv(d, kNSStepCols), cdiv(d, kNSStepRows) * cdiv(m, kNSStepCols));
    for (int it = 0; it < D.ns_iters; ++it) {
        na.Xin = it == 0 ? first : Xb[(it - 1) & 1];
        na.Xout = Xb[it & 1];
        na.part = it == 0 ? part : nullptr;
        na.Xf = (sizeof(T) == 2 && it == D.ns_iters - 1) ? Xf : nullptr;
        {
            ProfScope ps(PK_NS_GRAM, st);
            launch_ns_gram<T>(na, nmx, st);
        }
        if ((rc = check_launch("k_ns_gram", st)) != TTT_OK) return rc;
        na.tiles = stt;
        {
            ProfScope ps(PK_NS_STEP, st);
            launch_ns_step<T>(na, (unsigned)(nmx * stt), st);
        }
        if ((rc = check_launch("k_ns_step", st)) != TTT_OK) return rc;
    }
    *src = sizeof(T) == 2 ? Xf : reinterpret_cast<const float*>(Xb[(D.ns_iters - 1) & 1]);
    return TTT_OK;
}

template <typename T>
static ttt_status run_parallel_form(const ttt_desc& D, const PLayout& L, const T* q, const T* k, const T* v,
                                    const float* eta, const float* W0, T* o, float* W_out, float* M_inout, char* ws,
                                    hipStream_t st) {
    const int64_t S = (int64_t)D.B * D.H, dm = (int64_t)D.d_h * D.m_h;
    const int64_t Hw = D.w0_per_batch ? S : D.H;  // fast-weight blocks in W0
    ttt_status rc;
    // W_out's frozen W1 | W3 come from W0 (all of W when there are no tokens)
    auto copy_w0 = [&](int64_t floats) -> ttt_status {
        if (!W_out) return TTT_OK;
        for (int64_t b = 0; b < (D.w0_per_batch ? 1 : D.B); ++b) {
            hipError_t e = hipMemcpy2DAsync(W_out + b * Hw * 3 * dm, 3 * dm * 4, W0, 3 * dm * 4, floats * 4, Hw,
                                            hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return fail(TTT_ERR_DEVICE, "copying W0 into W_out: %s", hipGetErrorString(e));
        }
        return TTT_OK;
    };
    if (D.N == 0) return copy_w0(3 * dm);  // M_inout is left as it is
    // 1. W1 | W3 as contraction operands
    const T* W13;
    int64_t w13_stride;
    if constexpr (sizeof(T) == 2) {
        T* w = (T*)(ws + L.w13);
        const int64_t per4 = 2 * dm / 4, n4 = Hw * per4;
        {
            ProfScope ps(PK_W13, st);
            hipLaunchKernelGGL(k_w13_cvt<T>, dim3((unsigned)cdiv(n4, kThreads)), dim3(kThreads), 0, st, W0, 3 * dm, w,
                               n4, per4);
        }
        if ((rc = check_launch("k_w13_cvt", st)) != TTT_OK) return rc;
        W13 = w;
        w13_stride = 2 * dm;
    } else {
        W13 = reinterpret_cast<const T*>(W0);
        w13_stride = 3 * dm;
    }
    // 2. the features of every query and key
    T* phq = (T*)(ws + L.phq);
    T* phk = (T*)(ws + L.phk);
    PhiArgs<T> pa{{q, k}, {phq, phk}, {nullptr, nullptr}, W13, w13_stride, D.w0_per_batch ? 0 : D.H, D.N, D.d_h,
                  D.m_h, (int)S, (int)cdiv(D.N, kPhiRows), (int)cdiv(D.m_h, kPhiCols)};
    {
        ProfScope ps(PK_PHI, st);
        hipLaunchKernelGGL((k_phi<T, false>), dim3((unsigned)(2 * S * pa.ntt * pa.nct)), dim3(64 * kPhiWaves), 0, st, pa);
    }
    if ((rc = check_launch("k_phi", st)) != TTT_OK) return rc;
    // 3. chunked linear attention over the features, with W2 [d][m] as the state S [d_v][d_k]
    linattn_desc LD{D.B, D.H, D.N, D.m_h, D.d_h, D.chunk, D.io_dtype, D.mask, D.update_chunks};
    uint32_t flags[32] = {};
    if (D.mask == TTT_MASK_STRIDED)
        for (int64_t j = 0; j < L.nc; ++j)
            if (D.update_chunks[j]) flags[j >> 5] |= 1u << (j & 31);
    LinStateIO io;
    io.S0 = W0 + 2 * dm;
    io.s0_stride = 3 * dm;
    io.s0_heads = D.w0_per_batch ? 0 : D.H;
    io.Sout = W_out ? W_out + 2 * dm : nullptr;
    io.sout_stride = 3 * dm;
    ParMuon<T> pm{&D, &L, ws, M_inout, {}};
    if (D.rule == TTT_UPD_MUON) {  // W2 <- W2 - Muon(M_c): the scan subtracts what the hook leaves
        for (int w = 0; w < 32; ++w) pm.flags[w] = flags[w];
        io.between = &par_muon_between<T>;
        io.between_ctx = &pm;
        io.dsign = -1.0f;
        if ((rc = lin_chunked_run<T>(LD, flags, phq, phk, v, eta, o, io, ws + L.lin, st)) != TTT_OK) return rc;
        return copy_w0(2 * dm);
    }
    if (D.momentum != 0.0f) {  // M <- beta M + g, W <- W - M: the running term is m = -M
        io.mom = 1;
        io.beta = D.momentum;
        io.msign = -1.0f;
        if (M_inout) {
            io.M0 = M_inout + 2 * dm;
            io.Mout = M_inout + 2 * dm;
            io.m_stride = 3 * dm;
        }
    }
    io.dsign = D.ascent ? -1.0f : 1.0f;
    io.reps = D.inner_steps > 1 ? D.inner_steps : 1;
    if ((rc = lin_chunked_run<T>(LD, flags, phq, phk, v, eta, o, io, ws + L.lin, st)) != TTT_OK) return rc;
    return copy_w0(2 * dm);
}

ttt_status validate_ttt_desc(const ttt_desc* D) {
    if (!D) return fail(TTT_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (D->B < 0 || D->H < 0 || D->N < 0) return fail(TTT_ERR_INVALID_ARGUMENT, "B, H, N must be >= 0");
    if (D->d_h < 32 || D->d_h > kMaxDim || D->d_h % 32)
        return fail(TTT_ERR_INVALID_ARGUMENT, "d_h=%d must be a multiple of 32 in [32, %d]", D->d_h, kMaxDim);
    if (D->m_h < 32 || D->m_h > kMaxDim || D->m_h % 32)
        return fail(TTT_ERR_INVALID_ARGUMENT, "m_h=%d must be a multiple of 32 in [32, %d]", D->m_h, kMaxDim);
    if (D->chunk < 1) return fail(TTT_ERR_INVALID_ARGUMENT, "chunk must be >= 1");
    if (D->io_dtype != TTT_F32 && D->io_dtype != TTT_BF16) return fail(TTT_ERR_INVALID_ARGUMENT, "bad io_dtype");
    if (D->mask < TTT_MASK_FULL || D->mask > TTT_MASK_TOKEN_CAUSAL) return fail(TTT_ERR_INVALID_ARGUMENT, "bad mask");
    if (D->mask == TTT_MASK_TOKEN_CAUSAL)
        return fail(TTT_ERR_UNSUPPORTED, "TOKEN_CAUSAL is defined for the linear model (linattn_forward) only");
    if (D->mask == TTT_MASK_FULL && D->chunk < D->N)
        return fail(TTT_ERR_INVALID_ARGUMENT, "MASK_FULL needs chunk >= N (one chunk)");
    if (D->mask == TTT_MASK_STRIDED && !D->update_chunks && D->N > 0)
        return fail(TTT_ERR_INVALID_ARGUMENT, "MASK_STRIDED needs update_chunks");
    if (D->rule < TTT_UPD_GD || D->rule > TTT_UPD_MUON) return fail(TTT_ERR_INVALID_ARGUMENT, "bad update rule");
    if (D->ns_iters < 0 || D->ns_iters > 32) return fail(TTT_ERR_INVALID_ARGUMENT, "ns_iters must be in [0, 32]");
    if (!(D->momentum == D->momentum) || D->momentum > 1e30f || D->momentum < -1e30f)
        return fail(TTT_ERR_INVALID_ARGUMENT, "momentum must be finite");
    if (D->last_layer_only != 0 && D->last_layer_only != 1) return fail(TTT_ERR_INVALID_ARGUMENT, "last_layer_only must be 0/1");
    if (D->w0_per_batch != 0 && D->w0_per_batch != 1) return fail(TTT_ERR_INVALID_ARGUMENT, "w0_per_batch must be 0/1");
    if (D->inner_steps < 0 || D->inner_steps > 64) return fail(TTT_ERR_INVALID_ARGUMENT, "inner_steps must be in [0, 64]");
    if (D->ascent != 0 && D->ascent != 1) return fail(TTT_ERR_INVALID_ARGUMENT, "ascent must be 0/1");
    if (D->parallel_form != 0 && D->parallel_form != 1)
        return fail(TTT_ERR_INVALID_ARGUMENT, "parallel_form must be 0/1");
    if (D->chunk_rates != 0 && D->chunk_rates != 1) return fail(TTT_ERR_INVALID_ARGUMENT, "chunk_rates must be 0/1");
    if (D->chunk_rates && D->momentum != 0.0f)
        return fail(TTT_ERR_INVALID_ARGUMENT, "with chunk_rates the momentum comes from chunk_momentum; momentum must be 0");
    if (!D->chunk_rates && D->chunk_momentum)
        return fail(TTT_ERR_INVALID_ARGUMENT, "chunk_momentum is read only with chunk_rates = 1");
    if (D->chunk_rates && D->parallel_form)
        return fail(TTT_ERR_UNSUPPORTED, "parallel_form takes per-token rates only");
    if (D->parallel_form) {
        if (!D->last_layer_only || (D->rule != TTT_UPD_GD && D->rule != TTT_UPD_MUON))
            return fail(TTT_ERR_INVALID_ARGUMENT,
                        "parallel_form needs last_layer_only = 1 and rule TTT_UPD_GD or TTT_UPD_MUON (frozen W1, W3; "
                        "no weight norm)");
        if (D->rule == TTT_UPD_MUON && D->inner_steps > 1)
            return fail(TTT_ERR_UNSUPPORTED, "parallel_form with TTT_UPD_MUON takes one gradient step per chunk");
        const int64_t S = (int64_t)D->B * D->H, nc = D->N > 0 ? cdiv(D->N, D->chunk) : 0;
        if (D->mask == TTT_MASK_STRIDED && nc > 32 * 32)
            return fail(TTT_ERR_UNSUPPORTED, "parallel_form with MASK_STRIDED supports at most 1024 chunks");
        // launch sizes: the feature tiles, and the linear-attention tiles over chunks and state
        const int64_t nd = cdiv(D->d_h, 128), nm = cdiv(D->m_h, 128);
        const int64_t lim = 1LL << 31;
        if (2 * S * cdiv(D->N, kPhiRows) * cdiv(D->m_h, kPhiCols) >= lim || S * nc * nd * nm >= lim ||
            S * nc * cdiv(std::min<int64_t>(D->chunk, D->N), 128) * nd >= lim)
            return fail(TTT_ERR_UNSUPPORTED, "parallel_form: B*H, N, d_h, m_h too large for one launch");
    }
    const int64_t S = (int64_t)D->B * D->H;
    if (S > (1 << 20) || (int64_t)D->N > (1LL << 31) / 2) return fail(TTT_ERR_INVALID_ARGUMENT, "B*H or N too large");
    const int64_t bmax = D->N < D->chunk ? D->N : D->chunk;
    if (cdiv(D->m_h, kHB) * kBlk * cdiv(bmax, kTB) >= (1LL << 31))
        return fail(TTT_ERR_UNSUPPORTED, "m_h x chunk must stay below 2^31 elements");
    return TTT_OK;
}

static bool is_muon(const ttt_desc& D) { return D.rule == TTT_UPD_MUON_L2 || D.rule == TTT_UPD_MUON; }
// whether the update keeps a momentum: the chunk momentum beta, or per-chunk factors alpha_j
static bool has_mom(const ttt_desc& D) { return D.chunk_rates ? D.chunk_momentum != nullptr : D.momentum != 0.0f; }

template <typename T>
static ttt_status run_ttt(const ttt_desc& D, const Layout& L, const T* q, const T* k, const T* v,
                          const float* eta, const float* W0, T* o, float* W_out, float* M_inout,
                          char* ws, hipStream_t st, float* hist = nullptr, float* nrm = nullptr,
                          float* urec = nullptr) {
    const int S = D.B * D.H, d = D.d_h, m = D.m_h;
    const int64_t dm = (int64_t)d * m;
    const bool muon = is_muon(D);
    const bool mom = has_mom(D);
    const int nchunks = (int)cdiv(D.N, D.chunk);
    float* Wf[2] = {(float*)(ws + L.wf[0]), (float*)(ws + L.wf[1])};
    T* sh[2] = {(T*)(ws + L.sh[0]), (T*)(ws + L.sh[1])};
    float* G = (float*)(ws + L.g);
    float* part = (float*)(ws + L.part);
    float* M = mom ? (M_inout ? M_inout : (float*)(ws + L.mom)) : nullptr;
    ttt_status rc;

    if (mom && !M_inout) {
        const int64_t n4 = (int64_t)S * 3 * dm / 4;
        {
            ProfScope ps(PK_ZERO, st);
            hipLaunchKernelGGL(k_zero, dim3((unsigned)cdiv(n4, kThreads)), dim3(kThreads), 0, st, (float4*)M, n4);
        }
        if ((rc = check_launch("k_zero", st)) != TTT_OK) return rc;
    }
    const int upd_blocks = (2 * m + d) / kUpdRows;
    int cur = 0;
    const int nc = (int)cdiv(D.N, D.chunk);
    const bool uta = D.mask == TTT_MASK_FULL || D.mask == TTT_MASK_UPDATE_THEN_APPLY;
    const int nsteps = D.N == 0 ? 0 : (uta ? nc + 1 : nc);
    const int ntm = (int)cdiv(m, 128), ntd = (int)cdiv(d, 128);
    const int64_t bmax = D.N < D.chunk ? D.N : D.chunk;
    // the last step whose chunk updates: its last update writes W_out directly (no copy at the
    // end), and skips the shadows when no apply follows it
    int last_upd = -1;
    for (int step = 0; step < nsteps && step < nc; ++step)
        if (D.mask != TTT_MASK_STRIDED || D.update_chunks[step]) last_upd = step;
    // hist (the backward's record): the weights before update i go to hist + i S 3 d m, the last
    // update's result after them, with the norm each update's row norms to nrm + i S (2m + d), and
    // with Muon each update's U (fp32) to urec + i S 3 d m; W_out is then a copy of the last entry.
    // With o null nothing is applied.
    const int64_t hstride = (int64_t)S * 3 * dm;
    int ui = 0;  // updates so far
    {  // W0 -> shadows, and the master copy only if no update follows (the first update reads W0)
        UpdArgs<T> u{W0, 3 * dm, D.w0_per_batch ? 0 : 1, D.H, nullptr, 0, hist ? hist : last_upd < 0 ? Wf[0] : nullptr,
                     L.wf_stride, sh[0], L.sh_stride, d, m, 0, 0, 1};
        if ((rc = launch_update<T>(u, S * upd_blocks, st)) != TTT_OK) return rc;
    }
    bool w_in_master = hist || last_upd < 0;  // whether the current W is in Wf[cur], or still only in W0
    for (int step = 0; step < nsteps; ++step) {
        int ja = o ? (uta ? step - 1 : step) : -1;
        int ju = step < nc ? step : -1;
        if (D.mask == TTT_MASK_STRIDED && ju >= 0 && !D.update_chunks[ju]) ju = -1;
        // an updating chunk takes inner_steps gradient steps, each from the gradient at the current
        // W; the chunk's apply (queries and outputs) runs once, with the first of them
        const int nin = ju >= 0 ? std::max(1, D.inner_steps) : 1;
        for (int it = 0; it < nin; ++it) {
            if (it > 0) ja = -1;
            StepArgs<T> a{};
            a.q = q; a.k = k; a.v = v; a.eta = D.chunk_rates ? nullptr : eta; a.o = o;
            a.N = D.N; a.d = d; a.m = m;
            a.Hq = (T*)(ws + L.hq); a.HkE = (T*)(ws + L.hke); a.DA = (T*)(ws + L.da); a.DC = (T*)(ws + L.dc);
            a.inter_stride = L.inter_stride;
            a.pan = bmax * kPanel;
            a.ntb = (int)cdiv(bmax, kTB);
            a.sh = sh[cur]; a.sh_stride = L.sh_stride;
            a.G = G; a.g_stride = L.g_stride;
            a.eta_sign = D.ascent ? -1.0f : 1.0f;
            a.a0 = ja >= 0 ? (int64_t)ja * D.chunk : 0;
            a.la = ja >= 0 ? (int)(std::min<int64_t>((int64_t)(ja + 1) * D.chunk, D.N) - a.a0) : 0;
            a.u0 = ju >= 0 ? (int64_t)ju * D.chunk : 0;
            a.lu = ju >= 0 ? (int)(std::min<int64_t>((int64_t)(ju + 1) * D.chunk, D.N) - a.u0) : 0;
            a.nQ = a.la ? (int)(cdiv(a.la, kUpQRows) * cdiv(m, kUpCols)) : 0;
            a.nK = a.lu ? (int)(cdiv(a.lu, kUpKRows) * cdiv(m, kUpCols)) : 0;
            a.ksplit = a.lu ? grad_split(S, grad_tiles(D), a.lu) : 1;  // <= L.gparts: lu <= bmax
            a.kpart = (int)(cdiv(cdiv(a.lu, a.ksplit), kTB) * kTB);
            a.gpart_stride = (int64_t)S * L.g_stride;
            a.nG13 = (a.lu && !D.last_layer_only) ? ntm * ntd * a.ksplit : 0;
            a.nG2 = a.lu ? ntd * (int)cdiv(m, 256) * a.ksplit : 0;
            a.nO = a.la ? (int)cdiv(a.la, kORows) * ntd : 0;
            if (a.nQ + a.nK) {
                {
                    ProfScope ps(PK_UP, st);
                    hipLaunchKernelGGL(k_up<T>, dim3(S * (a.nQ + a.nK)), dim3(64 * kUpWaves), 0, st, a);
                }
                if ((rc = check_launch("k_up", st)) != TTT_OK) return rc;
            }
            if (a.nG13 + a.nG2 + a.nO) {
                {
                    ProfScope ps(PK_DOWN, st);
                    hipLaunchKernelGGL(k_down<T>, dim3(S * (a.nG13 + a.nG2 + a.nO)), dim3(kThreads), 0, st, a);
                }
                if ((rc = check_launch("k_down", st)) != TTT_OK) return rc;
            }
            // with momentum or Muon the prep kernel adds the partial-G buffers itself
            if (a.lu && a.ksplit > 1 && !(muon || mom)) {
                const int64_t n4 = (int64_t)S * L.g_stride / 4;
                {
                    ProfScope ps(PK_DOWN, st);
                    hipLaunchKernelGGL(k_gsum, dim3((unsigned)cdiv(n4, kThreads)), dim3(kThreads), 0, st, G, n4,
                                       a.ksplit, a.gpart_stride);
                }
                if ((rc = check_launch("k_gsum", st)) != TTT_OK) return rc;
            }
            if (a.lu == 0) continue;
            const int mat0 = D.last_layer_only ? 2 : 0, nmat = D.last_layer_only ? 1 : 3;
            const float* U = G;
            T* Xb[2] = {(T*)(ws + L.xb[0]), (T*)(ws + L.xb[1])};
            T* Xlo = sizeof(T) == 2 ? (T*)(ws + L.xlo) : nullptr;
            float* Xf = (float*)(ws + L.xf);
            // bf16 Newton-Schulz starts from U's hi + lo planes, which prep writes (hi into Xb[1])
            const bool split = muon && sizeof(T) == 2 && D.ns_iters > 0;
            if (muon || mom) {
                // the summed G is needed again only where U = G is read in fp32 (no momentum: fp32
                // Newton-Schulz, or zero steps)
                const bool keep_g = a.ksplit > 1 && !mom && (sizeof(T) == 4 || D.ns_iters == 0);
                PrepArgs<T> pa{G, L.g_stride, a.ksplit, a.gpart_stride, keep_g ? G : nullptr, M, 3 * dm, D.momentum, part,
                               L.nblk, split ? Xb[1] : nullptr, split ? Xlo : nullptr, L.x_stride, dm, mat0, nmat, 0,
                               D.chunk_rates ? D.chunk_momentum : nullptr, nchunks, ju};
                if (urec) {
                    pa.Urec = urec + ui * hstride;
                    pa.urec_stride = 3 * dm;
                }
                {
                    ProfScope ps(PK_MUON_PREP, st);
                    hipLaunchKernelGGL(k_muon_prep<T>, dim3(S * nmat * L.nblk), dim3(kThreads), 0, st, pa);
                }
                if ((rc = check_launch("k_muon_prep", st)) != TTT_OK) return rc;
                if (mom) U = M;
            }
            if (muon && D.ns_iters == 0) {
                NSArgs<T> na{U, 3 * dm, part, L.nblk, nullptr, nullptr, nullptr, Xf, L.x_stride, nullptr, 0,
                             d, m, mat0, nmat, 0};
                {
                    ProfScope ps(PK_NS_INIT, st);
                    hipLaunchKernelGGL(k_ns_init<T>, dim3(S * nmat * L.nblk), dim3(kThreads), 0, st, na);
                }
                if ((rc = check_launch("k_ns_init", st)) != TTT_OK) return rc;
                U = Xf;
            } else if (muon) {
                // step it reads hi plane Xin and writes Xout = Xb[it & 1]; the first step reads U's planes
                // (fp32 mode: U itself, whose stride 3 d m is the iterate's) and scales by 1 / ||U||_F;
                // in bf16 mode the last step writes fp32 into Xf
                const T* first = sizeof(T) == 2 ? Xb[1] : reinterpret_cast<const T*>(U);
                NSArgs<T> na{nullptr, 0, nullptr, L.nblk, first, Xb[0], Xlo, nullptr, L.x_stride, (T*)(ws + L.gram),
                             L.gram_stride, d, m, mat0, nmat, 0};
                const int p = d < m ? d : m;
                // step tiles: the larger of the tall (m x d) and wide (d x m) tilings
                const int stt = (int)std::max(cdiv(m, kNSStepRows) * cdiv(d, kNSStepCols),
                                              cdiv(d, kNSStepRows) * cdiv(m, kNSStepCols));
                for (int it = 0; it < D.ns_iters; ++it) {
                    na.Xin = it == 0 ? first : Xb[(it - 1) & 1];
                    na.Xout = Xb[it & 1];
                    na.part = it == 0 ? part : nullptr;
                    na.Xf = (sizeof(T) == 2 && it == D.ns_iters - 1) ? Xf : nullptr;
                    {
                        ProfScope ps(PK_NS_GRAM, st);
                        launch_ns_gram<T>(na, (int64_t)S * nmat, st);
                    }
                    if ((rc = check_launch("k_ns_gram", st)) != TTT_OK) return rc;
                    na.tiles = stt;
                    {
                        ProfScope ps(PK_NS_STEP, st);
                        launch_ns_step<T>(na, (unsigned)(S * nmat * stt), st);
                    }
                    if ((rc = check_launch("k_ns_step", st)) != TTT_OK) return rc;
                }
                U = sizeof(T) == 2 ? Xf : reinterpret_cast<const float*>(Xb[(D.ns_iters - 1) & 1]);
            }
            const int norm = (D.rule == TTT_UPD_GD_L2 || D.rule == TTT_UPD_MUON_L2) ? 1 : 0;
            const bool final_upd = step == last_upd && it == nin - 1;
            UpdArgs<T> u{Wf[cur], L.wf_stride, 0, D.H, U, 3 * dm, Wf[cur ^ 1], L.wf_stride, sh[cur ^ 1], L.sh_stride,
                         d, m, norm, D.last_layer_only, 1, D.chunk_rates ? eta : nullptr, nchunks, ju};
            if (hist) {
                u.src = hist + ui * hstride;
                u.dst = hist + (ui + 1) * hstride;
                u.nrm = nrm ? nrm + ui * (int64_t)S * (2 * m + d) : nullptr;
                u.nrm_stride = 2 * m + d;
            }
            ++ui;
            if (!w_in_master) {  // the first update reads W0 (per head or per scan)
                u.src = W0;
                u.src_stride = 3 * dm;
                u.src_per_head = D.w0_per_batch ? 0 : 1;
                w_in_master = true;
            }
            if (final_upd && W_out && !hist) {
                u.dst = W_out;  // [B][H][3 d m], the same stride as the master copy
                u.shadows = step < nsteps - 1;
            }
            if ((rc = launch_update<T>(u, S * upd_blocks, st)) != TTT_OK) return rc;
            cur ^= 1;
        }
    }
    if (W_out && (hist || last_upd < 0)) {  // no update wrote W_out: the record's last entry, or the master copy
        hipError_t e = hipMemcpyAsync(W_out, hist ? hist + ui * hstride : Wf[cur], (size_t)S * 3 * dm * 4,
                                      hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return fail(TTT_ERR_DEVICE, "copying W_out: %s", hipGetErrorString(e));
    }
    return TTT_OK;
}

// The forward recurrence run for its record alone (no output): every update's input weights and,
// with the norm, its row norms, as described at run_ttt.
size_t ttt_history_ws_bytes(const ttt_desc& D) { return make_layout(D, is_muon(D), has_mom(D)).total; }

template <typename T>
ttt_status ttt_run_history(const ttt_desc& D, const T* q, const T* k, const T* v, const float* eta, const float* W0,
                           T* o, float* W_out, float* hist, float* nrm, float* urec, char* ws, hipStream_t st) {
    const Layout L = make_layout(D, is_muon(D), has_mom(D));
    return run_ttt<T>(D, L, q, k, v, eta, W0, o, W_out, nullptr, ws, st, hist, nrm, urec);
}
template ttt_status ttt_run_history<uint16_t>(const ttt_desc&, const uint16_t*, const uint16_t*, const uint16_t*,
                                              const float*, const float*, uint16_t*, float*, float*, float*, float*,
                                              char*, hipStream_t);
template ttt_status ttt_run_history<float>(const ttt_desc&, const float*, const float*, const float*, const float*,
                                           const float*, float*, float*, float*, float*, float*, char*, hipStream_t);

// Newton-Schulz steps from X_0 (for the backward): for k < ns_iters the Gram matrix of X_k goes to
// P + k S 3 p^2 and, but for the last, X_{k+1} to X + (k + 1) S 3 d m (bf16: hi planes, with the lo
// plane Xlo carried in place as the forward's steps do).  X, Xlo: [S][3dm]; P: [S][3 p^2].
template <typename T>
ttt_status ns_steps(const ttt_desc& D, T* X, T* Xlo, T* P, hipStream_t st) {
    const int S = D.B * D.H, d = D.d_h, m = D.m_h;
    const int64_t dm = (int64_t)d * m, p = std::min(d, m);
    const int mat0 = D.last_layer_only ? 2 : 0, nmat = D.last_layer_only ? 1 : 3;
    const int nblk = (int)cdiv(dm, kPrepElems);
    ttt_status rc;
    const int stt = (int)std::max(cdiv(m, kNSStepRows) * cdiv(d, kNSStepCols), cdiv(d, kNSStepRows) * cdiv(m, kNSStepCols));
    const int64_t xs = (int64_t)S * 3 * dm, ps_ = (int64_t)S * 3 * p * p;
    for (int k = 0; k < D.ns_iters; ++k) {
        NSArgs<T> na{nullptr, 0, nullptr, nblk, X + k * xs, k + 1 < D.ns_iters ? X + (k + 1) * xs : nullptr,
                     sizeof(T) == 2 ? Xlo : nullptr, nullptr, 3 * dm, P + k * ps_, 3 * p * p, d, m, mat0, nmat, 0, 0};
        {
            ProfScope ps(PK_NS_GRAM, st);
            launch_ns_gram<T>(na, (int64_t)S * nmat, st);
        }
        if ((rc = check_launch("k_ns_gram", st)) != TTT_OK) return rc;
        if (k + 1 == D.ns_iters) break;  // the last iterate is not needed
        na.tiles = stt;
        {
            ProfScope ps(PK_NS_STEP, st);
            launch_ns_step<T>(na, (unsigned)(S * nmat * stt), st);
        }
        if ((rc = check_launch("k_ns_step", st)) != TTT_OK) return rc;
    }
    return TTT_OK;
}
template ttt_status ns_steps<uint16_t>(const ttt_desc&, uint16_t*, uint16_t*, uint16_t*, hipStream_t);
template ttt_status ns_steps<float>(const ttt_desc&, float*, float*, float*, hipStream_t);

}  // namespace ttt

using namespace ttt;

extern "C" ttt_status ttt_workspace_bytes(const ttt_desc* desc, size_t* bytes) {
    clear_error();
    ttt_status rc = validate_ttt_desc(desc);
    if (rc != TTT_OK) return rc;
    if (!bytes) return fail(TTT_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = desc->parallel_form ? make_playout(*desc).total
                                 : make_layout(*desc, is_muon(*desc), has_mom(*desc)).total;
    return TTT_OK;
}

namespace ttt {
// ttt_forward with the workspace either the caller's (scratch == false: checked against its HIP
// allocation like every other buffer) or the library's static scratch array (scratch == true:
// workspace_bytes is the array's size, and calls needing more are refused).
static ttt_status forward_impl(const ttt_desc* desc, const void* q, const void* k, const void* v, const float* eta,
                               const float* W0, void* o, float* W_out, float* M_inout, void* workspace,
                               size_t workspace_bytes, void* stream, bool scratch) {
    ttt_status rc = validate_ttt_desc(desc);
    if (rc != TTT_OK) return rc;
    const ttt_desc& D = *desc;
    const int64_t S = (int64_t)D.B * D.H;
    if (S == 0) return TTT_OK;
    const size_t es = D.io_dtype == TTT_BF16 ? 2 : 4;
    const size_t io_bytes = (size_t)S * D.N * D.d_h * es;
    const size_t w_bytes = (size_t)S * 3 * D.d_h * D.m_h * 4;
    const size_t w0_bytes = (size_t)(D.w0_per_batch ? S : D.H) * 3 * D.d_h * D.m_h * 4;
    if (!W0) return fail(TTT_ERR_INVALID_ARGUMENT, "W0 is NULL");
    if (D.N > 0 && (!q || !k || !v || !eta || !o)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, eta and o are required");
    const void* p16[] = {q, k, v, o, W0, W_out, M_inout};
    for (const void* p : p16)
        if (p && !aligned(p, 16)) return fail(TTT_ERR_INVALID_ARGUMENT, "q, k, v, o, W0, W_out, M must be 16-byte aligned");
    if (eta && !aligned(eta, 4)) return fail(TTT_ERR_INVALID_ARGUMENT, "eta must be 4-byte aligned");
    const size_t eta_bytes = (size_t)S * (D.chunk_rates ? cdiv(D.N, D.chunk) : D.N) * 4;
    if (overlaps(o, io_bytes, q, io_bytes) || overlaps(o, io_bytes, k, io_bytes) || overlaps(o, io_bytes, v, io_bytes) ||
        overlaps(o, io_bytes, eta, eta_bytes))
        return fail(TTT_ERR_INVALID_ARGUMENT, "o overlaps an input");
    if (overlaps(W_out, w_bytes, W0, w0_bytes)) return fail(TTT_ERR_INVALID_ARGUMENT, "W_out overlaps W0");
    hipStream_t st = (hipStream_t)stream;
    // every buffer the call touches lies in a device allocation that holds all of it
    auto buffers = [&](size_t ws_need) -> ttt_status {
        const size_t eb = D.N > 0 ? io_bytes : 0;
        const struct { const void* p; size_t n; const char* name; } bufs[] = {
            {q, eb, "q"}, {k, eb, "k"}, {v, eb, "v"}, {o, eb, "o"}, {eta, D.N > 0 ? eta_bytes : 0, "eta"},
            {D.chunk_rates ? D.chunk_momentum : nullptr, D.N > 0 ? (size_t)S * cdiv(D.N, D.chunk) * 4 : 0, "chunk_momentum"},
            {W0, w0_bytes, "W0"}, {W_out, w_bytes, "W_out"}, {M_inout, has_mom(D) ? w_bytes : 0, "M_inout"},
            {scratch ? nullptr : workspace, ws_need, "workspace"}};
        for (const auto& b : bufs) {
            const ttt_status r = check_buffer(b.p, b.n, b.name);
            if (r != TTT_OK) return r;
        }
        return TTT_OK;
    };
    if (D.parallel_form) {
        const PLayout PL = make_playout(D);
        if (PL.total > 0 && (!workspace || workspace_bytes < PL.total))
            return fail(TTT_ERR_WORKSPACE, scratch ? "the call needs %zu bytes of scratch, the library's array holds %zu"
                                                   : "workspace needs %zu bytes, got %zu", PL.total, workspace_bytes);
        if (workspace && !aligned(workspace, 256)) return fail(TTT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if ((rc = buffers(PL.total)) != TTT_OK) return rc;
        if (D.io_dtype == TTT_BF16)
            return run_parallel_form<uint16_t>(D, PL, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta,
                                               W0, (uint16_t*)o, W_out, M_inout, (char*)workspace, st);
        return run_parallel_form<float>(D, PL, (const float*)q, (const float*)k, (const float*)v, eta, W0, (float*)o,
                                        W_out, M_inout, (char*)workspace, st);
    }
    const Layout L = make_layout(D, is_muon(D), has_mom(D) && !M_inout);
    if (L.total > 0 && (!workspace || workspace_bytes < L.total))
        return fail(TTT_ERR_WORKSPACE, scratch ? "the call needs %zu bytes of scratch, the library's array holds %zu"
                                               : "workspace needs %zu bytes, got %zu", L.total, workspace_bytes);
    if (workspace && !aligned(workspace, 256)) return fail(TTT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if ((rc = buffers(L.total)) != TTT_OK) return rc;
    if (D.io_dtype == TTT_BF16)
        return run_ttt<uint16_t>(D, L, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, eta, W0,
                                 (uint16_t*)o, W_out, M_inout, (char*)workspace, st);
    return run_ttt<float>(D, L, (const float*)q, (const float*)k, (const float*)v, eta, W0, (float*)o, W_out,
                          M_inout, (char*)workspace, st);
}

// Scratch of the entry point that allocates nothing: one array per device, holding the workspace of
// one call, kept until the process ends.  Host code never uses the array's name as an address (on
// the host it stands for a host-side shadow); it uses the device address hipGetSymbolAddress gives
// for the current device, looked up once per device.
constexpr size_t kScratchBytes = TTT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static ttt_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(TTT_ERR_DEVICE, "no usable HIP device (%s)", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(TTT_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(TTT_ERR_DEVICE, "scratch array address on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TTT_OK;
}
}  // namespace ttt

extern "C" ttt_status ttt_forward(const ttt_desc* desc, const void* q, const void* k, const void* v,
                                  const float* eta, const float* W0, void* o, float* W_out, float* M_inout,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    clear_error();
    return forward_impl(desc, q, k, v, eta, W0, o, W_out, M_inout, workspace, workspace_bytes, stream, false);
}

extern "C" ttt_status ttt_forward_noalloc(const ttt_desc* desc, const void* q, const void* k, const void* v,
                                          const float* eta, const float* W0, void* o, float* W_out, float* M_inout,
                                          void* stream) {
    clear_error();
    ttt_status rc = validate_ttt_desc(desc);
    if (rc != TTT_OK) return rc;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != TTT_OK) return rc;
    ProfSuppress quiet;  // the profiler creates events per launch; this call creates nothing
    return forward_impl(desc, q, k, v, eta, W0, o, W_out, M_inout, ws, kScratchBytes, stream, true);
}
