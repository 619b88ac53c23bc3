// The SwiGLU features phi(x) = SiLU(W1 x) o (W3 x) of the TTT layer's fast weight with W1 and W3
// frozen (PaperTrace "5.2.1 LaCT and TTT-E2E", Eq. (3); "TTT with KV Binding Is Secretly Linear
// Attention", Thm. 5.2-5.3 and Sec. 6.1: the layer is then linear attention over phi(q), phi(k)),
// and their backward (the same paper, Sec. 6.2: training through the parallel form).  Shared by the
// parallel form and its backward.
#pragma once
#include <type_traits>

#include "tile.hpp"

namespace ttt {

constexpr int kPhiWaves = 8;   // 8 waves, one workgroup per CU
constexpr int kPhiRows = 256;  // token rows per tile
constexpr int kPhiCols = 128;  // hidden units per tile

// W1 | W3 (the first 2 d m floats of each fast-weight block) in bf16, as contraction operands
template <typename T>
__global__ __launch_bounds__(kThreads) void k_w13_cvt(const float* W0, int64_t w_stride, T* out, int64_t n4,
                                                      int64_t per4) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    const int64_t h = i / per4, j = i % per4;
    const float4 w = *reinterpret_cast<const float4*>(W0 + h * w_stride + 4 * j);
    Pack4<T>::store(out + 4 * i, w.x, w.y, w.z, w.w);
}

template <typename T> struct PhiArgs {
    const T* x[2]; T* out[2];        // q and k [S][N][d]; phi [S][N][m], or dA | dC [S][N][2m]
    const T* dphi[2];                // backward: the gradients of phi(q), phi(k) [S][N][m]
    const T* W; int64_t w_stride;    // W1 of weight block hw at W + hw * w_stride, W3 d m after it
    int w_heads;                     // hw = s % w_heads, or s when 0 (one block per scan)
    int64_t N; int d, m, nscan, ntt, nct;  // token and hidden tiles per scan
};

// Tiles of 256 tokens x 128 hidden units on 8 waves: a = x W1^T and c = x W3^T on MFMA.  Forward:
// the epilogue writes phi = SiLU(a) c row-major (hidden units contiguous).  BWD: it reads dphi at
// the same positions and writes dA = dphi c SiLU'(a) and dC = dphi SiLU(a) side by side in rows of
// 2m (dA in columns 0 .. m-1, dC in m .. 2m-1), with SiLU'(a) = s (1 + a (1 - s)), s = sigmoid(a).
template <typename T, bool BWD>
__global__ __launch_bounds__(64 * kPhiWaves, 1) void k_phi(PhiArgs<T> a) {
    using TQ = Tile<T, kPhiRows, kPhiCols, 2, 4, 1, 2, 2, false, false, false, kPhiWaves>;
    __shared__ __attribute__((aligned(16))) char smem[TQ::LDS];
    const int per = a.ntt * a.nct;
    const int lb = xcd_block(gridDim.x);
    const int u = lb / per, t = lb % per;
    const int which = u / a.nscan, s = u % a.nscan;
    const int hw = a.w_heads ? s % a.w_heads : s;
    const int r0 = (t / a.nct) * kPhiRows, c0 = (t % a.nct) * kPhiCols;
    const int64_t dm = (int64_t)a.d * a.m;
    const T* W1 = a.W + (int64_t)hw * a.w_stride;
    const T* W3 = W1 + dm;
    const int rows = (int)(a.N - r0);
    const Opnd<T> A[1] = {{a.x[which] + ((int64_t)s * a.N + r0) * a.d, a.d, rows, a.d}};
    const Opnd<T> B[2] = {{W1 + (int64_t)c0 * a.d, a.d, a.m - c0, a.d}, {W3 + (int64_t)c0 * a.d, a.d, a.m - c0, a.d}};
    TQ tl;
    tl.template run<PMQ>(A, B, a.d, smem);
    if constexpr (!BWD) {
        T* P = a.out[which] + ((int64_t)s * a.N + r0) * a.m + c0;
        auto epi = [&](auto check) {
            tl.for_each([&](const float (&v)[2], int row, int col) {
                if (!decltype(check)::value || (row < rows && c0 + col < a.m))
                    P[(int64_t)row * a.m + col] = Elt<T>::st(v[0] * sigmoidf_(v[0]) * v[1]);
            });
        };
        if (kPhiRows <= rows && c0 + kPhiCols <= a.m) epi(std::false_type{});
        else epi(std::true_type{});
    } else {
        const T* G = a.dphi[which] + ((int64_t)s * a.N + r0) * a.m + c0;
        T* P = a.out[which] + ((int64_t)s * a.N + r0) * 2 * a.m + c0;
        // the tile's dphi, every load issued before the first use (positions out of range read 0)
        float g[TQ::ELEMS];
        TQ::for_each_pos([&](int idx, int row, int col) {
            const bool in = row < rows && c0 + col < a.m;
            g[idx] = in ? Elt<T>::ld(G[(uint32_t)row * (uint32_t)a.m + (uint32_t)col]) : 0.f;
        });
        int idx = 0;
        tl.for_each([&](const float (&v)[2], int row, int col) {
            const float sg = sigmoidf_(v[0]), gi = g[idx++];
            if (row < rows && c0 + col < a.m) {
                const uint32_t off = (uint32_t)row * (uint32_t)(2 * a.m) + (uint32_t)col;
                P[off] = Elt<T>::st(gi * v[1] * sg * (1.f + v[0] * (1.f - sg)));
                P[off + a.m] = Elt<T>::st(gi * v[0] * sg);
            }
        });
    }
}

}  // namespace ttt
