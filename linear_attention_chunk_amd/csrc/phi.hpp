// The SwiGLU features phi(x) = SiLU(W1 x) o (W3 x) of the TTT layer's fast weight with W1 and W3
// frozen (PaperTrace "5.2.1 LaCT and TTT-E2E", Eq. (3); "TTT with KV Binding Is Secretly Linear
// Attention", Thm. 5.2-5.3 and Sec. 6.1: the layer is then linear attention over phi(q), phi(k)),
// and the factors their backward needs (the same paper, Sec. 6.2: training through the parallel
// form).  Shared by the parallel form and its backward.
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
    const T* x[2]; T* out[2];        // q and k [S][N][d]; phi(q), phi(k) [S][N][m]
    T* gate[2];                      // GATE: the factors of phi's backward [S][N][2m] (see k_phi)
    const T* W; int64_t w_stride;    // W1 of weight block hw at W + hw * w_stride, W3 d m after it
    int w_heads;                     // hw = s % w_heads, or s when 0 (one block per scan)
    int64_t N; int d, m, nscan, ntt, nct;  // token and hidden tiles per scan
};

// Tiles of 256 tokens x 128 hidden units on 8 waves: a = x W1^T and c = x W3^T on MFMA; the
// epilogue writes phi = SiLU(a) c row-major (hidden units contiguous).  GATE also writes the two
// factors that carry a gradient g of phi back to a and c, side by side in rows of 2m:
// u = c SiLU'(a) in columns 0 .. m-1 and w = SiLU(a) in m .. 2m-1 (dA = g u, dC = g w), with
// SiLU(a) = a s, SiLU'(a) = s (1 + a (1 - s)), s = sigmoid(a).
template <typename T, bool GATE>
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
    T* P = a.out[which] + ((int64_t)s * a.N + r0) * a.m + c0;
    T* U = GATE ? a.gate[which] + ((int64_t)s * a.N + r0) * 2 * a.m + c0 : nullptr;
    auto epi = [&](auto check) {
        tl.for_each([&](const float (&v)[2], int row, int col) {
            if (!decltype(check)::value || (row < rows && c0 + col < a.m)) {
                const float sg = sigmoidf_(v[0]), w = v[0] * sg;
                P[(int64_t)row * a.m + col] = Elt<T>::st(w * v[1]);
                if constexpr (GATE) {
                    const uint32_t off = (uint32_t)row * (uint32_t)(2 * a.m) + (uint32_t)col;
                    U[off] = Elt<T>::st(v[1] * sg * (1.f + v[0] * (1.f - sg)));
                    U[off + a.m] = Elt<T>::st(w);
                }
            }
        });
    };
    if (kPhiRows <= rows && c0 + kPhiCols <= a.m) epi(std::false_type{});
    else epi(std::true_type{});
}

}  // namespace ttt
