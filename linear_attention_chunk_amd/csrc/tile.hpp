// Device building blocks for gfx950 (CDNA4): element traits, LDS staging of operand tiles and a
// 256-thread (4-wave) MFMA tile engine computing C[i][j] = sum_k A[i][k] * B[j][k].
//
// LDS holds every operand tile k-contiguous: row r of a tile occupies SEG 64-byte k-segments
// followed by 16 bytes of padding, so the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks.  An operand whose source is k-contiguous in memory is copied 16 bytes at a time;
// one whose source is k-strided (token-major data contracted over tokens) is transposed in
// registers, one VEC x VEC block per thread, on its way into LDS.
//
// MFMA fragments: for v_mfma_f32_16x16x32_bf16 lane l supplies row (l % 16) and the 8 k-values of
// group (l / 16); for fp32 four v_mfma_f32_16x16x4_f32 consume the 4 k-values of a lane's 16-byte
// read one at a time.  A and B use the same lane-to-k assignment, so the contraction is complete
// whatever order the hardware walks k in.  Result element r of lane l is C[4*(l/16) + r][l % 16].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <typename T> struct Elt;

template <> struct Elt<uint16_t> {  // bfloat16 storage
    static constexpr int VEC = 8;   // elements per 16 bytes
    __device__ static float ld(uint16_t x) { return bf2f(x); }
    __device__ static uint16_t st(float x) { return f2bf(x); }
    __device__ static void mma(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    // in[i] holds row-elements (0..7) of k = i; out[j] holds k-elements (0..7) of row j
    __device__ static void transpose(const u32x4_t (&in)[8], u32x4_t (&out)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t x = in[2 * u][j >> 1], y = in[2 * u + 1][j >> 1];
                out[j][u] = (j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
            }
        }
    }
};

template <> struct Elt<float> {
    static constexpr int VEC = 4;
    __device__ static float ld(float x) { return x; }
    __device__ static float st(float x) { return x; }
    __device__ static void mma(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c, 0, 0, 0);
    }
    __device__ static void transpose(const u32x4_t (&in)[4], u32x4_t (&out)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = u32x4_t{in[0][j], in[1][j], in[2][j], in[3][j]};
    }
};

// One operand of a tile.  Element (row, k) of the tile is p[row * ld + k] for a k-contiguous
// source and p[k * ld + row] for a k-strided one.  Rows at or beyond `rows` and k at or beyond
// `kvalid` read as zero and are never dereferenced.
template <typename T> struct Opnd {
    const T* p;
    int64_t ld;
    int rows;
    int kvalid;
};

template <int SEG> struct Pitch { static constexpr int value = SEG * 64 + 16; };

template <typename T, int R, int SEG, bool KS> struct Stager;

// k-contiguous source: 16-byte vectors copied as they are
template <typename T, int R, int SEG> struct Stager<T, R, SEG, false> {
    static constexpr int VEC = Elt<T>::VEC;
    static constexpr int VPR = SEG * 4;  // vectors per row per stage
    static constexpr int NV = R * VPR;
    static constexpr int PER = (NV + kThreads - 1) / kThreads;
    static constexpr int PITCH = Pitch<SEG>::value;
    u32x4_t r[PER];
    __device__ __forceinline__ void load(const Opnd<T>& o, int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * kThreads;
            const int row = v / VPR, c = v % VPR;
            const int k = k0 + c * VEC;
            u32x4_t val = {0u, 0u, 0u, 0u};
            if ((NV % kThreads == 0 || v < NV) && row < o.rows && k < o.kvalid)
                val = *reinterpret_cast<const u32x4_t*>(o.p + (int64_t)row * o.ld + k);
            r[i] = val;
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * kThreads;
            if (NV % kThreads == 0 || v < NV) {
                const int row = v / VPR, c = v % VPR;
                *reinterpret_cast<u32x4_t*>(lds + row * PITCH + c * 16) = r[i];
            }
        }
    }
};

// k-strided source: each thread loads VEC k-rows of VEC row-elements and transposes them
template <typename T, int R, int SEG> struct Stager<T, R, SEG, true> {
    static constexpr int VEC = Elt<T>::VEC;
    static constexpr int KB = SEG * 4;     // k-blocks of VEC per stage (SEG*64 bytes of k)
    static constexpr int RB = R / VEC;     // row blocks
    static constexpr int NB = KB * RB;
    static constexpr int PER = (NB + kThreads - 1) / kThreads;
    static constexpr int PITCH = Pitch<SEG>::value;
    static_assert(R % VEC == 0, "tile rows must be a multiple of the vector width");
    u32x4_t r[PER][VEC];
    __device__ __forceinline__ void load(const Opnd<T>& o, int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = threadIdx.x + i * kThreads;
            const int kb = blk / RB, rb = blk % RB;
            const bool live = (NB % kThreads == 0 || blk < NB) && rb * VEC < o.rows;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int k = k0 + kb * VEC + e;
                u32x4_t val = {0u, 0u, 0u, 0u};
                if (live && k < o.kvalid)
                    val = *reinterpret_cast<const u32x4_t*>(o.p + (int64_t)k * o.ld + rb * VEC);
                r[i][e] = val;
            }
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = threadIdx.x + i * kThreads;
            if (NB % kThreads == 0 || blk < NB) {
                const int kb = blk / RB, rb = blk % RB;
                u32x4_t t[VEC];
                Elt<T>::transpose(r[i], t);
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    *reinterpret_cast<u32x4_t*>(lds + (rb * VEC + j) * PITCH + kb * 16) = t[j];
            }
        }
    }
};

// Tile engine.  NA A-operands of BM rows and NB B-operands of BN rows are staged per k-step;
// accumulator p is A[PM::a[p]] x B[PM::b[p]].  Waves form a WGM x (4/WGM) grid over the tile.
template <typename T, int BM_, int BN_, int SEG, int WGM, int NA, int NB, int NP>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WGN = 4 / WGM;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int PITCH = Pitch<SEG>::value;
    static constexpr int A_BYTES = BM * PITCH, B_BYTES = BN * PITCH;
    static constexpr int STAGE = NA * A_BYTES + NB * B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int KSTEP = SEG * 64 / (int)sizeof(T);  // k elements per stage
    static_assert(WGM * WGN == 4 && FM >= 1 && FN >= 1, "bad wave grid");

    f32x4_t acc[NP][FM][FN];

    template <class PM, bool KSA, bool KSB>
    __device__ __forceinline__ void run(const Opnd<T> (&A)[NA], const Opnd<T> (&B)[NB], int K, char* lds) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[p][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        Stager<T, BM, SEG, KSA> sa[NA];
        Stager<T, BN, SEG, KSB> sb[NB];
        const int nk = (K + KSTEP - 1) / KSTEP;
        if (nk <= 0) return;
#pragma unroll
        for (int a = 0; a < NA; ++a) sa[a].load(A[a], 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) sb[b].load(B[b], 0);
#pragma unroll
        for (int a = 0; a < NA; ++a) sa[a].store(lds + a * A_BYTES);
#pragma unroll
        for (int b = 0; b < NB; ++b) sb[b].store(lds + NA * A_BYTES + b * B_BYTES);
        __syncthreads();
        for (int it = 0; it < nk; ++it) {
            const bool more = it + 1 < nk;
            if (more) {
#pragma unroll
                for (int a = 0; a < NA; ++a) sa[a].load(A[a], (it + 1) * KSTEP);
#pragma unroll
                for (int b = 0; b < NB; ++b) sb[b].load(B[b], (it + 1) * KSTEP);
            }
            compute<PM>(lds + (it & 1) * STAGE);
            if (more) {
                char* nxt = lds + ((it + 1) & 1) * STAGE;
#pragma unroll
                for (int a = 0; a < NA; ++a) sa[a].store(nxt + a * A_BYTES);
#pragma unroll
                for (int b = 0; b < NB; ++b) sb[b].store(nxt + NA * A_BYTES + b * B_BYTES);
            }
            __syncthreads();
        }
    }

    template <class PM>
    __device__ __forceinline__ void compute(const char* st) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
        const int lrow = lane & 15, lk = (lane >> 4) * 16;
#pragma unroll
        for (int seg = 0; seg < SEG; ++seg) {
            u32x4_t af[NA][FM], bfr[NB][FN];
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[a][i] = *reinterpret_cast<const u32x4_t*>(
                        st + a * A_BYTES + (wm * WM + i * 16 + lrow) * PITCH + seg * 64 + lk);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[b][j] = *reinterpret_cast<const u32x4_t*>(
                        st + NA * A_BYTES + b * B_BYTES + (wn * WN + j * 16 + lrow) * PITCH + seg * 64 + lk);
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) Elt<T>::mma(acc[p][i][j], af[PM::a[p]][i], bfr[PM::b[p]][j]);
        }
    }

    // f(const float (&v)[NP], int row, int col) for every accumulator element of this thread
    template <class F>
    __device__ __forceinline__ void for_each(F&& f) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v[NP];
#pragma unroll
                    for (int p = 0; p < NP; ++p) v[p] = acc[p][i][j][r];
                    f(v, wm * WM + i * 16 + (lane >> 4) * 4 + r, wn * WN + j * 16 + (lane & 15));
                }
    }
};

struct PM1 { static constexpr int a[1] = {0}; static constexpr int b[1] = {0}; };
struct PMQ { static constexpr int a[2] = {0, 0}; static constexpr int b[2] = {0, 1}; };
struct PMK { static constexpr int a[3] = {0, 0, 1}; static constexpr int b[3] = {0, 1, 2}; };

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace ttt
