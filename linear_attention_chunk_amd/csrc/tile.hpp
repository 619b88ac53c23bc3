// Device building blocks for gfx950 (CDNA4): element traits, LDS staging of operand tiles and a
// 256-thread (4-wave) MFMA tile engine computing C[i][j] = sum_k A[i][k] * B[j][k].
//
// LDS holds every operand tile k-contiguous: row r of a tile occupies SEG 64-byte k-segments
// followed by 16 bytes of padding, so the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks.  An operand whose source is k-contiguous in memory is copied 16 bytes at a time;
// one whose source is k-strided (token-major data contracted over tokens) is transposed in
// registers, one VEC x VEC block per thread, on its way into LDS.
//
// MFMA fragments.  The tile engine works in 32 x 32 output blocks: for v_mfma_f32_32x32x16_bf16
// lane l supplies row (l % 32) and the 8 k-values of group (l / 32) of a 16-wide k window; in fp32
// four v_mfma_f32_32x32x2_f32 consume the 4 k-values of a lane's 16-byte read one at a time.  A and
// B use the same lane-to-k assignment, so the contraction is complete whatever order the hardware
// walks k in.  Result element r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].  (The 16 x 16
// helpers, Elt<T>::mma, follow the same scheme with 16-row blocks: C[4*(l/16) + r][l % 16].)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// sigmoid with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each)
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Workgroup barrier for handing LDS tiles between waves.  It waits for this wave's own LDS
// operations (lgkmcnt) and meets at s_barrier, but leaves global loads in flight: __syncthreads()
// adds a release fence that also drains every outstanding global load (vmcnt(0)), which would
// cancel the prefetch of later stages.  The asm is a compiler memory barrier, so no LDS access
// moves across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

// Four consecutive elements in the storage type, as one 8-byte (bf16) or 16-byte (fp32) store.
template <typename T> struct Pack4;
template <> struct Pack4<uint16_t> {
    typedef uint32_t raw __attribute__((ext_vector_type(2)));
    __device__ static void store(uint16_t* p, float a, float b, float c, float d) {
        *reinterpret_cast<raw*>(p) = raw{(uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16),
                                         (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16)};
    }
    // four elements as stored (load_raw), and as floats (unpack)
    __device__ static raw load_raw(const uint16_t* p) { return *reinterpret_cast<const raw*>(p); }
    __device__ static void unpack(const raw& r, float (&x)[4]) {
        x[0] = bf2f((uint16_t)(r[0] & 0xFFFFu));
        x[1] = bf2f((uint16_t)(r[0] >> 16));
        x[2] = bf2f((uint16_t)(r[1] & 0xFFFFu));
        x[3] = bf2f((uint16_t)(r[1] >> 16));
    }
};
template <> struct Pack4<float> {
    __device__ static void store(float* p, float a, float b, float c, float d) {
        *reinterpret_cast<f32x4_t*>(p) = f32x4_t{a, b, c, d};
    }
    typedef f32x4_t raw;
    __device__ static raw load_raw(const float* p) { return *reinterpret_cast<const raw*>(p); }
    __device__ static void unpack(const raw& r, float (&x)[4]) {
        x[0] = r[0];
        x[1] = r[1];
        x[2] = r[2];
        x[3] = r[3];
    }
};

// 32 x 32 blocks: one 32-byte k window per call (16 bf16 / 8 fp32 values of k)
template <typename T> struct Mma32;
template <> struct Mma32<uint16_t> {
    __device__ static void mma(f32x16_t& c, const u32x4_t& a, const u32x4_t& b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <> struct Mma32<float> {
    __device__ static void mma(f32x16_t& c, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c, 0, 0, 0);
    }
};

// One operand of a tile.  Element (row, k) of the tile is p[row * ld + k] for a k-contiguous
// source and p[k * ld + row] for a k-strided one.  Rows at or beyond `rows` and k at or beyond
// `kvalid` read as zero and are never dereferenced.
//
// Panels: the contiguous index (k, or row for a k-strided source) may be split into panels of
// 2^ps elements that lie pstride elements apart, i.e. index i is found at (i >> ps) * pstride +
// (i & (2^ps - 1)) instead of i.  A 16-byte vector never straddles two panels (2^ps is a multiple
// of it), and the default ps = 30 means one panel.
template <typename T> struct Opnd {
    const T* p;
    int64_t ld;
    int rows;
    int kvalid;
    int ps = 30;
    int64_t pstride = 0;
    const float* kscale = nullptr;  // per-k factors, used by a k-strided stager built with SCALE
    __device__ __forceinline__ int64_t inner(int i) const {
        return (int64_t)(i >> ps) * pstride + (i & ((1 << ps) - 1));
    }
};

template <int SEG> struct Pitch { static constexpr int value = SEG * 64 + 16; };

template <typename T, int R, int SEG, bool KS, bool SCALE = false, int NT = kThreads> struct Stager;

// k-contiguous source: 16-byte vectors copied as they are
template <typename T, int R, int SEG, int NT> struct Stager<T, R, SEG, false, false, NT> {
    static constexpr int VEC = Elt<T>::VEC;
    static constexpr int VPR = SEG * 4;  // vectors per row per stage
    static constexpr int NV = R * VPR;
    static constexpr int PER = (NV + NT - 1) / NT;
    static constexpr int PITCH = Pitch<SEG>::value;
    // Vector v goes to (row, c).  With one 64-byte segment per row (SEG == 1) four lanes fill a
    // row; the second four lanes of each group of eight take the row 4 further on (80-byte pitch:
    // 4 rows = 320 bytes, which lands on the other 16 of the 32 banks), so every 8-lane store is
    // bank-conflict-free while each row is still read as 64 contiguous bytes.
    static_assert(SEG != 1 || R % 8 == 0, "tile rows must be a multiple of 8");
    __device__ static void place(int v, int& row, int& c) {
        if constexpr (SEG == 1) {
            const int q = v >> 2, g = q >> 1, h = q & 1;
            row = (g & 3) + 4 * h + 8 * (g >> 2);
            c = v & 3;
        } else {
            row = v / VPR;
            c = v % VPR;
        }
    }
    u32x4_t r[PER];
    uint32_t ok;  // bit i: r[i] is in range
    // Branch-free loads: an out-of-range vector is loaded from the operand's first element (always
    // valid) and zeroed only when stored, so no load result is consumed before the LDS store and
    // the loads of a later stage can stay in flight.  FULL: the caller guarantees that every row
    // and k of the tile is in range, and the masking is left out.
    template <bool FULL>
    __device__ __forceinline__ void load(const Opnd<T>& o, int k0) {
        ok = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * NT;
            int row, c;
            place(v, row, c);
            const int k = k0 + c * VEC;
            if constexpr (FULL) {
                if (NV % NT == 0 || v < NV)
                    r[i] = *reinterpret_cast<const u32x4_t*>(o.p + (int64_t)row * o.ld + o.inner(k));
            } else {
                const bool in = (NV % NT == 0 || v < NV) && row < o.rows && k < o.kvalid;
                r[i] = *reinterpret_cast<const u32x4_t*>(o.p + (in ? (int64_t)row * o.ld + o.inner(k) : 0));
                ok |= (uint32_t)in << i;
            }
        }
    }
    template <bool FULL>
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * NT;
            if (NV % NT == 0 || v < NV) {
                int row, c;
                place(v, row, c);
                *reinterpret_cast<u32x4_t*>(lds + row * PITCH + c * 16) =
                    (FULL || ((ok >> i) & 1u)) ? r[i] : u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    }
};

// k-strided source.  A thread takes a unit of KPT consecutive k-rows by VEC row-elements (KPT 16-byte
// loads), and writes, for each of its VEC rows, the KPT k-values as one 4/8/16-byte LDS store.  All
// threads take part (KPT is chosen so that there are about as many units as threads).  The rows
// are stored permuted: logical row rb*VEC + j lives in LDS row j*RB + rb, so that the lanes of one
// store (consecutive rb) hit consecutive LDS rows and distinct banks.  Fragment reads stay on
// consecutive LDS rows; the tile maps result rows back through row_of().
// SCALE: element (row, k) is multiplied by o.kscale[k] on its way into LDS (bf16: rounded once).
template <typename T, int R, int SEG, bool SCALE, int NT> struct Stager<T, R, SEG, true, SCALE, NT> {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int VEC = Elt<T>::VEC;
    static constexpr int KSTEP = SEG * 64 / ES;   // k per stage
    static constexpr int RB = R / VEC;            // row blocks
    static constexpr int KMIN = ES == 2 ? 2 : 1;  // at least one 32-bit word per store
    static constexpr int KWANT = KSTEP * RB / NT;
    static constexpr int KPT = KWANT <= KMIN ? KMIN : (KWANT >= VEC ? VEC : (KWANT >= 4 ? 4 : 2));
    static constexpr int KC = KSTEP / KPT;
    static constexpr int NU = KC * RB;
    static constexpr int PER = (NU + NT - 1) / NT;
    static constexpr int PITCH = Pitch<SEG>::value;
    static constexpr int WORDS = KPT * ES / 4;   // 32-bit words per row piece
    // lanes of one LDS store cycle (128 bytes): 8 consecutive row blocks x KG k-chunks, which puts
    // the group's pieces on 32 distinct banks (rows are 20 dwords apart, chunks KPT*ES bytes apart)
    static constexpr int KG = 128 / (KPT * ES) / 8;
    static_assert(R % VEC == 0 && KSTEP % KPT == 0 && RB % 8 == 0 && KC % KG == 0, "bad k-strided staging shape");
    __device__ static int row_of(int lds_row) { return (lds_row % RB) * VEC + lds_row / RB; }
    __device__ static void place(int u, int& rb, int& kc) {
        const int rb_lo = u % 8;
        int t = u / 8;
        const int kc_lo = t % KG;
        t /= KG;
        rb = (t % (RB / 8)) * 8 + rb_lo;
        kc = (t / (RB / 8)) * KG + kc_lo;
    }

    u32x4_t r[PER][KPT];
    float sc[SCALE ? PER : 1][SCALE ? KPT : 1];
    uint32_t ok;  // bit i * KPT + e: r[i][e] is in range (see the k-contiguous stager)
    static_assert(PER * KPT <= 32, "too many vectors per thread");
    template <bool FULL>
    __device__ __forceinline__ void load(const Opnd<T>& o, int k0) {
        ok = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = threadIdx.x + i * NT;
            int rb, kc;
            place(u, rb, kc);
            const bool live = (NU % NT == 0 || u < NU) && (FULL || rb * VEC < o.rows);
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int k = k0 + kc * KPT + e;
                if constexpr (FULL) {
                    if (NU % NT == 0 || u < NU) {
                        r[i][e] = *reinterpret_cast<const u32x4_t*>(o.p + (int64_t)k * o.ld + o.inner(rb * VEC));
                        if constexpr (SCALE) sc[i][e] = o.kscale[k];
                    }
                } else {
                    const bool in = live && k < o.kvalid;
                    r[i][e] = *reinterpret_cast<const u32x4_t*>(o.p + (in ? (int64_t)k * o.ld + o.inner(rb * VEC) : 0));
                    if constexpr (SCALE) sc[i][e] = o.kscale[in ? k : 0];
                    ok |= (uint32_t)in << (i * KPT + e);
                }
            }
        }
    }
    template <bool FULL>
    __device__ __forceinline__ uint32_t elt(int i, int e, int w) const {
        uint32_t x = r[i][e][w];
        if constexpr (SCALE) {
            const float f = sc[i][e];
            if constexpr (ES == 2) {
                x = (uint32_t)f2bf(bf2f((uint16_t)(x & 0xFFFFu)) * f) | ((uint32_t)f2bf(bf2f((uint16_t)(x >> 16)) * f) << 16);
            } else {
                x = __float_as_uint(__uint_as_float(x) * f);
            }
        }
        return (FULL || ((ok >> (i * KPT + e)) & 1u)) ? x : 0u;
    }
    template <bool FULL>
    __device__ __forceinline__ uint32_t word(int i, int j, int w) const {
        if constexpr (ES == 2) {
            const uint32_t x = elt<FULL>(i, 2 * w, j >> 1), y = elt<FULL>(i, 2 * w + 1, j >> 1);
            return (j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
        } else {
            return elt<FULL>(i, w, j);
        }
    }
    template <bool FULL>
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = threadIdx.x + i * NT;
            if (NU % NT == 0 || u < NU) {
                int rb, kc;
                place(u, rb, kc);
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    char* dst = lds + (j * RB + rb) * PITCH + kc * KPT * ES;
                    if constexpr (WORDS == 1) {
                        *reinterpret_cast<uint32_t*>(dst) = word<FULL>(i, j, 0);
                    } else if constexpr (WORDS == 2) {
                        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
                        *reinterpret_cast<u2*>(dst) = u2{word<FULL>(i, j, 0), word<FULL>(i, j, 1)};
                    } else {
                        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{word<FULL>(i, j, 0), word<FULL>(i, j, 1),
                                                                   word<FULL>(i, j, 2), word<FULL>(i, j, 3)};
                    }
                }
            }
        }
    }
};

template <typename T, int R, int SEG, bool KS> struct RowMap {
    __device__ static int row_of(int r) { return r; }
};
template <typename T, int R, int SEG> struct RowMap<T, R, SEG, true> {
    __device__ static int row_of(int r) { return Stager<T, R, SEG, true>::row_of(r); }
};

// Tile engine (NW waves, 4 by default).  NA A-operands of BM rows and NB B-operands of BN rows
// are staged per k-step
// (k-strided sources when KSA / KSB; SCALE_A multiplies the A operands' k-slices by per-k
// factors); accumulator p is A[PM::a[p]] x B[PM::b[p]].  Waves form a
// WGM x (NW/WGM) grid over the tile and each wave owns (WM/32) x (WN/32) blocks of 32 x 32 per
// accumulator.  Global loads run one stage ahead of the LDS stores (one register set), LDS is
// double-buffered, one barrier per stage.
template <typename T, int BM_, int BN_, int SEG, int WGM, int NA, int NB, int NP, bool KSA, bool KSB,
          bool SCALE_A = false, int NW = 4, int NBUF = 2>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int NT = 64 * NW;  // threads of the workgroup
    static constexpr int WGN = NW / WGM;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int PITCH = Pitch<SEG>::value;
    static constexpr int A_BYTES = BM * PITCH, B_BYTES = BN * PITCH;
    static constexpr int STAGE = NA * A_BYTES + NB * B_BYTES;
    static constexpr int LDS = NBUF * STAGE;  // NBUF = 1: one LDS stage (two barriers per stage)
    static constexpr int KSTEP = SEG * 64 / (int)sizeof(T);  // k elements per stage
    static_assert(WGM * WGN == NW && FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "bad wave grid");
    static_assert(!SCALE_A || KSA, "per-k scaling is done by the k-strided stager");
    using SA = Stager<T, BM, SEG, KSA, SCALE_A, NT>;
    using SB = Stager<T, BN, SEG, KSB, false, NT>;

    f32x16_t acc[NP][FM][FN];

    struct Regs {
        SA a[NA];
        SB b[NB];
    };

    // SYM: the B operand is the A operand (a tile on the diagonal of A A^T); only A is loaded and
    // staged, and compute() reads the B fragments from A's rows
    template <bool FULL, bool SYM = false>
    __device__ __forceinline__ static void issue(Regs& g, const Opnd<T> (&A)[NA], const Opnd<T> (&B)[NB], int k0) {
#pragma unroll
        for (int a = 0; a < NA; ++a) g.a[a].template load<FULL>(A[a], k0);
        if constexpr (!SYM) {
#pragma unroll
            for (int b = 0; b < NB; ++b) g.b[b].template load<FULL>(B[b], k0);
        }
    }
    template <bool FULL, bool SYM = false>
    __device__ __forceinline__ static void put(const Regs& g, char* st) {
#pragma unroll
        for (int a = 0; a < NA; ++a) g.a[a].template store<FULL>(st + a * A_BYTES);
        if constexpr (!SYM) {
#pragma unroll
            for (int b = 0; b < NB; ++b) g.b[b].template store<FULL>(st + NA * A_BYTES + b * B_BYTES);
        }
    }

    // Whether every row and k of a tile over these operands is in range (then the stagers need
    // no masking): all operands hold full tiles and K is a whole number of stages.
    __device__ __forceinline__ static bool full(const Opnd<T> (&A)[NA], const Opnd<T> (&B)[NB], int K) {
        bool f = K % KSTEP == 0;
#pragma unroll
        for (int a = 0; a < NA; ++a) f = f && A[a].rows >= BM && A[a].kvalid >= K;
#pragma unroll
        for (int b = 0; b < NB; ++b) f = f && B[b].rows >= BN && B[b].kvalid >= K;
        return f;
    }

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[p][i][j][r] = 0.f;
    }

    // One output tile: acc = sum over k of the staged products.  LDS is double-buffered and one
    // register set carries the global loads: while stage s is in the MFMAs, stage s + 1 is in LDS
    // and the loads of stage s + 2 are in flight.  With a single set, every load outstanding when a
    // stage is stored belongs to that stage, so the compiler's wait before the LDS store is exact
    // (with two sets its conservative count across the loop edge also waited for the newer set).
    template <class PM, bool FULL, bool SYM = false>
    __device__ __forceinline__ void run_(const Opnd<T> (&A)[NA], const Opnd<T> (&B)[NB], int K, char* lds,
                                         bool keep = false) {
        if (K <= 0) {
            if (!keep) zero();
            return;
        }
        Regs g;
        issue<FULL, SYM>(g, A, B, 0);
        run_issued<PM, FULL, SYM>(g, A, B, K, lds, keep);
    }
    // The same with stage 0 already issued into g (issue<FULL>(g, A, B, 0) with the same FULL), so
    // that a caller can start a tile's first loads early.  K must be positive.  On entry every wave
    // must be done reading the LDS stages.
    template <class PM, bool FULL, bool SYM = false>
    __device__ __forceinline__ void run_issued(Regs& g, const Opnd<T> (&A)[NA], const Opnd<T> (&B)[NB], int K,
                                               char* lds, bool keep = false) {
        if (!keep) zero();
        const int nk = (K + KSTEP - 1) / KSTEP;
        if constexpr (NBUF == 1) {
            // one LDS stage: the loads of stage s + 1 are in flight while stage s is computed; the
            // stage is stored once every wave has finished reading the previous one
            put<FULL, SYM>(g, lds);
            if (nk > 1) issue<FULL, SYM>(g, A, B, KSTEP);
            lds_barrier();
            for (int s = 0; s < nk; ++s) {
                compute<PM, SYM>(lds);
                if (s + 1 < nk) {
                    lds_barrier();
                    put<FULL, SYM>(g, lds);
                    if (s + 2 < nk) issue<FULL, SYM>(g, A, B, (s + 2) * KSTEP);
                    lds_barrier();
                }
            }
            return;
        }
        put<FULL, SYM>(g, lds);
        if (nk > 1) issue<FULL, SYM>(g, A, B, KSTEP);
        lds_barrier();
        for (int s = 0; s < nk; ++s) {
            compute<PM, SYM>(lds + (s & 1) * STAGE);
            if (s + 1 < nk) put<FULL, SYM>(g, lds + ((s + 1) & 1) * STAGE);
            if (s + 2 < nk) issue<FULL, SYM>(g, A, B, (s + 2) * KSTEP);
            lds_barrier();
        }
    }
    // Full tiles (the common case) take the unmasked path; the branch is uniform per workgroup.
    template <class PM>
    // keep: add to the accumulators instead of starting from zero
    __device__ __forceinline__ void run(const Opnd<T> (&A)[NA], const Opnd<T> (&B)[NB], int K, char* lds,
                                        bool keep = false) {
        if (full(A, B, K)) run_<PM, true>(A, B, K, lds, keep);
        else run_<PM, false>(A, B, K, lds, keep);
    }
    // A tile on the diagonal of A A^T: run() with B = A, loading and staging A only
    template <class PM>
    __device__ __forceinline__ void run_sym(const Opnd<T> (&A)[NA], int K, char* lds) {
        static_assert(NA == 1 && NB == 1 && BM == BN && KSA == KSB && !SCALE_A, "B must stage exactly like A");
        if (full(A, A, K)) run_<PM, true, true>(A, A, K, lds);
        else run_<PM, false, true>(A, A, K, lds);
    }

    template <class PM, bool SYM = false>
    __device__ __forceinline__ void compute(const char* st) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
        const int lrow = lane & 31, lk = (lane >> 5) * 16;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int win = 0; win < SEG * 2; ++win) {  // 32-byte k windows
            u32x4_t af[NA][FM], bfr[NB][FN];
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[a][i] = *reinterpret_cast<const u32x4_t*>(
                        st + a * A_BYTES + (wm * WM + i * 32 + lrow) * PITCH + win * 32 + lk);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[b][j] = *reinterpret_cast<const u32x4_t*>(
                        st + (SYM ? 0 : NA * A_BYTES + b * B_BYTES) + (wn * WN + j * 32 + lrow) * PITCH + win * 32 + lk);
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) Mma32<T>::mma(acc[p][i][j], af[PM::a[p]][i], bfr[PM::b[p]][j]);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // compute() over the stage's 32-byte k windows W0 .. W1 - 1 only (k from W0 * 32 / sizeof(T) on)
    template <class PM, int W0, int W1>
    __device__ __forceinline__ void compute_win(const char* st) {
        static_assert(0 <= W0 && W0 < W1 && W1 <= SEG * 2, "windows of one stage");
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
        const int lrow = lane & 31, lk = (lane >> 5) * 16;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int win = W0; win < W1; ++win) {
            u32x4_t af[NA][FM], bfr[NB][FN];
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[a][i] = *reinterpret_cast<const u32x4_t*>(
                        st + a * A_BYTES + (wm * WM + i * 32 + lrow) * PITCH + win * 32 + lk);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[b][j] = *reinterpret_cast<const u32x4_t*>(
                        st + NA * A_BYTES + b * B_BYTES + (wn * WN + j * 32 + lrow) * PITCH + win * 32 + lk);
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) Mma32<T>::mma(acc[p][i][j], af[PM::a[p]][i], bfr[PM::b[p]][j]);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    static constexpr int ELEMS = FM * FN * 16;  // accumulator elements per thread and accumulator

    // f(int idx, int row, int col) over the positions for_each visits, in the same order
    // (idx = 0 .. ELEMS-1); usable before run(), e.g. to prefetch epilogue operands
    template <class F>
    __device__ __forceinline__ static void for_each_pos(F&& f) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = RowMap<T, BN, SEG, KSB>::row_of(wn * WN + j * 32 + (lane & 31));
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    f((i * FN + j) * 16 + r,
                      RowMap<T, BM, SEG, KSA>::row_of(wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)), col);
            }
    }

    // f(const float (&v)[NP][4], int row, int col) for every group of 4 accumulator elements of
    // this thread that share a column and cover rows row .. row + 3 (row a multiple of 4).  Only
    // for k-contiguous A operands, whose tile rows are not permuted.
    template <class F>
    __device__ __forceinline__ void for_each4(F&& f) const {
        static_assert(!KSA, "row groups need unpermuted rows");
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = RowMap<T, BN, SEG, KSB>::row_of(wn * WN + j * 32 + (lane & 31));
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[NP][4];
#pragma unroll
                    for (int p = 0; p < NP; ++p)
#pragma unroll
                        for (int u = 0; u < 4; ++u) v[p][u] = acc[p][i][j][4 * g + u];
                    f(v, wm * WM + i * 32 + 8 * g + 4 * (lane >> 5), col);
                }
            }
    }

    // Row-major view of the accumulators through LDS, for tiles whose output columns are permuted
    // (k-strided B operand) so that a lane's elements lie 8 columns apart.  For each accumulator p
    // and each band of WM staged rows (the rows of one wave row), the waves that own the band write
    // it to LDS with its columns in logical order, then all threads read it back four columns at a
    // time and call f(idx, p, row, col, float4): row is the logical tile row (k-strided A rows are
    // mapped back), col a multiple of 4, and idx = 0 .. RV_N - 1 in the order of rows_via_lds_pos.
    // A wave covers whole 4 * BN-byte row segments.  Needs RV_LDS bytes of LDS; every wave must be
    // done with the tile's LDS stages.
    static constexpr int RV_PITCH = BN + 4;  // floats: rows stay 16-byte aligned
    static constexpr int RV_LDS = WM * RV_PITCH * 4;
    static constexpr int RV_K = WM * BN / 4 / NT;  // float4 per thread per band
    static constexpr int RV_N = NP * WGM * RV_K;   // float4 per thread in all
    static_assert((WM * BN / 4) % NT == 0, "a band is a whole number of rounds of the workgroup");

    // f(idx, p, row, col) over the positions rows_via_lds visits, in the same order; usable before
    // run(), e.g. to prefetch epilogue operands
    template <class F>
    __device__ __forceinline__ static void rows_via_lds_pos(F&& f) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int h = 0; h < WGM; ++h)
#pragma unroll
                for (int k = 0; k < RV_K; ++k) {
                    const int q = k * NT + (int)threadIdx.x;
                    f((p * WGM + h) * RV_K + k, p, RowMap<T, BM, SEG, KSA>::row_of(h * WM + q / (BN / 4)),
                      (q % (BN / 4)) * 4);
                }
    }

    // (NPU: only the first NPU accumulators are written out)
    template <int NPU = NP, class F>
    __device__ __forceinline__ void rows_via_lds(char* lds, F&& f) const {
        static_assert(NPU >= 1 && NPU <= NP, "bad accumulator count");
        float* band = reinterpret_cast<float*>(lds);
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
        for (int p = 0; p < NPU; ++p)
#pragma unroll
            for (int h = 0; h < WGM; ++h) {
                lds_barrier();
                if (wm == h) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const int col = RowMap<T, BN, SEG, KSB>::row_of(wn * WN + j * 32 + (lane & 31));
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                band[(i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * RV_PITCH + col] = acc[p][i][j][r];
                        }
                }
                lds_barrier();
#pragma unroll
                for (int k = 0; k < RV_K; ++k) {
                    const int q = k * NT + (int)threadIdx.x, row = q / (BN / 4), c = (q % (BN / 4)) * 4;
                    f((p * WGM + h) * RV_K + k, p, RowMap<T, BM, SEG, KSA>::row_of(h * WM + row), c,
                      *reinterpret_cast<const float4*>(band + row * RV_PITCH + c));
                }
            }
    }

    // f(const float (&v)[NP], int row, int col) for every accumulator element of this thread,
    // with row / col the logical tile coordinates
    template <class F>
    __device__ __forceinline__ void for_each(F&& f) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / WGN, wn = wave % WGN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = RowMap<T, BN, SEG, KSB>::row_of(wn * WN + j * 32 + (lane & 31));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v[NP];
#pragma unroll
                    for (int p = 0; p < NP; ++p) v[p] = acc[p][i][j][r];
                    f(v, RowMap<T, BM, SEG, KSA>::row_of(wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)), col);
                }
            }
    }
};

struct PM1 { static constexpr int a[1] = {0}; static constexpr int b[1] = {0}; };
struct PMQ { static constexpr int a[2] = {0, 0}; static constexpr int b[2] = {0, 1}; };
struct PMK { static constexpr int a[3] = {0, 0, 1}; static constexpr int b[3] = {0, 1, 2}; };
struct PMG { static constexpr int a[2] = {0, 1}; static constexpr int b[2] = {0, 0}; };
struct PMKT { static constexpr int a[3] = {0, 1, 2}; static constexpr int b[3] = {0, 0, 1}; };

// Workgroups are dispatched to the 8 XCDs round-robin (block b runs on XCD b % 8).  Renumbering so
// that the blocks one XCD receives are consecutive logical blocks keeps tiles that share operands
// (the same scan, the same rows) in the same L2.
__device__ __forceinline__ int xcd_block(int nblocks) {
    const int b = blockIdx.x;
    if (nblocks % 8 != 0) return b;
    return (b % 8) * (nblocks / 8) + b / 8;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace ttt
