// Host-side driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the library's host
// code (the dispatcher: descriptor validation, workspace layouts, buffer checks, status strings and
// the profiler's host side).  It needs no GPU: every call either fails validation, or reaches the
// device-buffer check with fake addresses and stops there (TTT_ERR_DEVICE without a device,
// TTT_ERR_INVALID_ARGUMENT with one), so nothing is ever launched.  A fixed table of edge cases is
// followed by a seeded fuzz over descriptors, valid and invalid.  Exit status 0 means every call
// returned a known status with a message where one is due, and the sanitizers reported nothing.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ttt.h"

static int g_fail = 0;
#define EXPECT(c)                                                               \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                           \
        }                                                                       \
    } while (0)

// splitmix64: a small deterministic generator for the fuzz
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int pick(const int* v, int n) { return v[next_u64() % (uint64_t)n]; }

static const uintptr_t P = 0x7F0000000000ull;  // fake device addresses, never dereferenced

static bool known(ttt_status s) { return s >= TTT_OK && s <= TTT_ERR_DEVICE; }

static void check_message(ttt_status s) {
    EXPECT(known(s));
    EXPECT(ttt_status_string(s) != nullptr);
    if (s != TTT_OK) EXPECT(strlen(ttt_last_error()) > 0);
}

static void run_ttt(ttt_desc D) {
    size_t need = 0;
    ttt_status s = ttt_workspace_bytes(&D, &need);
    check_message(s);
    // every buffer far apart, 256-byte aligned; a workspace of exactly the size asked for
    const void* q = (const void*)(P);
    const void* k = (const void*)(P + (1ull << 36));
    const void* v = (const void*)(P + (2ull << 36));
    const float* eta = (const float*)(P + (3ull << 36));
    const float* W0 = (const float*)(P + (4ull << 36));
    void* o = (void*)(P + (5ull << 36));
    float* Wout = (float*)(P + (6ull << 36));
    float* M = (float*)(P + (7ull << 36));
    void* ws = (void*)(P + (8ull << 36));
    ttt_status f = ttt_forward(&D, q, k, v, eta, W0, o, Wout, D.momentum != 0.f ? M : nullptr, ws, need, nullptr);
    check_message(f);
    if (s != TTT_OK) {
        EXPECT(f == s || f == TTT_ERR_INVALID_ARGUMENT);  // the same descriptor fails the call too
    } else if ((int64_t)D.B * D.H > 0) {
        EXPECT(f == TTT_ERR_DEVICE || f == TTT_ERR_INVALID_ARGUMENT);  // stops at the buffer check
    }
    // a workspace one byte short is refused before any buffer is looked at
    if (s == TTT_OK && need > 0 && (int64_t)D.B * D.H > 0)
        EXPECT(ttt_forward(&D, q, k, v, eta, W0, o, Wout, nullptr, ws, need - 1, nullptr) == TTT_ERR_WORKSPACE);
    // the backward: the forward's checks, then the layer it covers (W2 alone by GD [+ L2], per-token rates)
    size_t bneed = 0;
    ttt_status bs = ttt_backward_workspace_bytes(&D, &bneed);
    check_message(bs);
    if (s != TTT_OK) EXPECT(bs == s);
    // (W2 alone by GD, else the recurrence with at most 65536 recorded updates)
    const int64_t nupd = (D.N > 0 && D.chunk > 0 ? ((int64_t)D.N + D.chunk - 1) / D.chunk : 0) * (D.inner_steps > 1 ? D.inner_steps : 1);
    const bool gd = D.rule == TTT_UPD_GD || D.rule == TTT_UPD_GD_L2;
    const bool covered = D.chunk_rates == 0 && ((D.last_layer_only == 1 && gd) || nupd <= 65536);
    if (s == TTT_OK && !covered) EXPECT(bs == TTT_ERR_UNSUPPORTED);
    const void* dO = (const void*)(P + (9ull << 36));
    void* dq = (void*)(P + (10ull << 36));
    void* dk = (void*)(P + (11ull << 36));
    void* dv = (void*)(P + (12ull << 36));
    float* deta = (float*)(P + (13ull << 36));
    float* dW0 = (float*)(P + (14ull << 36));
    void* bws = (void*)(P + (15ull << 36));
    ttt_status bf = ttt_backward(&D, q, k, v, eta, W0, dO, nullptr, dq, dk, dv, deta, dW0, bws, bneed, nullptr);
    check_message(bf);
    if (bs != TTT_OK) EXPECT(bf == bs || bf == TTT_ERR_INVALID_ARGUMENT);
    else if ((int64_t)D.B * D.H > 0) EXPECT(bf == TTT_ERR_DEVICE || bf == TTT_ERR_INVALID_ARGUMENT);
    if (bs == TTT_OK && bneed > 0 && (int64_t)D.B * D.H > 0)
        EXPECT(ttt_backward(&D, q, k, v, eta, W0, dO, nullptr, dq, dk, dv, deta, dW0, bws, bneed - 1, nullptr) ==
               TTT_ERR_WORKSPACE);
    // the training pair: the recurrence's backward only, then the same buffer checks
    size_t rb = 0, rw = 0, bw = 0;
    ttt_status rs = ttt_record_bytes(&D, &rb, &rw);
    check_message(rs);
    if (s != TTT_OK) EXPECT(rs == s);
    if (s == TTT_OK && bs == TTT_OK && (!gd || D.last_layer_only == 0)) EXPECT(rs == TTT_OK);
    if (rs == TTT_OK && (int64_t)D.B * D.H > 0) {
        void* rec = (void*)(P + (16ull << 36));
        ttt_status fr = ttt_forward_record(&D, q, k, v, eta, W0, o, Wout, rec, rb, ws, rw, nullptr);
        check_message(fr);
        EXPECT(fr == TTT_ERR_DEVICE || fr == TTT_ERR_INVALID_ARGUMENT);
        EXPECT(ttt_backward_record_workspace_bytes(&D, &bw) == TTT_OK);
        ttt_status br = ttt_backward_record(&D, q, k, v, eta, rec, rb, dO, nullptr, dq, dk, dv, deta, dW0, bws, bw, nullptr);
        check_message(br);
        EXPECT(br == TTT_ERR_DEVICE || br == TTT_ERR_INVALID_ARGUMENT);
        EXPECT(ttt_backward_record(&D, q, k, v, eta, rec, rb - 1, dO, nullptr, dq, dk, dv, deta, dW0, bws, bw, nullptr) ==
               TTT_ERR_WORKSPACE);
    }
}

static void run_lin(linattn_desc D) {
    size_t need = 0;
    ttt_status s = linattn_workspace_bytes(&D, &need);
    check_message(s);
    ttt_status f = linattn_forward(&D, (const void*)P, (const void*)(P + (1ull << 36)), (const void*)(P + (2ull << 36)),
                                   (const float*)(P + (3ull << 36)), (const float*)(P + (4ull << 36)),
                                   (void*)(P + (5ull << 36)), (float*)(P + (6ull << 36)), (void*)(P + (8ull << 36)),
                                   need, nullptr);
    check_message(f);
    if (s == TTT_OK && (int64_t)D.B * D.H > 0) EXPECT(f == TTT_ERR_DEVICE || f == TTT_ERR_INVALID_ARGUMENT);
    // the backward: its own validation (chunked masks only), then the same buffer check
    size_t bneed = 0;
    ttt_status bs = linattn_backward_workspace_bytes(&D, &bneed);
    check_message(bs);
    if (s != TTT_OK) EXPECT(bs != TTT_OK);
    if (D.mask == TTT_MASK_TOKEN_CAUSAL && s == TTT_OK) EXPECT(bs == TTT_ERR_UNSUPPORTED);
    ttt_status bf = linattn_backward(&D, (const void*)P, (const void*)(P + (1ull << 36)), (const void*)(P + (2ull << 36)),
                                     (const float*)(P + (3ull << 36)), nullptr, (const void*)(P + (4ull << 36)), nullptr,
                                     (void*)(P + (5ull << 36)), (void*)(P + (6ull << 36)), (void*)(P + (7ull << 36)),
                                     (float*)(P + (9ull << 36)), nullptr, (void*)(P + (10ull << 36)), bneed, nullptr);
    check_message(bf);
    // (N = 0 with no dS0 asked for has nothing to do)
    if (bs == TTT_OK && (int64_t)D.B * D.H > 0)
        EXPECT(D.N == 0 ? bf == TTT_OK : (bf == TTT_ERR_DEVICE || bf == TTT_ERR_INVALID_ARGUMENT));
    if (bs == TTT_OK && (int64_t)D.B * D.H > 0 && bneed > 0)
        EXPECT(linattn_backward(&D, (const void*)P, (const void*)(P + (1ull << 36)), (const void*)(P + (2ull << 36)),
                                (const float*)(P + (3ull << 36)), nullptr, (const void*)(P + (4ull << 36)), nullptr,
                                (void*)(P + (5ull << 36)), (void*)(P + (6ull << 36)), (void*)(P + (7ull << 36)),
                                (float*)(P + (9ull << 36)), nullptr, (void*)(P + (10ull << 36)), bneed - 1,
                                nullptr) == TTT_ERR_WORKSPACE);
}

static ttt_desc base_desc() {
    ttt_desc D;
    memset(&D, 0, sizeof D);
    D.B = 2; D.H = 4; D.N = 256; D.d_h = 64; D.m_h = 128; D.chunk = 64;
    D.io_dtype = TTT_BF16; D.mask = TTT_MASK_APPLY_THEN_UPDATE; D.rule = TTT_UPD_GD_L2; D.ns_iters = 5;
    D.inner_steps = 1;
    return D;
}

int main() {
    static uint8_t flags[4096];
    for (int i = 0; i < 4096; ++i) flags[i] = (uint8_t)(i % 3 != 1);

    EXPECT(ttt_abi_version() == TTT_ABI_VERSION);
    for (int s = 0; s < 8; ++s) EXPECT(ttt_status_string((ttt_status)s) != nullptr);
    EXPECT(strcmp(ttt_status_string(TTT_STATUS_MAX_ENUM), "unknown status") == 0);
    EXPECT(ttt_workspace_bytes(nullptr, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    {
        ttt_desc D = base_desc();
        EXPECT(ttt_workspace_bytes(&D, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    }
    EXPECT(linattn_workspace_bytes(nullptr, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    EXPECT(ttt_forward(nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    EXPECT(linattn_forward(nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    EXPECT(linattn_backward_workspace_bytes(nullptr, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    EXPECT(ttt_backward_workspace_bytes(nullptr, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    EXPECT(ttt_backward(nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    EXPECT(linattn_backward(nullptr, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, nullptr) == TTT_ERR_INVALID_ARGUMENT);

    // the profiler's host side: names, selection, a read with nothing recorded, bad sizes
    for (int i = -2; i < TTT_PROF_KERNELS + 2; ++i) EXPECT(ttt_profile_kernel_name(i) != nullptr);
    EXPECT(ttt_profile_select(0x5u) == TTT_OK);
    EXPECT(ttt_profile_select(0xFFFFFFFFu) == TTT_OK);
    {
        float ms[TTT_PROF_KERNELS];
        int32_t cnt[TTT_PROF_KERNELS];
        EXPECT(ttt_profile_read(ms, cnt, TTT_PROF_KERNELS) == TTT_OK);
        for (int i = 0; i < TTT_PROF_KERNELS; ++i) EXPECT(cnt[i] == 0);
        EXPECT(ttt_profile_read(nullptr, cnt, TTT_PROF_KERNELS) == TTT_ERR_INVALID_ARGUMENT);
        EXPECT(ttt_profile_read(ms, cnt, -1) == TTT_ERR_INVALID_ARGUMENT);
        EXPECT(ttt_profile_read(ms, cnt, TTT_PROF_KERNELS + 1) == TTT_ERR_INVALID_ARGUMENT);
    }
    EXPECT(ttt_probe_mfma_bf16(0, 1, (float*)P, nullptr) == TTT_ERR_INVALID_ARGUMENT);

    // fixed edge cases of the layer
    {
        const int dims[][2] = {{32, 32}, {64, 160}, {384, 768}, {2048, 64}, {64, 2048}, {2048, 2048}, {96, 32}};
        const int masks[] = {TTT_MASK_FULL, TTT_MASK_UPDATE_THEN_APPLY, TTT_MASK_APPLY_THEN_UPDATE, TTT_MASK_STRIDED};
        const int rules[] = {TTT_UPD_GD, TTT_UPD_GD_L2, TTT_UPD_MUON_L2, TTT_UPD_MUON};
        for (const auto& dm : dims)
            for (int mk : masks)
                for (int r : rules)
                    for (int io = 0; io < 2; ++io)
                        for (int last = 0; last < 2; ++last) {
                            ttt_desc D = base_desc();
                            D.d_h = dm[0]; D.m_h = dm[1]; D.mask = mk; D.rule = r; D.io_dtype = io;
                            D.last_layer_only = last;
                            D.momentum = (r >= TTT_UPD_MUON_L2) ? 0.9f : 0.f;
                            D.N = 300; D.chunk = mk == TTT_MASK_FULL ? 300 : 96;
                            D.update_chunks = flags;
                            run_ttt(D);
                            D.parallel_form = 1;
                            run_ttt(D);
                        }
        ttt_desc D = base_desc();
        D.N = 0; run_ttt(D);
        D = base_desc(); D.B = 0; run_ttt(D);
        D = base_desc(); D.N = 1; D.chunk = 4096; run_ttt(D);
        D = base_desc(); D.B = 8; D.H = 4; D.N = 32768; D.d_h = 384; D.m_h = 768; D.chunk = 2048; run_ttt(D);
        D.rule = TTT_UPD_MUON_L2; D.momentum = 0.9f; run_ttt(D);
        D = base_desc(); D.B = 8; D.H = 4; D.N = 32768; D.d_h = 384; D.m_h = 768; D.chunk = 2048;
        D.rule = TTT_UPD_GD; D.last_layer_only = 1; run_ttt(D);            // the backward's workload
        D.w0_per_batch = 1; D.ascent = 1; D.inner_steps = 4; run_ttt(D);
        D = base_desc(); D.B = 1 << 20; D.H = 2; run_ttt(D);            // B*H beyond the limit
        D = base_desc(); D.N = 0x7FFFFFFF; D.chunk = 0x7FFFFFFF; run_ttt(D);
        D = base_desc(); D.m_h = 2048; D.chunk = 1 << 20; D.N = 1 << 20; run_ttt(D);
    }
    // fixed edge cases of linear attention
    {
        const int masks[] = {TTT_MASK_FULL, TTT_MASK_UPDATE_THEN_APPLY, TTT_MASK_APPLY_THEN_UPDATE, TTT_MASK_STRIDED,
                             TTT_MASK_TOKEN_CAUSAL};
        const int dk[] = {32, 128, 256, 384, 2048}, dv[] = {32, 96, 4096};
        const int ch[] = {1, 16, 128, 2048};
        for (int mk : masks)
            for (int a : dk)
                for (int b : dv)
                    for (int c : ch) {
                        linattn_desc D;
                        memset(&D, 0, sizeof D);
                        D.B = 2; D.H = 3; D.N = 1000; D.d_k = a; D.d_v = b; D.chunk = mk == TTT_MASK_FULL ? 1000 : c;
                        D.io_dtype = TTT_BF16; D.mask = mk; D.update_chunks = flags;
                        run_lin(D);
                    }
    }
    // sliding-window attention: valid and invalid descriptors, every call stopping at the buffer check
    {
        const int ds[] = {-32, 0, 31, 32, 96, 128, 192, 256, 320, 384, 416}, ws[] = {-1, 0, 1, 7, 2048, 1 << 30};
        const int Ns[] = {-1, 0, 1, 127, 128, 129, 1000}, ios[] = {-1, 0, 1, 2};
        for (int it = 0; it < 4000; ++it) {
            swa_desc D;
            memset(&D, 0, sizeof D);
            D.B = (int)(next_u64() % 4) - 1; D.H = (int)(next_u64() % 4); D.N = pick(Ns, 7); D.d = pick(ds, 11);
            D.window = pick(ws, 6); D.io_dtype = pick(ios, 4);
            size_t need = 0;
            ttt_status s = swa_workspace_bytes(&D, &need);
            check_message(s);
            ttt_status f = swa_forward(&D, (const void*)P, (const void*)(P + (1ull << 36)), (const void*)(P + (2ull << 36)),
                                       (const float*)(P + (3ull << 36)), nullptr, (const float*)(P + (4ull << 36)), nullptr,
                                       (void*)(P + (5ull << 36)), (void*)(P + (8ull << 36)), need, nullptr);
            check_message(f);
            if (s == TTT_OK && (int64_t)D.B * D.H > 0 && D.N > 0) EXPECT(f == TTT_ERR_DEVICE || f == TTT_ERR_INVALID_ARGUMENT);
            if (s == TTT_OK && (int64_t)D.B * D.H > 0 && D.N > 0)
                EXPECT(swa_forward(&D, (const void*)P, (const void*)P, (const void*)P, nullptr, nullptr, nullptr, nullptr,
                                   (void*)(P + (5ull << 36)), (void*)(P + (8ull << 36)), need - 1, nullptr) == TTT_ERR_WORKSPACE);
        }
        EXPECT(swa_workspace_bytes(nullptr, nullptr) == TTT_ERR_INVALID_ARGUMENT);
    }
    // seeded fuzz: each field from a list of valid values and out-of-range ones
    {
        const int Bs[] = {-1, 0, 1, 2, 3, 8}, Hs[] = {0, 1, 4, 16}, Ns[] = {-5, 0, 1, 63, 64, 300, 2049, 65536};
        const int ds[] = {-32, 0, 31, 32, 64, 100, 384, 2048, 2080}, chunks[] = {-1, 0, 1, 7, 64, 96, 2048, 70000};
        const int ios[] = {-1, 0, 1, 2}, maskv[] = {-1, 0, 1, 2, 3, 4, 5}, rulev[] = {-1, 0, 1, 2, 3, 4};
        const int nsv[] = {-1, 0, 1, 5, 32, 33}, bits[] = {-1, 0, 1, 2}, inner[] = {-1, 0, 1, 3, 64, 65};
        const float moms[] = {0.f, 0.5f, 0.9f, -1.f, 1e31f};
        for (int it = 0; it < 20000; ++it) {
            ttt_desc D;
            memset(&D, 0, sizeof D);
            D.B = pick(Bs, 6); D.H = pick(Hs, 4); D.N = pick(Ns, 8);
            D.d_h = pick(ds, 9); D.m_h = pick(ds, 9); D.chunk = pick(chunks, 8);
            D.io_dtype = pick(ios, 4); D.mask = pick(maskv, 7); D.rule = pick(rulev, 6);
            D.ns_iters = pick(nsv, 6); D.momentum = moms[next_u64() % 5];
            D.last_layer_only = pick(bits, 4); D.w0_per_batch = pick(bits, 4);
            D.update_chunks = (next_u64() & 7) ? flags : nullptr;
            D.inner_steps = pick(inner, 6); D.ascent = pick(bits, 4); D.parallel_form = pick(bits, 4);
            D.chunk_rates = pick(bits, 4);
            D.chunk_momentum = (next_u64() & 1) ? (const float*)(P + (9ull << 36)) : nullptr;
            // flags cover at most 4096 chunks: keep strided fuzz cases within them
            if (D.mask == TTT_MASK_STRIDED && D.chunk > 0 && D.N > 0 && (D.N + (int64_t)D.chunk - 1) / D.chunk > 4096)
                D.chunk = D.N;
            run_ttt(D);
            linattn_desc L;
            memset(&L, 0, sizeof L);
            L.B = D.B; L.H = D.H; L.N = D.N; L.d_k = pick(ds, 9); L.d_v = pick(ds, 9); L.chunk = D.chunk;
            L.io_dtype = D.io_dtype; L.mask = D.mask; L.update_chunks = D.update_chunks;
            run_lin(L);
        }
    }
    if (g_fail) {
        fprintf(stderr, "%d expectation(s) failed\n", g_fail);
        return 1;
    }
    printf("sanitized host driver: all calls returned known statuses\n");
    return 0;
}
