/*
 * ttt.h -- C ABI of the MI355X (gfx950) large-chunk TTT-KVB layer and chunked linear attention.
 *
 * The layer is the one described in the PaperTrace notes "5.2.1 LaCT and TTT-E2E" (Eqs. (2)-(6)
 * and (10), section 1.1 on mask orders) and shown to be learned linear attention in
 * "Test-Time Training with KV Binding Is Secretly Linear Attention" (Thm. 5.1-5.3, Sec. 6.1,
 * App. E and H).  Per (batch, head) and per chunk of `chunk` tokens it
 *   - applies the bias-free SwiGLU fast weight f_W(x) = W2 [SiLU(W1 x) o (W3 x)] to the queries
 *     (Eq. (3); all queries of a chunk see one W),
 *   - takes the gradient g of sum_i eta_i * (-f_W(k_i)^T v_i) over the chunk (Eqs. (2), (4)),
 *   - updates W <- W - g, W <- L2-Normalize(W - g) (Eq. (5)) or
 *     W <- L2-Normalize(W - Muon(g)) (Eq. (6), Newton-Schulz, optional chunk momentum),
 *   - carries W to the next chunk, in the order the mask selects (section 1.1, Eq. (10)).
 * linattn_forward computes the linear, bias-free reduction: S <- S + sum_i eta_i v_i k_i^T,
 * o = S q (paper Thm. 5.2 and Sec. 6.1 Step 6).
 *
 * Conventions shared by every entry point
 *   - Layout: q, k, v, o are [B][H][N][d] row-major (token rows, feature columns); eta is
 *     [B][H][N] fp32.  A head's fast weight is one fp32 block [W1 | W3 | W2]: W1 and W3 are
 *     m_h x d_h row-major (output unit, input feature), W2 is d_h x m_h row-major.
 *     L2-Normalize scales each row (an output unit over its inputs) to unit norm.
 *   - Memory: every pointer except `desc` and `update_chunks` is a device pointer on the
 *     current HIP device.  The caller allocates every buffer, including the workspace, and
 *     keeps it alive until the stream reaches the end of the call; the library allocates no
 *     device memory and keeps no pointer after a call returns.
 *   - Streams: work is enqueued on `stream` (a hipStream_t; NULL = the null stream); the call
 *     returns before the work finishes.
 *   - Errors: arguments are checked before anything is enqueued, so a call that returns an
 *     error has written nothing.  Besides sizes, enums and alignment, every device pointer must
 *     lie in an allocation that HIP made on a device and that holds all the bytes the call reads
 *     or writes from it (hipMemGetAddressRange); otherwise TTT_ERR_INVALID_ARGUMENT, or
 *     TTT_ERR_DEVICE when no HIP device is usable.  A failed launch returns TTT_ERR_DEVICE; a
 *     device fault shows up at the caller's next synchronisation, or, with the environment
 *     variable TTT_DEBUG_SYNC set (not "0"), as TTT_ERR_DEVICE from the call that launched the
 *     kernel (every launch is then followed by a stream synchronisation: a debugging aid, not for
 *     streams under graph capture).  ttt_last_error() gives a message for the latest failed call
 *     on the calling thread.
 *   - Pass choice (testing aid): chunked linear attention's chunk updates and scan over chunks run
 *     either as one fused pass or as two (the updates to memory, then the scan), chosen by shape;
 *     the environment variable TTT_LIN_PASS, read on every call, forces "fused" or "split" where
 *     no step runs between the two (not for Muon's parallel form).  Both give the same results.
 *   - Aliasing: o must not overlap q, k, v or eta.  W_out may not overlap W0.
 *   - Thread safety: calls on different streams may run concurrently; the only mutable global
 *     state is the per-thread error message and the optional launch profiler below.
 */
#ifndef TTT_MI355X_H
#define TTT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TTT_ABI_VERSION 7

typedef enum {
    TTT_OK = 0,
    TTT_ERR_INVALID_ARGUMENT = 1, /* a size, pointer, alignment or enum value is out of range     */
    TTT_ERR_UNSUPPORTED = 2,      /* a valid combination the library does not implement         */
    TTT_ERR_WORKSPACE = 3,        /* workspace pointer missing or smaller than *_workspace_bytes  */
    TTT_ERR_DEVICE = 4,           /* a HIP call or kernel launch failed                          */
    TTT_STATUS_MAX_ENUM = 0x7FFFFFFF  /* not a status: makes every value 0 .. INT32_MAX a valid
                                         ttt_status, so ttt_status_string() may be asked about any */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* The update/apply orders of the notes' section 1.1 ("the order of update and apply decides the
 * mask").  Chunk j covers tokens [j*chunk, min((j+1)*chunk, N)); the last chunk may be shorter. */
typedef enum {
    TTT_MASK_FULL = 0,              /* one chunk (chunk >= N): update, then apply -> bidirectional */
    TTT_MASK_UPDATE_THEN_APPLY = 1, /* per chunk: update, then apply -> own chunk visible           */
    TTT_MASK_APPLY_THEN_UPDATE = 2, /* per chunk: apply, then update -> earlier chunks only, Eq.(10)*/
    TTT_MASK_STRIDED = 3,           /* apply then update, update only where update_chunks[j] != 0  */
    TTT_MASK_TOKEN_CAUSAL = 4       /* linattn_forward only: token t sees tokens s <= t            */
} ttt_mask_mode;

typedef enum {
    TTT_UPD_GD = 0,      /* W <- W - U                                                         */
    TTT_UPD_GD_L2 = 1,   /* W <- L2-Normalize(W - U), Eq. (5)                                   */
    TTT_UPD_MUON_L2 = 2, /* W <- L2-Normalize(W - Muon(U)), Eq. (6)                             */
    TTT_UPD_MUON = 3     /* W <- W - Muon(U): Muon without the weight norm (paper Table 2, V2)  */
} ttt_update_rule;
/* U is the chunk gradient g, or the momentum M <- momentum * M + g when momentum != 0 (the
 * notes' text after Eq. (6)).  Muon(U): X <- U / (||U||_F + 1e-7), then ns_iters steps of
 * X <- 1.5 X - 0.5 (X X^T) X taken on the side with the smaller Gram matrix. */

typedef struct ttt_desc {
    int32_t B, H, N;          /* batch, heads, tokens per sequence (any may be 0: nothing to do) */
    int32_t d_h, m_h;         /* head width and SwiGLU hidden width: multiples of 32, <= 2048   */
    int32_t chunk;            /* tokens per chunk, >= 1                                         */
    int32_t io_dtype;         /* ttt_dtype of q, k, v, o.  Fast weights are always fp32.        */
    int32_t mask;             /* ttt_mask_mode, not TOKEN_CAUSAL                                */
    int32_t rule;             /* ttt_update_rule                                                */
    int32_t ns_iters;         /* Newton-Schulz steps for the Muon rules, 0..32                  */
    float momentum;           /* beta of the chunk momentum; 0 = none                           */
    int32_t last_layer_only;  /* 1: only W2 is updated (paper Sec. 6.1 Step 1)                  */
    int32_t w0_per_batch;     /* 0: W0 is [H][3*d_h*m_h]; 1: W0 is [B][H][3*d_h*m_h]            */
    const uint8_t* update_chunks; /* host, ceil(N/chunk) flags; read only for TTT_MASK_STRIDED  */
    int32_t inner_steps;      /* gradient steps per updating chunk, 0..64 (0 means 1), each from
                                 the gradient at the current W ("TTT with KV Binding Is Secretly
                                 Linear Attention", Sec. 4.1)                                   */
    int32_t ascent;           /* 1: gradient ascent, W moves along +g instead of -g (same paper,
                                 Sec. 4.2); 0: descent                                          */
    int32_t parallel_form;    /* 1: compute the layer in its parallel static-kernel form.  Needs
                                 last_layer_only = 1 and rule TTT_UPD_GD or TTT_UPD_MUON (no
                                 weight norm): W1 and W3 are then frozen, phi(x) = SiLU(W1 x) *
                                 (W3 x) is fixed, and a chunk's W2 gradient -sum eta v phi(k)^T
                                 does not depend on W2, so W2 follows a prefix over chunks ("TTT
                                 with KV Binding Is Secretly Linear Attention", Thm. 5.2-5.3,
                                 Sec. 6.1-6.2, Table 2).  TTT_UPD_GD: chunked linear attention
                                 with queries phi(q), keys phi(k), values v, state W2 (momentum,
                                 inner_steps and ascent included).  TTT_UPD_MUON (Table 2's Variant
                                 2): the chunk momentum as a scan over chunks, Newton-Schulz on
                                 every chunk's momentum at once, W2 minus their prefix sum; one
                                 gradient step per chunk (inner_steps > 1: UNSUPPORTED).  Same
                                 results as 0 (the chunk recurrence) up to rounding.  Other rules:
                                 INVALID_ARGUMENT */
    int32_t chunk_rates;      /* 1: per-chunk rates outside the optimizer step ("TTT with KV
                                 Binding Is Secretly Linear Attention", App. E.1 written per chunk
                                 as in App. H.1-H.2; App. E.3 with Muon).  eta is then
                                 [B][H][ceil(N/chunk)] fp32, one rate eta_j per chunk; the chunk
                                 gradient g_j weighs every token by 1; the momentum step is
                                 dW <- g_j + alpha_j dW with alpha_j from chunk_momentum (NULL:
                                 dW = g_j); the update is W <- [L2-Normalize](W - eta_j Opt(dW)),
                                 Opt = Muon for the Muon rules, the identity otherwise.  momentum
                                 must be 0 and parallel_form 0.  0: eta is per token, inside the
                                 gradient sum (the notes' Eq. (2)).                             */
    const float* chunk_momentum; /* device, [B][H][ceil(N/chunk)] fp32 alpha_j, 4-byte aligned;
                                 NULL (no momentum) or used with chunk_rates = 1 only             */
} ttt_desc;

typedef struct linattn_desc {
    int32_t B, H, N;
    int32_t d_k, d_v;         /* multiples of 32; d_v <= 4096; d_k <= 2048 on the chunk-parallel
                                 path, <= 256 on the sequential one (TTT_ERR_UNSUPPORTED beyond) */
    int32_t chunk;            /* tokens per chunk, >= 1 (ignored by TOKEN_CAUSAL)               */
    int32_t io_dtype;         /* ttt_dtype of q, k, v, o; the state S is fp32                   */
    int32_t mask;             /* any ttt_mask_mode                                              */
    const uint8_t* update_chunks; /* host, ceil(N/chunk) flags; read only for TTT_MASK_STRIDED  */
} linattn_desc;

/* Version of this ABI (the TTT_ABI_VERSION the library was compiled with). */
int32_t ttt_abi_version(void);

/* Static description of a status code; never NULL. */
const char* ttt_status_string(ttt_status s);

/* Message for the latest failed call on this thread ("" if none). */
const char* ttt_last_error(void);

/* Device workspace that ttt_forward needs for `desc`, in bytes (written to *bytes). */
ttt_status ttt_workspace_bytes(const ttt_desc* desc, size_t* bytes);

/*
 * The TTT-KVB layer (notes Eqs. (2)-(6), (10); paper App. E).
 *   q, k, v   [B][H][N][d_h] of io_dtype, 16-byte aligned
 *   eta       [B][H][N] fp32 per-token learning rates (any sign; negative = gradient ascent), or
 *             with chunk_rates [B][H][ceil(N/chunk)] per-chunk rates
 *   W0        initial fast weights, fp32, [H] or [B][H] blocks of [W1 | W3 | W2], 16-byte aligned
 *   o         [B][H][N][d_h] of io_dtype, output
 *   W_out     nullable; [B][H][3*d_h*m_h] fp32 fast weights after the last chunk
 *   M_inout   nullable; [B][H][3*d_h*m_h] fp32 momentum, read at the start and written at the
 *             end (NULL: momentum starts at zero and is dropped).  Used only if momentum != 0.
 *   workspace device buffer of at least ttt_workspace_bytes(desc) bytes, 256-byte aligned
 */
ttt_status ttt_forward(const ttt_desc* desc, const void* q, const void* k, const void* v,
                       const float* eta, const float* W0, void* o, float* W_out, float* M_inout,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * ttt_forward for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, layout, checks and results as
 * ttt_forward (the same kernels run), except that there is no workspace argument: the workspace is
 * a static array of TTT_NOALLOC_SCRATCH_BYTES bytes in the library's device code, one per device,
 * which stays allocated on every device the library runs on until the process ends.  The call
 * itself allocates nothing (no hipMalloc, no events: the launch profiler is off for its launches).
 *   - A call whose ttt_workspace_bytes() exceeds TTT_NOALLOC_SCRATCH_BYTES returns
 *     TTT_ERR_WORKSPACE with a message, before anything is enqueued.
 *   - All calls on one device share that device's array, and nothing in it carries over from one
 *     call to the next.  Calls that overlap on one device (concurrent streams, or a second call
 *     enqueued from another thread before the first has finished on the device) race on the array:
 *     the caller must order them, for example by using one stream per device.
 *   - The first call on a device looks the array's address up (hipGetSymbolAddress); it may fail
 *     with TTT_ERR_DEVICE if the device is unusable.
 */
#define TTT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ttt_status ttt_forward_noalloc(const ttt_desc* desc, const void* q, const void* k, const void* v,
                               const float* eta, const float* W0, void* o, float* W_out, float* M_inout,
                               void* stream);

/*
 * Device workspace that ttt_backward needs, in bytes (the size with dW0 requested, which covers a
 * call without it).  last_layer_only = 1: the io-dtype copies of W1 | W3 and their transposes,
 * phi(q), phi(k), and the factors of phi's backward for both sides, later dA | dC (12 m_h bytes per
 * token and scan in bf16, twice in fp32), the scans' dW2, the partial sums of dW1 | dW3, and the
 * linear-attention backward's workspace over d_k = m_h, d_v = d_h
 * (linattn_backward_workspace_bytes); with TTT_UPD_GD_L2 also W2 after every step of every chunk in
 * fp32, and its row norms.  last_layer_only = 0: the forward's own workspace (ttt_workspace_bytes
 * without Muon), the weights before every update and after the last (fp32, 12 d_h m_h bytes per
 * scan and update), with the norm every update's row norms, the running weight and momentum
 * gradients, the contraction operands of one update, and per-chunk intermediates (about
 * 14 m_h io-dtype elements per token of one chunk and scan, plus 12 m_h fp32 scratch bytes in fp32,
 * and 3 m_h elements per token of the longest run of chunks that read one set of weights); Muon
 * adds each update's U (12 d_h m_h bytes per scan and update) and one update's fp32 Newton-Schulz
 * iterates and Gram matrices.
 */
ttt_status ttt_backward_workspace_bytes(const ttt_desc* desc, size_t* bytes);

/*
 * Backward of ttt_forward for any rule with chunk_rates 0 (else TTT_ERR_UNSUPPORTED); inner_steps,
 * ascent, momentum, ns_iters, the chunked masks and w0_per_batch are as for the forward.  A
 * recurrence of more than 65536 updates (chunks x inner steps) is TTT_ERR_UNSUPPORTED.
 *
 * last_layer_only = 0 (all three weights learning, parallel_form 0), or a Muon rule: the reverse of
 * the chunk recurrence (notes Eqs. (2)-(6), section 1.1): the forward runs again and records the
 * weights before every update (and, with Muon, each update's U); then, from the last update back,
 * the gradient of an update's output weights goes through the row norm's transpose, the step
 * W - U or W - Muon(U) (Newton-Schulz walked back from its iterates, ns_iters as in the forward),
 * the momentum (M <- momentum M + g, which starts from zero) and the chunk gradient
 * g = grad_W sum eta L(f_W(k), v), whose own derivative in W, k, v and eta (SiLU'' included)
 * carries it on; the queries that read a set of weights add the gradient of their outputs.  With
 * last_layer_only (Muon) W1 and W3 stay frozen.
 *
 * last_layer_only = 1 with TTT_UPD_GD or TTT_UPD_GD_L2 (the layer whose inner loop trains W2
 * alone; parallel_form is ignored, both forms compute the same layer).  With W1 and W3
 * frozen, phi(x) = SiLU(W1 x) * (W3 x) is fixed and W2 is the state of chunked linear attention with
 * queries phi(q), keys phi(k) and values v: each of an updating chunk's max(inner_steps, 1) steps
 * adds u = (ascent ? -1 : 1) * sum eta v phi(k)^T to W2, directly or, with momentum, through
 * M <- momentum M - u, W2 <- W2 - M, and TTT_UPD_GD_L2 then L2-normalizes W2's rows (notes Eq. (5);
 * Variant 1 of "TTT with KV Binding Is Secretly Linear Attention", Sec. 6.1, without Muon)
 * (the same paper, Thm. 5.2-5.3, Sec. 6.1-6.2 and Fig. 4: the outer-loop gradients of training
 * through the parallel form).  The momentum is the one a forward call with M_inout = NULL keeps: it
 * starts from zero and its final state is not part of the loss.
 * The gradients are those of
 *     L = sum over tokens of dO . o + <dW_out, W_out>
 * (W_out as ttt_forward writes it: W1 and W3 as given, W2 after the last chunk), for every input:
 *   q, k, v, eta, W0   the forward's inputs, as for ttt_forward
 *   dO        [B][H][N][d_h] of io_dtype, 16-byte aligned: the gradient of o
 *   dW_out    nullable; [B][H][3*d_h*m_h] fp32, 16-byte aligned: the gradient of W_out (NULL = 0)
 *   dq, dk, dv [B][H][N][d_h] of io_dtype, 16-byte aligned; deta [B][H][N] fp32, 4-byte aligned
 *   dW0       nullable; fp32 with W0's shape ([H] or [B][H] blocks of [dW1 | dW3 | dW2]), 16-byte
 *             aligned; per-head weights sum their scans' gradients over the batch.  NULL: not
 *             computed (the weight-gradient contraction is skipped)
 *   workspace device buffer of at least ttt_backward_workspace_bytes(desc) bytes, 256-byte aligned
 *             (may be NULL when that is 0); TTT_ERR_WORKSPACE if it is too small
 * No output may overlap an input or another output (TTT_ERR_INVALID_ARGUMENT).  Products run in the
 * io dtype with fp32 accumulation (bf16: phi, dA | dC, W1 | W3 and the linear-attention states and
 * state gradients are rounded to bf16 as contraction operands; the states are summed in fp32; with
 * all weights learning the weights and their gradients are carried in fp32 and rounded to bf16 as
 * operands, and so are the per-token intermediates; Muon's walk back carries the gradient in fp32
 * with io-dtype operands), and every sum is
 * taken in a fixed order, so results do not depend on scheduling.
 */
ttt_status ttt_backward(const ttt_desc* desc, const void* q, const void* k, const void* v,
                        const float* eta, const float* W0, const void* dO, const float* dW_out,
                        void* dq, void* dk, void* dv, float* deta, float* dW0,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The training pair for the backward of the recurrence (any rule, chunk_rates 0, at most 65536
 * updates; the layer whose inner loop trains W2 alone by GD included, which ttt_backward takes
 * through linear attention instead, as its parallel form computes it).  A training step
 * runs ttt_forward_record, which writes o and W_out as ttt_forward does (momentum from zero, its
 * final value not returned) and keeps a record of the recurrence: the weights before every update
 * and after the last (fp32), with the L2 rules every update's row norms, with Muon every update's
 * Newton-Schulz input; then ttt_backward_record, which reads the record instead of running the
 * forward again.  Results are those of ttt_backward, bit for bit.  The record is opaque device
 * memory; its content is valid for the descriptor and inputs of the forward that wrote it.
 *
 * ttt_record_bytes: the record's size and the workspace ttt_forward_record needs.  Descriptors
 * outside the pair's scope are TTT_ERR_UNSUPPORTED.  With last_layer_only and TTT_UPD_GD or
 * TTT_UPD_GD_L2 the pair's results equal ttt_backward's within rounding (not bit for bit: the two
 * take different routes).
 */
ttt_status ttt_record_bytes(const ttt_desc* desc, size_t* record_bytes, size_t* workspace_bytes);

/*
 * The forward with a record.  Arguments as for ttt_forward (no momentum state: it starts from zero),
 * plus record (device, 256-byte aligned, at least record_bytes from ttt_record_bytes;
 * TTT_ERR_WORKSPACE if record_bytes is smaller).  No output, the record or the workspace may
 * overlap an input or each other.
 */
ttt_status ttt_forward_record(const ttt_desc* desc, const void* q, const void* k, const void* v,
                              const float* eta, const float* W0, void* o, float* W_out, void* record,
                              size_t record_bytes, void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace that ttt_backward_record needs, in bytes (ttt_backward's without the record and
 * the forward's own workspace). */
ttt_status ttt_backward_record_workspace_bytes(const ttt_desc* desc, size_t* bytes);

/*
 * ttt_backward from a record that ttt_forward_record wrote with the same descriptor and inputs: q,
 * k, v, eta, dO, dW_out and the outputs as for ttt_backward; W0 is not read (the record holds it).
 */
ttt_status ttt_backward_record(const ttt_desc* desc, const void* q, const void* k, const void* v,
                               const float* eta, const void* record, size_t record_bytes, const void* dO,
                               const float* dW_out, void* dq, void* dk, void* dv, float* deta, float* dW0,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device workspace that linattn_forward needs, in bytes.  Zero when the call runs the sequential
 * kernel (chunks so small that 4 d_k d_v > 2 chunk (d_k + d_v), or token-causal mode with N < 256);
 * otherwise room for every chunk's own update (fp32) and the state each chunk's queries see (io
 * dtype), 6 bytes per state element per chunk and scan in bf16, 8 in fp32 (the chunk-parallel path;
 * token-causal mode counts chunks of 128 tokens).
 */
ttt_status linattn_workspace_bytes(const linattn_desc* desc, size_t* bytes);

/*
 * Chunked linear attention, the linear bias-free fast weight under plain GD with the dot-product
 * loss (paper Thm. 5.2, Sec. 6.1 Step 6; "From Linear Attention to Test-Time Training",
 * causal linear attention).  Per (batch, head): S is d_v x d_k fp32; a chunk's update is
 * S <- S + sum_i eta_i v_i k_i^T and its apply is o_i = S q_i, ordered by `mask`.
 *   q, k      [B][H][N][d_k] of io_dtype; v, o [B][H][N][d_v]; eta [B][H][N] fp32
 *   S0        nullable; [B][H][d_v][d_k] fp32 initial state (NULL = zeros)
 *   S_out     nullable; [B][H][d_v][d_k] fp32 state after the last chunk
 *   workspace device buffer of at least linattn_workspace_bytes(desc) bytes, 256-byte aligned
 *             (may be NULL when that is 0); TTT_ERR_WORKSPACE if it is too small
 * The state is carried in fp32.  Products run in the io dtype with fp32 accumulation: the
 * chunk-parallel path hands each chunk's state to the apply rounded once to the io dtype, the
 * sequential kernel keeps a bf16 hi + lo copy of it (about 16 bits).
 */
ttt_status linattn_forward(const linattn_desc* desc, const void* q, const void* k, const void* v,
                           const float* eta, const float* S0, void* o, float* S_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device workspace that linattn_backward needs, in bytes: the update (fp32), the state and the
 * state gradient (io dtype) of every chunk and scan (8 bytes per state element per chunk in bf16,
 * 12 in fp32), plus B*H*N*4 bytes per 128 columns of d_k when d_k > 128; zero when N is 0.
 */
ttt_status linattn_backward_workspace_bytes(const linattn_desc* desc, size_t* bytes);

/*
 * Backward of linattn_forward under the chunked masks (FULL, UPDATE_THEN_APPLY, APPLY_THEN_UPDATE,
 * STRIDED): the gradients that training through the parallel form needs (paper Sec. 6.2, Fig. 4),
 * for the loss L = sum over tokens of dO . o + <dS_out, S_out>.  With S_c the state chunk c's queries
 * see and R_j the sum of dS_out and of sum_{t in c} dO_t q_t^T over the chunks c whose S_c holds
 * chunk j's update:  dq_t = S_c^T dO_t,  dv_s = eta_s R_j k_s,  dk_s = eta_s R_j^T v_s,
 * deta_s = v_s . (R_j k_s),  dS0 = dS_out + sum over all chunks of sum_t dO_t q_t^T.  Chunks a
 * strided mask does not update get zero dk, dv and deta.  TOKEN_CAUSAL is TTT_ERR_UNSUPPORTED.
 *   q, k, v, eta, S0  as for linattn_forward (the forward's inputs; S0 nullable = zeros)
 *   dO        [B][H][N][d_v] of io_dtype: the gradient of o
 *   dS_out    nullable; [B][H][d_v][d_k] fp32 gradient of S_out (NULL = zeros)
 *   dq, dk    [B][H][N][d_k] of io_dtype; dv [B][H][N][d_v] of io_dtype; deta [B][H][N] fp32
 *   dS0       nullable; [B][H][d_v][d_k] fp32 gradient of S0 (not written if NULL)
 *   workspace device buffer of at least linattn_backward_workspace_bytes(desc) bytes, 256-byte
 *             aligned (may be NULL when that is 0); TTT_ERR_WORKSPACE if it is too small
 * Pointer alignment: q, k, v, dO, dq, dk, dv 16 bytes; the fp32 buffers 4 bytes.  No output may
 * overlap an input or another output (TTT_ERR_INVALID_ARGUMENT).  Products run in the io dtype
 * with fp32 accumulation; the chunk states and state gradients are summed in fp32 and enter the
 * products rounded once to the io dtype, as in the forward.
 */
ttt_status linattn_backward(const linattn_desc* desc, const void* q, const void* k, const void* v,
                            const float* eta, const float* S0, const void* dO, const float* dS_out,
                            void* dq, void* dk, void* dv, float* deta, float* dS0,
                            void* workspace, size_t workspace_bytes, void* stream);


/*
 * LaCT's sliding-window attention, the local branch beside the TTT layer (PaperTrace "5.2.1 LaCT and
 * TTT-E2E", section 1.1, the window-attention paragraphs, and the remark after Eq. (10)): causal
 * softmax attention over a window as wide as the chunk, on the same q, k, v as the fast-weight
 * branch, with a per-channel scale and shift on q and k.  Per (batch, head), token t attends to the
 * tokens s with t - window < s <= t:
 *     o_t = sum_s softmax_s(q'_t . k'_s / sqrt(d)) v_s,  q' = q * q_scale + q_shift,
 *                                                        k' = k * k_scale + k_shift (per channel).
 *   q, k, v, o  [B][H][N][d] of io_dtype, 16-byte aligned; d a multiple of 32, at most 384
 *   q_scale, q_shift, k_scale, k_shift   [H][d] fp32 per-head, per-channel parameters, 16-byte
 *               aligned; NULL means scale 1 or shift 0.  k_shift adds the same amount to every score
 *               of a query, which softmax removes: it does not change o and is not read.
 *   workspace   device buffer of at least swa_workspace_bytes(desc) bytes, 256-byte aligned, not
 *               overlapping q, k, v or o: for bf16 heads whose d is a multiple of 64 other than 320
 *               it holds v rearranged in blocks of 32 keys, otherwise q * q_scale + q_shift, times
 *               k_scale
 * Scores, the softmax and the output accumulation are fp32; in bf16 mode the softmax weights are
 * rounded to bf16 before they multiply v.
 */
typedef struct swa_desc {
    int32_t B, H, N, d;
    int32_t window;           /* >= 1 tokens, the query included                                 */
    int32_t io_dtype;         /* ttt_dtype of q, k, v, o                                        */
} swa_desc;

ttt_status swa_workspace_bytes(const swa_desc* desc, size_t* bytes);
ttt_status swa_forward(const swa_desc* desc, const void* q, const void* k, const void* v,
                       const float* q_scale, const float* q_shift, const float* k_scale,
                       const float* k_shift, void* o, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Optional per-kernel timing for measurement tools (not needed for normal use).  While enabled,
 * every kernel launch this library makes is bracketed by two HIP events recorded on the stream
 * it is launched on.  ttt_profile_read waits for the recorded events, writes for each kernel
 * class i < n the summed milliseconds ms[i] and the launch count count[i] since the previous
 * read, and forgets them.  Kernel classes are numbered 0 .. TTT_PROF_KERNELS-1 and named by
 * ttt_profile_kernel_name.  Enabling or reading while another thread launches is allowed.
 */
#define TTT_PROF_KERNELS 32
ttt_status ttt_profile_enable(int32_t on);
/* Restricts the bracketing to the kernel classes i whose bit (1u << i) is set in mask; the
 * default is every class.  Each bracket records two events on the launch's stream, which costs
 * the stream a few microseconds, so a tool that times one kernel class selects only that one. */
ttt_status ttt_profile_select(uint32_t mask);
ttt_status ttt_profile_read(float* ms, int32_t* count, int32_t n);
const char* ttt_profile_kernel_name(int32_t i);

/*
 * MFMA-loop probe for measurement tools: enqueues on `stream` one kernel of `blocks` workgroups of
 * 256 threads in which every wave issues iters x 4 independent bf16 32x32x16 MFMAs on register
 * operands (32768 FLOP each), and writes one float per workgroup to the device buffer out
 * (caller-owned, blocks floats).  Timing it gives the matrix-core rate the device sustains:
 * FLOP = blocks x 4 waves x iters x 4 x 32768.  blocks, iters >= 1 and out non-NULL, else
 * TTT_ERR_INVALID_ARGUMENT before anything is enqueued.
 */
ttt_status ttt_probe_mfma_bf16(int32_t blocks, int32_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TTT_MI355X_H */
