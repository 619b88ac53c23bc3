"""GPU parity of ttt_forward (through the C ABI) against the fp64 oracle.

Tolerances: relative L2 over the compared tensor <= 1e-5 with fp32 inputs and <= 2e-2 with bf16
inputs (fp32 fast weights in both), for the outputs o and the final fast weights W_out.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import linear_attention_chunk_amd as T
from gpu_util import assert_close, bulk_ttt_inputs, dev, full_ttt_inputs, host, rel, say

pytestmark = pytest.mark.gpu

TOL = {False: 1e-5, True: 2e-2}


def split_w(Wout, d, m):
    W = host(Wout) if not isinstance(Wout, np.ndarray) else Wout
    dm = d * m
    return W[..., :dm].reshape(*W.shape[:-1], m, d), W[..., dm:2 * dm].reshape(*W.shape[:-1], m, d), \
        W[..., 2 * dm:].reshape(*W.shape[:-1], d, m)


def check(o_gpu, W_gpu, o_ref, W_ref, d, m, tol, chunk=None, label=""):
    """o against the oracle over the whole tensor, per (batch, head), per chunk and per token row;
    each of W1, W3, W2 per (batch, head) and per row (W_gpu None: o only)."""
    say(f"  {label}")
    assert_close(host(o_gpu), o_ref, tol, "o", chunk)
    if W_gpu is not None:
        for name, a, b in zip(("W1", "W3", "W2"), split_w(W_gpu, d, m), W_ref):
            assert_close(a, b, tol, name)


def run_small(seed, B, H, N, d, m, chunk, mask, rule, bf16, momentum=0.0, last=False, flags=None, ns=5, inner=1,
              ascent=False, parallel=False, want_W=True):
    say(f"ttt case B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} rule{rule} mom{momentum} last{last} bf16={bf16}"
        f" inner{inner} ascent{ascent} parallel{parallel} want_W{want_W}")
    (q, k, v, eta, W0), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(seed, B, H, N, d, m, bf16)
    o, Wout = T.ttt_forward(q, k, v, eta, W0, chunk, mask, rule, m_h=m, ns_iters=ns, momentum=momentum,
                            last_layer_only=last, update_chunks=flags, inner_steps=inner, ascent=ascent,
                            parallel_form=parallel, want_W=want_W)
    torch.cuda.synchronize()
    assert (Wout is not None) == want_W
    o_ref, W_ref, _ = O.ttt_forward_ref(hq, hk, hv, he, W1, W3, W2, chunk, mask, rule, ns, momentum, last, flags,
                                        inner_steps=inner, ascent=ascent)
    check(o, Wout, o_ref, W_ref, d, m, TOL[bf16], chunk, label="all slices")


def test_config1_tiny_fp32():
    """B1 H1 N256 b64 d32 m32, fp32, apply-then-update, L2-Normalize(W - g), seed 0."""
    run_small(0, 1, 1, 256, 32, 32, 64, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, False)


CASES = [
    # mask, rule, momentum, last_layer_only
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, 0.0, False),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, 0.0, False),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, 0.9, False),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_GD_L2, 0.0, False),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, 0.5, True),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, 0.9, True),
    # Variant 1 of the paper's ablation (Sec. 6.1 Step 1, Table 2): only the last layer learns, the
    # weight norm, momentum and Muon stay; W1 and W3 stay frozen while W2 is normalised
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, 0.0, True),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, 0.9, True),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,rule,mom,last", CASES)
def test_modes_ragged(mask, rule, mom, last, bf16):
    # 3 full chunks of 96 and a tail of 20; m = 160 leaves partial MFMA tiles in every kernel
    run_small(3, 1, 2, 308, 64, 160, 96, mask, rule, bf16, mom, last)


@pytest.mark.parametrize("bf16", [False, True])
def test_full_mask_and_strided(bf16):
    run_small(4, 2, 1, 200, 32, 96, 200, O.MASK_FULL, O.UPD_GD_L2, bf16)
    run_small(5, 1, 2, 256, 64, 64, 64, O.MASK_STRIDED, O.UPD_MUON_L2, bf16, flags=[1, 0, 1, 0])


@pytest.mark.parametrize("bf16", [False, True])
def test_multi_tile_ragged(bf16):
    # two full chunks of 512 and a tail of 276: several full up/down tiles in every direction
    # (d = 128, m = 384) next to partial ones, for both apply orders
    run_small(9, 1, 2, 1300, 128, 384, 512, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16)
    run_small(10, 1, 1, 1300, 128, 384, 512, O.MASK_UPDATE_THEN_APPLY, O.UPD_GD, bf16)


def test_wide_layer_bf16():
    # d = 512, m = 1024: more hidden tiles per scan than the LaCT LM shape
    run_small(11, 1, 1, 600, 512, 1024, 256, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, True)


@pytest.mark.parametrize("bf16", [False, True])
def test_maximum_widths(bf16):
    # m_h and d_h at their maximum (2048) against a narrow other side: 16 hidden tiles per scan
    # with one partial d tile, update rows of 2048 (8 float4 per lane, 64-128 KB of LDS for W2^T),
    # and the other way round, 32 64-wide k-steps per up tile and 16 row blocks of W2
    run_small(22, 1, 1, 160, 64, 2048, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16)
    run_small(23, 1, 1, 160, 2048, 64, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, bf16, ns=2)


def test_tall_and_wide_muon_fp32():
    # d > m exercises the other Gram side for W1/W3 and W2
    run_small(6, 1, 1, 128, 96, 32, 64, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, False, ns=3)


def test_muon_gram_mirror_fp32():
    # p = min(d, m) = 160 spans three 64-wide Gram tiles, the last partial: the off-diagonal tiles
    # also write their mirror blocks; both Gram sides (m > d, then d > m)
    run_small(12, 1, 1, 256, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, False, ns=3)
    run_small(13, 1, 1, 256, 320, 160, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, False, ns=2)
    # 32 scans in one launch (each XCD takes a contiguous range of the blocks)
    run_small(21, 8, 4, 128, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, False, ns=2)


def test_newton_schulz_tiles_bf16():
    # d = 160, m = 320: W1/W3 take the tall step (320 x 160) and W2 the wide one (160 x 320), each
    # with full 128 x 64 step tiles beside ragged ones; the iterate is the bf16 hi + lo pair
    run_small(24, 1, 1, 256, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, True, ns=3)
    run_small(25, 1, 2, 300, 160, 320, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, True, momentum=0.9, ns=5)


@pytest.mark.parametrize("bf16", [False, True])
def test_newton_schulz_full_step_tiles(bf16):
    # d and m multiples of 128: every step tile lies inside its matrix, and the step runs its
    # full-tile workgroups (one LDS stage, the iterate read in the epilogue); both orientations
    run_small(40, 1, 2, 300, 128, 256, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, bf16, momentum=0.9, ns=5)
    run_small(41, 2, 1, 256, 256, 128, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, bf16, ns=3)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("ns", [0, 1])
def test_newton_schulz_step_counts(ns, bf16):
    # no step (only the Frobenius scaling), and one step, which is both the first (it applies the
    # scaling) and the last (it writes the fp32 result)
    run_small(26 + ns, 1, 1, 256, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, bf16, momentum=0.9,
              ns=ns)


@pytest.mark.parametrize("bf16", [False, True])
def test_inner_steps_and_ascent(bf16):
    # several gradient steps per updating chunk, and gradient ascent, against the oracle; N = 300
    # leaves a ragged last chunk
    run_small(14, 1, 2, 300, 64, 128, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16, inner=3)
    run_small(15, 1, 1, 300, 64, 128, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, bf16, momentum=0.9, inner=2,
              ascent=True, ns=3)
    run_small(16, 1, 1, 256, 64, 64, 64, O.MASK_STRIDED, O.UPD_GD, bf16, last=True, flags=[1, 0, 1, 1],
              ascent=True, inner=2)


@pytest.mark.parametrize("bf16", [False, True])
def test_outputs_only_without_w_out(bf16):
    # W_out NULL: the last update writes no final weights (and, under apply-then-update, no shadows)
    run_small(37, 1, 2, 308, 64, 160, 96, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16, want_W=False)
    run_small(38, 2, 1, 200, 64, 96, 64, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, bf16, momentum=0.9, want_W=False)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,rule,mom", [(O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, 0.9),
                                           (O.MASK_UPDATE_THEN_APPLY, O.UPD_GD_L2, 0.0)])
def test_per_batch_w0_and_carried_momentum(mask, rule, mom, bf16):
    """W0 given per (batch, head) with B = 2, and a non-zero starting momentum M that the call reads
    and writes back, against the oracle started from the same per-slice W0 and M."""
    B, H, N, d, m, chunk = 2, 2, 300, 64, 160, 128
    say(f"per-batch W0 B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} rule{rule} mom{mom} bf16={bf16}")
    (q, k, v, eta, _), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(39, B, H, N, d, m, bf16)
    scale = np.array([[1.0 + 0.15 * (2 * b + h) for h in range(H)] for b in range(B)])[:, :, None, None]
    Wb = [W[None] * scale for W in (W1, W3, W2)]
    W0 = dev(np.concatenate([x.reshape(B, H, -1) for x in Wb], axis=-1))
    rng = np.random.default_rng(40)
    Mh = [0.01 * rng.standard_normal(x.shape) for x in Wb]
    M = dev(np.concatenate([x.reshape(B, H, -1) for x in Mh], axis=-1))
    o, Wout = T.ttt_forward(q, k, v, eta, W0, chunk, mask, rule, m_h=m, momentum=mom, M=M)
    torch.cuda.synchronize()
    o_ref, W_ref, M_ref = O.ttt_forward_ref(hq, hk, hv, he, *Wb, chunk, mask, rule, 5, mom, M=tuple(Mh))
    tol = TOL[bf16]
    check(o, Wout, o_ref, W_ref, d, m, tol, chunk, label="per-(batch, head) W0")
    if mom:
        for name, a, b in zip(("M1", "M3", "M2"), split_w(M, d, m), M_ref):
            assert_close(a, b, tol, name)


def test_nan_in_v_reaches_exactly_the_outputs_that_depend_on_it():
    """A NaN in one value entry, token t of chunk j of one scan, enters that chunk's gradient: every
    output of the scan's later chunks and its final weights become NaN, while its chunks up to j
    (apply before update) and every other scan give exactly what they give without the NaN."""
    B, H, N, d, m, chunk = 2, 2, 320, 64, 128, 64
    (q, k, v, eta, W0), _ = full_ttt_inputs(41, B, H, N, d, m, True)
    kw = dict(m_h=m, momentum=0.9)
    for rule in (O.UPD_GD_L2, O.UPD_MUON_L2):
        o_ref, W_ref = T.ttt_forward(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, rule, **kw)
        vn = v.clone()
        b, h, t, e = 1, 0, 150, 7           # token 150 lies in chunk 2 (tokens 128 .. 191)
        vn[b, h, t, e] = float("nan")
        o_n, W_n = T.ttt_forward(q, k, vn, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, rule, **kw)
        torch.cuda.synchronize()
        say(f"  rule {rule}: NaN at v[{b},{h},{t},{e}]")
        j_end = (t // chunk + 1) * chunk
        assert torch.equal(o_n[b, h, :j_end], o_ref[b, h, :j_end])
        assert torch.isnan(o_n[b, h, j_end:].float()).all()
        assert torch.isnan(W_n[b, h]).all()
        for bb in range(B):
            for hh in range(H):
                if (bb, hh) != (b, h):
                    assert torch.equal(o_n[bb, hh], o_ref[bb, hh]) and torch.equal(W_n[bb, hh], W_ref[bb, hh])


def test_host_and_short_buffers_are_refused_before_enqueueing():
    """Pointers that are not device memory, and device buffers too short for the call, are refused
    with TTT_ERR_INVALID_ARGUMENT before anything runs (the library checks each allocation's
    extent); the Python binding refuses the same mistakes with ValueError."""
    import ctypes
    from linear_attention_chunk_amd import _lib as C
    B, H, N, d, m, chunk = 1, 2, 128, 64, 96, 64
    (q, k, v, eta, W0), _ = full_ttt_inputs(42, B, H, N, d, m, True)
    D, keep = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    nws = T.ttt_workspace_bytes(D)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    nbytes = q.numel() * 2
    short = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(short), nbytes - 256) == 0   # exact-size allocation, 256 B short
    host_buf = (ctypes.c_uint8 * nbytes)()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    L = C.lib()
    try:
        o = torch.empty_like(q)
        def call(o_ptr, q_ptr=None):
            return L.ttt_forward(ctypes.byref(D), q_ptr or P(q), P(k), P(v), P(eta), P(W0), o_ptr, None, None, P(ws),
                                 nws, None)
        o.fill_(0.5)
        sentinel = o.clone()
        assert call(ctypes.cast(host_buf, ctypes.c_void_p)) == C.TTT_ERR_INVALID_ARGUMENT
        assert b"not in device memory" in L.ttt_last_error()
        assert call(short) == C.TTT_ERR_INVALID_ARGUMENT
        assert b"allocation holds" in L.ttt_last_error()
        assert call(P(o), ctypes.cast(host_buf, ctypes.c_void_p)) == C.TTT_ERR_INVALID_ARGUMENT
        assert torch.equal(o, sentinel)      # nothing was written by the refused calls
        assert call(P(o)) == C.TTT_OK
        torch.cuda.synchronize()
    finally:
        hip.hipFree(short)
    del keep
    with pytest.raises(ValueError, match="device tensor"):
        T.ttt_forward(q, k, v, eta, W0, chunk, m_h=m, out=torch.empty(q.shape, dtype=q.dtype))
    with pytest.raises(ValueError, match="workspace"):
        T.ttt_forward(q, k, v, eta, W0, chunk, m_h=m, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError, match="M has shape"):
        T.ttt_forward(q, k, v, eta, W0, chunk, m_h=m, momentum=0.9,
                      M=torch.zeros((B, H, 3 * d * m - 4), device="cuda"))


CHUNK_RATE_CASES = [
    # mask, rule, per-chunk momentum, last layer only
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, True, False),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, True, False),
    (O.MASK_STRIDED, O.UPD_MUON, True, True),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, False, False),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,rule,with_alpha,last", CHUNK_RATE_CASES)
def test_chunk_rates(mask, rule, with_alpha, last, bf16):
    """Per-chunk rates eta_j outside the optimizer step and per-chunk momentum factors alpha_j (the
    paper's App. E.1 in App. H's chunk form; E.3 with Muon) against the oracle; N = 308 leaves a
    ragged chunk, one alpha_j is 0 (the momentum restarts there)."""
    B, H, N, d, m, chunk = 1, 2, 308, 64, 160, 96
    nc = -(-N // chunk)
    say(f"chunk rates B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} rule{rule} alpha{with_alpha} last{last} bf16={bf16}")
    (q, k, v, _, W0), (hq, hk, hv, _, W1, W3, W2) = full_ttt_inputs(70, B, H, N, d, m, bf16)
    rng = np.random.default_rng(71)
    lr = (0.05 + 0.25 * rng.random((B, H, nc))).astype(np.float32)
    alpha = (0.9 * rng.random((B, H, nc))).astype(np.float32) if with_alpha else None
    if alpha is not None:
        alpha[0, 1, 2] = 0.0
    flags = [1, 0, 1, 1] if mask == O.MASK_STRIDED else None
    o, Wout = T.ttt_forward(q, k, v, dev(lr), W0, chunk, mask, rule, m_h=m, last_layer_only=last, update_chunks=flags,
                            chunk_rates=True, chunk_momentum=None if alpha is None else dev(alpha))
    torch.cuda.synchronize()
    o_ref, W_ref, _ = O.ttt_forward_ref(hq, hk, hv, lr, W1, W3, W2, chunk, mask, rule, 5, 0.0, last, flags,
                                        chunk_rates=True, chunk_alpha=alpha)
    check(o, Wout, o_ref, W_ref, d, m, TOL[bf16], chunk, label="per-chunk rates")


def test_ascent_is_descent_with_negated_eta():
    """The pages reduce gradient ascent to a sign flip of the step: the library's ascent must give
    the bits that descent gives with -eta."""
    (q, k, v, eta, W0), _ = full_ttt_inputs(17, 1, 2, 300, 64, 128, True)
    kw = dict(m_h=128, momentum=0.9, ns_iters=3, inner_steps=2)
    oa, Wa = T.ttt_forward(q, k, v, eta, W0, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, ascent=True, **kw)
    od, Wd = T.ttt_forward(q, k, v, (-eta).contiguous(), W0, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(oa, od) and torch.equal(Wa, Wd)


@pytest.mark.parametrize("bf16", [False, True])
def test_few_scans_split_gradients(bf16):
    # one scan with 4096-token chunks: the gradient tiles split the chunk into 8 token parts whose
    # partial gradients are summed; the 904-token tail is not split
    run_small(18, 1, 1, 5000, 64, 128, 4096, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16)
    run_small(19, 1, 1, 5000, 64, 128, 4096, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, bf16, momentum=0.9, ns=3)
    run_small(20, 1, 1, 4096, 64, 128, 4096, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, bf16, last=True)
    # the token parts summed by the momentum / Muon prep: Muon without momentum (fp32 then reads the
    # summed G as its first iterate), zero Newton-Schulz steps, and momentum without Muon
    run_small(34, 1, 1, 5000, 64, 128, 4096, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, bf16, ns=2)
    run_small(35, 1, 1, 4096, 64, 128, 4096, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, bf16, ns=0)
    run_small(36, 1, 1, 5000, 64, 128, 4096, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16, momentum=0.5)


PARALLEL_CASES = [
    # mask, momentum, inner steps, ascent, strided flags
    (O.MASK_APPLY_THEN_UPDATE, 0.0, 1, False, None),
    (O.MASK_APPLY_THEN_UPDATE, 0.9, 1, False, None),
    (O.MASK_UPDATE_THEN_APPLY, 0.5, 2, False, None),
    (O.MASK_STRIDED, 0.0, 1, True, [1, 0, 1, 1]),
    (O.MASK_STRIDED, 0.9, 3, True, [0, 1, 1, 0]),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,mom,inner,ascent,flags", PARALLEL_CASES)
def test_parallel_form_last_layer(mask, mom, inner, ascent, flags, bf16):
    # the parallel static-kernel form (features phi(q), phi(k), then chunked linear attention with
    # W2 as the state) against the oracle's chunk recurrence; N = 308 leaves a ragged last chunk
    # of 20 tokens, and m = 160 partial feature and state tiles
    run_small(30, 1, 2, 308, 64, 160, 96, mask, O.UPD_GD, bf16, mom, last=True, flags=flags, inner=inner,
              ascent=ascent, parallel=True)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,mom,inner,ascent,flags", PARALLEL_CASES)
def test_parallel_form_last_layer_fused_pass(mask, mom, inner, ascent, flags, bf16, monkeypatch):
    # the same through the linear attention's fused update-and-scan pass (which the shape alone
    # would not pick here): W0 as the state per head, the momentum, repeats and sign of the steps
    monkeypatch.setenv("TTT_LIN_PASS", "fused")
    run_small(30, 1, 2, 308, 64, 160, 96, mask, O.UPD_GD, bf16, mom, last=True, flags=flags, inner=inner,
              ascent=ascent, parallel=True)


PARALLEL_MUON_CASES = [
    # mask, momentum, ascent, strided flags, Newton-Schulz steps
    (O.MASK_APPLY_THEN_UPDATE, 0.9, False, None, 5),
    (O.MASK_APPLY_THEN_UPDATE, 0.0, False, None, 5),
    (O.MASK_UPDATE_THEN_APPLY, 0.9, False, None, 3),
    (O.MASK_UPDATE_THEN_APPLY, 0.0, True, None, 5),
    (O.MASK_STRIDED, 0.9, False, [1, 0, 1, 1], 5),
    (O.MASK_STRIDED, 0.0, True, [0, 1, 1, 0], 1),
    (O.MASK_APPLY_THEN_UPDATE, 0.9, False, None, 0),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,mom,ascent,flags,ns", PARALLEL_MUON_CASES)
def test_parallel_form_muon_last_layer(mask, mom, ascent, flags, ns, bf16):
    # Variant 2 (only W2 learns; momentum, per-token eta and Muon kept, no weight norm) in its parallel
    # form -- momentum scanned over chunks, Newton-Schulz on every chunk's momentum at once, W2 as a
    # prefix sum -- against the oracle's chunk recurrence; N = 308 leaves a ragged chunk of 20 tokens
    run_small(60, 1, 2, 308, 64, 160, 96, mask, O.UPD_MUON, bf16, mom, last=True, flags=flags, ns=ns,
              ascent=ascent, parallel=True)


def test_parallel_form_muon_matches_recurrence():
    # several feature tiles, 128-wide state tiles and Newton-Schulz step tiles per chunk: the parallel
    # form with Muon against the library's own chunk recurrence, momentum carried in and out of M
    B, H, N, d, m, chunk = 2, 2, 1100, 128, 384, 256
    say(f"parallel Muon form vs recurrence B{B} H{H} N{N} d{d} m{m} b{chunk}")
    (q, k, v, eta, W0), _ = full_ttt_inputs(61, B, H, N, d, m, True)
    M0 = 0.01 * torch.randn((B, H, 3 * d * m), dtype=torch.float32, device="cuda")
    Mr, Mp = M0.clone(), M0.clone()
    kw = dict(m_h=m, momentum=0.9, last_layer_only=True)
    o_r, W_r = T.ttt_forward(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, M=Mr, **kw)
    o_p, W_p = T.ttt_forward(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, M=Mp,
                             parallel_form=True, **kw)
    torch.cuda.synchronize()
    assert_close(host(o_p), host(o_r), 2e-2, "o (parallel vs recurrence)", chunk)
    dm = d * m
    for name, a, b in zip(("W2", "M2"), (W_p[..., 2 * dm:], Mp[..., 2 * dm:]), (W_r[..., 2 * dm:], Mr[..., 2 * dm:])):
        assert_close(host(a).reshape(B, H, d, m), host(b).reshape(B, H, d, m), 2e-2, name)
    assert torch.equal(W_p[..., :2 * dm], W0[None].expand(B, H, -1)[..., :2 * dm])
    assert torch.equal(Mp[..., :2 * dm], M0[..., :2 * dm])


def test_parallel_form_many_strided_chunks_fp32():
    # 40 chunks of 32 tokens: the strided update flags span two 32-bit words
    flags = [(j * 7) % 3 != 0 for j in range(40)]
    run_small(33, 1, 1, 1280, 64, 96, 32, O.MASK_STRIDED, O.UPD_GD, False, 0.9, last=True, flags=flags,
              parallel=True)


@pytest.mark.parametrize("bf16", [False, True])
def test_parallel_form_full_mask(bf16):
    run_small(31, 2, 1, 200, 32, 96, 200, O.MASK_FULL, O.UPD_GD, bf16, last=True, parallel=True)


@pytest.mark.parametrize("lin_pass", ["fused", "split"])
def test_parallel_form_matches_recurrence(lin_pass, monkeypatch):
    # several 256-token feature tiles and 128-wide state tiles: the parallel form with W0 given per
    # (batch, head) against the chunk recurrence with W0 per head, momentum carried in M (and out of
    # it), through either pass of the linear attention's chunk updates and scan
    monkeypatch.setenv("TTT_LIN_PASS", lin_pass)
    B, H, N, d, m, chunk = 2, 2, 1100, 128, 384, 256
    say(f"parallel form vs recurrence B{B} H{H} N{N} d{d} m{m} b{chunk}")
    (q, k, v, eta, W0), _ = full_ttt_inputs(32, B, H, N, d, m, True)
    M0 = 0.01 * torch.randn((B, H, 3 * d * m), dtype=torch.float32, device="cuda")
    Mr, Mp = M0.clone(), M0.clone()
    kw = dict(m_h=m, momentum=0.9, last_layer_only=True)
    o_r, W_r = T.ttt_forward(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, M=Mr, **kw)
    W0b = W0[None].expand(B, H, -1).contiguous()
    o_p, W_p = T.ttt_forward(q, k, v, eta, W0b, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, M=Mp,
                             parallel_form=True, **kw)
    torch.cuda.synchronize()
    eo, ew, em = rel(host(o_p), host(o_r)), rel(host(W_p), host(W_r)), rel(host(Mp), host(Mr))
    say(f"  rel_o={eo:.3e} rel_W={ew:.3e} rel_M={em:.3e}")
    assert eo <= 2e-2 and ew <= 2e-2 and em <= 2e-2
    # the frozen W1 | W3 blocks of W_out and M come through unchanged
    dm = d * m
    assert torch.equal(W_p[..., :2 * dm], W0b[..., :2 * dm])
    assert torch.equal(Mp[..., :2 * dm], M0[..., :2 * dm])


def test_parallel_form_zero_tokens_returns_w0():
    (q, k, v, eta, W0), _ = full_ttt_inputs(0, 2, 2, 0, 32, 64, True)
    o, Wout = T.ttt_forward(q, k, v, eta, W0, 16, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, m_h=64, last_layer_only=True,
                            parallel_form=True)
    torch.cuda.synchronize()
    assert o.numel() == 0
    Wg = host(Wout)
    ref = host(W0)
    assert np.array_equal(Wg[0], ref) and np.array_equal(Wg[1], ref)


def test_zero_tokens_returns_w0():
    (q, k, v, eta, W0), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(0, 2, 2, 0, 32, 64, True)
    o, Wout = T.ttt_forward(q, k, v, eta, W0, 16, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, m_h=64)
    torch.cuda.synchronize()
    assert o.numel() == 0
    Wg = host(Wout)
    ref = host(W0)
    assert np.array_equal(Wg[0], ref) and np.array_equal(Wg[1], ref)


def test_deterministic_and_chained():
    say("determinism + chaining")
    B, H, N, d, m, chunk = 1, 2, 256, 64, 128, 64
    (q, k, v, eta, W0), _ = full_ttt_inputs(7, B, H, N, d, m, True)
    M = torch.zeros((B, H, 3 * d * m), dtype=torch.float32, device="cuda")
    o1, W1 = T.ttt_forward(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, m_h=m, momentum=0.9,
                           M=M)
    M2 = torch.zeros_like(M)
    o2, W2 = T.ttt_forward(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, m_h=m, momentum=0.9,
                           M=M2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(W1, W2) and torch.equal(M, M2)
    # first half, then second half from (W_out, M) of the first: identical to one call
    h = N // 2
    Ma = torch.zeros_like(M)
    oa, Wa = T.ttt_forward(q[:, :, :h].contiguous(), k[:, :, :h].contiguous(), v[:, :, :h].contiguous(),
                           eta[:, :, :h].contiguous(), W0, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, m_h=m,
                           momentum=0.9, M=Ma)
    ob, Wb = T.ttt_forward(q[:, :, h:].contiguous(), k[:, :, h:].contiguous(), v[:, :, h:].contiguous(),
                           eta[:, :, h:].contiguous(), Wa, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, m_h=m,
                           momentum=0.9, M=Ma)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=2), o1)
    assert torch.equal(Wb, W1) and torch.equal(Ma, M)


FULL = {
    # the LaCT language-model layer: B8 H4 N32768 d384 m768, chunk 2048, GD + L2
    "lact_lm_gd_l2": dict(B=8, H=4, N=32768, d=384, m=768, chunk=2048, mask=O.MASK_APPLY_THEN_UPDATE,
                          rule=O.UPD_GD_L2, mom=0.0, flags=None),
    # the same shapes with momentum 0.9 and Muon (5 Newton-Schulz steps) before L2
    "lact_lm_muon": dict(B=8, H=4, N=32768, d=384, m=768, chunk=2048, mask=O.MASK_APPLY_THEN_UPDATE,
                         rule=O.UPD_MUON_L2, mom=0.9, flags=None),
    # view-synthesis strided mask: 16 chunks of 4096, updates on the first 12, Muon, no momentum
    "nvs_strided_muon": dict(B=2, H=4, N=65536, d=256, m=512, chunk=4096, mask=O.MASK_STRIDED,
                             rule=O.UPD_MUON_L2, mom=0.0, flags=[1] * 12 + [0] * 4),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_slices(name):
    c = FULL[name]
    B, H, N, d, m = c["B"], c["H"], c["N"], c["d"], c["m"]
    # 8 scans spread over batches and heads (all of them when there are only 8)
    sample = sorted({(i % B, (i + i // B) % H) for i in range(min(8, B * H))})
    say(f"full-size {name}: sampled slices {sample}")
    q, k, v, eta, W0, ex, W = bulk_ttt_inputs(0, B, H, N, d, m, True, exact=sample)
    o, Wout = T.ttt_forward(q, k, v, eta, W0, c["chunk"], c["mask"], c["rule"], m_h=m, momentum=c["mom"],
                            update_chunks=c["flags"])
    torch.cuda.synchronize()
    say("  gpu done; oracle on sampled slices")
    for (b, h) in sample:
        qs, ks, vs, es = ex[(b, h)]
        o_ref, W_ref, _ = O.ttt_scan_ref(qs, ks, vs, es, W[0][h], W[1][h], W[2][h], c["chunk"], c["mask"], c["rule"],
                                         5, c["mom"], False, c["flags"])
        check(o[b, h], Wout[b, h], o_ref, W_ref, d, m, 2e-2, c["chunk"], label=f"slice ({b},{h})")
