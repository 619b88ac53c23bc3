"""GPU parity of ttt_forward (through the C ABI) against the fp64 oracle.

Tolerances: relative L2 over the compared tensor <= 1e-5 with fp32 inputs and <= 2e-2 with bf16
inputs (fp32 fast weights in both), for the outputs o and the final fast weights W_out.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import linear_attention_chunk_amd as T
from gpu_util import bulk_ttt_inputs, full_ttt_inputs, host, rel, say

pytestmark = pytest.mark.gpu

TOL = {False: 1e-5, True: 2e-2}


def split_w(Wout, d, m):
    W = host(Wout)
    dm = d * m
    return W[..., :dm].reshape(*W.shape[:-1], m, d), W[..., dm:2 * dm].reshape(*W.shape[:-1], m, d), \
        W[..., 2 * dm:].reshape(*W.shape[:-1], d, m)


def check(o_gpu, W_gpu, o_ref, W_ref, d, m, tol, slices=None, label=""):
    og = host(o_gpu)
    Wg = split_w(W_gpu, d, m)
    if slices is not None:
        idx = tuple(np.array(s) for s in zip(*slices))
        og, o_ref = og[idx], o_ref[idx]
        Wg = [w[idx] for w in Wg]
        W_ref = [w[idx] for w in W_ref]
    eo = rel(og, o_ref)
    ew = max(rel(a, b) for a, b in zip(Wg, W_ref))
    say(f"  {label} rel_o={eo:.3e} rel_W={ew:.3e} tol={tol}")
    assert np.isfinite(og).all()
    assert eo <= tol, f"output rel L2 {eo} > {tol}"
    assert ew <= tol, f"W_out rel L2 {ew} > {tol}"


def run_small(seed, B, H, N, d, m, chunk, mask, rule, bf16, momentum=0.0, last=False, flags=None, ns=5, inner=1,
              ascent=False, parallel=False):
    say(f"ttt case B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} rule{rule} mom{momentum} last{last} bf16={bf16}"
        f" inner{inner} ascent{ascent} parallel{parallel}")
    (q, k, v, eta, W0), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(seed, B, H, N, d, m, bf16)
    o, Wout = T.ttt_forward(q, k, v, eta, W0, chunk, mask, rule, m_h=m, ns_iters=ns, momentum=momentum,
                            last_layer_only=last, update_chunks=flags, inner_steps=inner, ascent=ascent,
                            parallel_form=parallel)
    torch.cuda.synchronize()
    o_ref, W_ref, _ = O.ttt_forward_ref(hq, hk, hv, he, W1, W3, W2, chunk, mask, rule, ns, momentum, last, flags,
                                        inner_steps=inner, ascent=ascent)
    check(o, Wout, o_ref, W_ref, d, m, TOL[bf16], label="all slices")


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
    # p = min(d, m) = 160 spans two 128-wide Gram tiles, the second partial: the off-diagonal tile
    # also writes its mirror block; both Gram sides (m > d, then d > m)
    run_small(12, 1, 1, 256, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, False, ns=3)
    run_small(13, 1, 1, 256, 320, 160, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, False, ns=2)
    # 32 scans: enough 128-wide Gram tiles that the kernel keeps them (fewer scans take 64-wide ones)
    run_small(21, 8, 4, 128, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, False, ns=2)


def test_newton_schulz_tiles_bf16():
    # d = 160, m = 320: W1/W3 take the tall step (320 x 160) and W2 the wide one (160 x 320), each
    # with full 128 x 64 step tiles beside ragged ones; the iterate is the bf16 hi + lo pair
    run_small(24, 1, 1, 256, 160, 320, 128, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, True, ns=3)
    run_small(25, 1, 2, 300, 160, 320, 128, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, True, momentum=0.9, ns=5)


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


def test_parallel_form_many_strided_chunks_fp32():
    # 40 chunks of 32 tokens: the strided update flags span two 32-bit words
    flags = [(j * 7) % 3 != 0 for j in range(40)]
    run_small(33, 1, 1, 1280, 64, 96, 32, O.MASK_STRIDED, O.UPD_GD, False, 0.9, last=True, flags=flags,
              parallel=True)


@pytest.mark.parametrize("bf16", [False, True])
def test_parallel_form_full_mask(bf16):
    run_small(31, 2, 1, 200, 32, 96, 200, O.MASK_FULL, O.UPD_GD, bf16, last=True, parallel=True)


def test_parallel_form_matches_recurrence():
    # several 256-token feature tiles and 128-wide state tiles: the parallel form with W0 given per
    # (batch, head) against the chunk recurrence with W0 per head, momentum carried in M
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
    sample = [(0, 0), (B - 1, H - 1)]
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
        og = host(o[b, h])
        Wg = split_w(Wout[b, h], d, m)
        eo = rel(og, o_ref)
        ew = max(rel(a, bb) for a, bb in zip(Wg, W_ref))
        say(f"  slice ({b},{h}) rel_o={eo:.3e} rel_W={ew:.3e}")
        assert eo <= 2e-2 and ew <= 2e-2
