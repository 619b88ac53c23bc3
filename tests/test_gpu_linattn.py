"""GPU parity of linattn_forward (through the C ABI) against the fp64 oracle.

Tolerances: relative L2 <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs (fp32 state)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import synth
import linear_attention_chunk_amd as T
from gpu_util import assert_close, dev, host, rel, say

pytestmark = pytest.mark.gpu

TOL = {False: 1e-5, True: 2e-2}


def run(seed, B, H, N, dk, dv, chunk, mask, bf16, S0=False, flags=None):
    say(f"linattn case B{B} H{H} N{N} dk{dk} dv{dv} b{chunk} mask{mask} bf16={bf16} S0={S0}")
    q, k, v, eta = synth.make_linattn_inputs(seed, B, H, N, dk, dv, bf16)
    s0 = None
    if S0:
        rng = np.random.default_rng(seed + 99)
        s0 = (rng.standard_normal((B, H, dv, dk)) * 0.1).astype(np.float32)
    dt = torch.bfloat16 if bf16 else torch.float32
    o, S = T.linattn_forward(dev(q, dt), dev(k, dt), dev(v, dt), dev(eta), chunk, mask,
                             S0=None if s0 is None else dev(s0), update_chunks=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = O.linattn_forward_ref(q, k, v, eta, chunk, mask, s0, flags)
    # per (batch, head), per chunk (of 128 tokens in token-causal mode) and per row as well
    assert_close(host(o), o_ref, TOL[bf16], "o", chunk if mask != O.MASK_TOKEN_CAUSAL else 128)
    assert_close(host(S), S_ref, TOL[bf16], "S_out")
    return o, S


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask", [O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY, O.MASK_TOKEN_CAUSAL])
def test_masks_ragged(mask, bf16):
    # chunks of 80 leave partial sub-blocks; N = 300 leaves a ragged last chunk
    run(1, 1, 3, 300, 64, 96, 80, mask, bf16, S0=True)


@pytest.mark.parametrize("bf16", [False, True])
def test_full_and_strided(bf16):
    run(2, 2, 1, 150, 32, 64, 150, O.MASK_FULL, bf16, S0=True)
    run(3, 1, 2, 256, 128, 64, 32, O.MASK_STRIDED, bf16, flags=[1, 0, 0, 1, 1, 0, 1, 0])


@pytest.mark.parametrize("bf16", [False, True])
def test_strided_chunk_parallel(bf16):
    # chunk 128 at d_k = d_v = 64 takes the chunk-parallel path; N = 700 leaves a ragged last chunk
    run(5, 1, 2, 700, 64, 64, 128, O.MASK_STRIDED, bf16, S0=True, flags=[1, 0, 1, 1, 0, 1])
    # and the all-zero flags: the state never moves
    run(6, 1, 1, 300, 64, 64, 128, O.MASK_STRIDED, bf16, S0=True, flags=[0, 0, 0])


PASS_CASES = [
    # seed, B, H, N, d_k, d_v, chunk, mask, S0, strided flags
    (21, 1, 3, 300, 64, 96, 80, O.MASK_APPLY_THEN_UPDATE, True, None),    # ragged chunk, partial tiles
    (22, 1, 3, 300, 64, 96, 80, O.MASK_UPDATE_THEN_APPLY, True, None),
    (23, 2, 1, 150, 32, 64, 150, O.MASK_FULL, True, None),
    (24, 1, 2, 700, 64, 64, 128, O.MASK_STRIDED, True, [1, 0, 1, 1, 0, 1]),
    (25, 1, 1, 300, 64, 64, 128, O.MASK_STRIDED, True, [0, 0, 0]),
    (26, 1, 2, 1024, 128, 128, 256, O.MASK_APPLY_THEN_UPDATE, False, None),  # whole tiles and stages
    (27, 1, 2, 1100, 96, 160, 512, O.MASK_UPDATE_THEN_APPLY, True, None),    # several stages per chunk
    (28, 1, 1, 600, 384, 160, 64, O.MASK_TOKEN_CAUSAL, True, None),
    # chunks of 128 tokens go two to a 256-token bf16 stage in the fused pass: whole pairs, an odd
    # chunk count with a ragged last chunk, and strided pairs with one, both or neither updating
    (29, 1, 2, 1024, 128, 128, 128, O.MASK_UPDATE_THEN_APPLY, True, None),
    (30, 1, 2, 600, 96, 160, 128, O.MASK_APPLY_THEN_UPDATE, True, None),
    (31, 1, 2, 1100, 64, 64, 128, O.MASK_STRIDED, True, [1, 0, 0, 0, 1, 1, 0, 1, 1]),
    (32, 1, 1, 1024, 128, 64, 128, O.MASK_TOKEN_CAUSAL, False, None),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", PASS_CASES)
def test_fused_and_split_passes(case, bf16, monkeypatch):
    # the chunk updates and the scan as one fused pass and as two: each against the oracle, and the
    # two bit for bit (the same token sums in the same order, the same fp32 state additions)
    seed, B, H, N, dk, dv, chunk, mask, S0, flags = case
    got = {}
    for p in ("fused", "split"):
        monkeypatch.setenv("TTT_LIN_PASS", p)
        say(f"pass {p}")
        got[p] = run(seed, B, H, N, dk, dv, chunk, mask, bf16, S0=S0, flags=flags)
    for a, b in zip(got["fused"], got["split"]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("bf16", [False, True])
def test_causal_long_ragged(bf16):
    # 700 tokens: 11 sub-blocks of 64, the last ragged; the chunk size plays no part in this mode
    run(8, 1, 2, 700, 64, 96, 50, O.MASK_TOKEN_CAUSAL, bf16, S0=True)


def test_small_chunks_sequential():
    # chunk 16 at d_k = d_v = 64 stays on the sequential kernel for the chunked masks too
    run(7, 1, 2, 200, 64, 64, 16, O.MASK_APPLY_THEN_UPDATE, True, S0=True)
    run(7, 1, 2, 200, 64, 64, 16, O.MASK_UPDATE_THEN_APPLY, False, S0=True)


@pytest.mark.parametrize("dk", [96, 256])
def test_wide_heads(dk):
    run(4, 1, 1, 200, dk, 32, 64, O.MASK_TOKEN_CAUSAL, True)
    run(4, 1, 1, 200, dk, 32, 64, O.MASK_APPLY_THEN_UPDATE, False)


@pytest.mark.parametrize("bf16", [False, True])
def test_wide_keys_chunk_parallel(bf16):
    # d_k beyond the sequential kernel's 256 runs on the chunk-parallel path: 384 spans three
    # 128-wide state tiles, 320 leaves a partial one; N = 1100 leaves a ragged last chunk
    run(8, 1, 2, 1100, 384, 384, 512, O.MASK_APPLY_THEN_UPDATE, bf16, S0=True)
    run(9, 1, 1, 1100, 320, 96, 512, O.MASK_UPDATE_THEN_APPLY, bf16)
    # token-causal mode takes the same path over 128-token blocks (600 tokens: a ragged last block)
    run(10, 1, 1, 600, 384, 160, 64, O.MASK_TOKEN_CAUSAL, bf16, S0=True)


def test_maximum_widths():
    # d_k at its maximum (2048, sixteen 128-wide state tiles) in chunked and token-causal mode, and
    # d_v at its maximum (4096) on the sequential kernel (chunk 32) and the chunk-parallel one
    run(11, 1, 1, 600, 2048, 96, 256, O.MASK_APPLY_THEN_UPDATE, True, S0=True)
    run(12, 1, 1, 300, 2048, 64, 64, O.MASK_TOKEN_CAUSAL, True)
    run(13, 1, 1, 300, 64, 4096, 32, O.MASK_APPLY_THEN_UPDATE, True)
    run(14, 1, 1, 300, 64, 4096, 128, O.MASK_UPDATE_THEN_APPLY, True, S0=True)


@pytest.mark.parametrize("mask", [O.MASK_APPLY_THEN_UPDATE, O.MASK_TOKEN_CAUSAL])
def test_linear_attention_workload_full_size(mask):
    """B4 H16 N8192 chunk 256, d_k = d_v = 128, bf16 q/k/v, eta = 0.05 sigmoid, fp32 state; the oracle
    checks sampled (batch, head) slices, generated by the seeded generator."""
    B, H, N, d, chunk = 4, 16, 8192, 128, 256
    sample = [(0, 0), (1, 7), (3, 15)]
    say(f"linattn full size mask{mask}")
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    s = 1.0 / np.sqrt(d)
    q = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    k = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    v = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(torch.bfloat16)
    eta = 0.05 * torch.sigmoid(torch.randn((B, H, N), generator=g, device="cuda"))
    ex = {}
    for b, h in sample:
        qs, ks, vs, es = synth.slice_inputs(0, b, h, N, d, d, "sigmoid", 0.05, True)
        q[b, h], k[b, h], v[b, h], eta[b, h] = dev(qs, torch.bfloat16), dev(ks, torch.bfloat16), \
            dev(vs, torch.bfloat16), dev(es)
        ex[(b, h)] = (qs, ks, vs, es)
    o, S = T.linattn_forward(q, k, v, eta.contiguous(), chunk, mask)
    torch.cuda.synchronize()
    for b, h in sample:
        qs, ks, vs, es = ex[(b, h)]
        o_ref, S_ref = O.linattn_scan_ref(qs, ks, vs, es, np.zeros((d, d)), chunk, mask)
        say(f"  slice ({b},{h})")
        assert_close(host(o[b, h]), o_ref, 2e-2, "o", chunk)
        assert_close(host(S[b, h]), S_ref, 2e-2, "S_out")


@pytest.mark.parametrize("lin_pass", ["fused", "split"])
@pytest.mark.parametrize("mask,chunk", [(O.MASK_APPLY_THEN_UPDATE, 128), (O.MASK_UPDATE_THEN_APPLY, 128),
                                        (O.MASK_TOKEN_CAUSAL, 64), (O.MASK_APPLY_THEN_UPDATE, 16)])
def test_nan_in_v_reaches_exactly_the_outputs_that_depend_on_it(mask, chunk, lin_pass, monkeypatch):
    """A NaN in value entry e of token t enters the state's row e only, so only column e of the
    outputs can turn NaN, and every other output and every other scan keep the bits of the run
    without it.  Under the chunked masks the NaN set is exactly the tokens that see token t (from
    the next chunk on, or from t's own chunk under update-then-apply): chunk-parallel path at chunk
    128, sequential kernel at chunk 16.  In token-causal mode every t' >= t sees it; the intra-block
    product P v of the 64 query rows holding t (a 128-token block's P v runs in two 64-row halves,
    the first over the block's first 64 keys only) also multiplies the NaN by the zeros of the causal
    mask, so those rows' earlier tokens turn NaN as well (0 * NaN is NaN in any MFMA)."""
    monkeypatch.setenv("TTT_LIN_PASS", lin_pass)  # (both ways through the chunk updates and the scan)
    B, H, N, dk, dv = 1, 2, 512, 64, 64
    q, k, v, eta = synth.make_linattn_inputs(43, B, H, N, dk, dv, True)
    dt = torch.bfloat16
    qd, kd, vd, ed = dev(q, dt), dev(k, dt), dev(v, dt), dev(eta)
    o_ref, S_ref = T.linattn_forward(qd, kd, vd, ed, chunk, mask)
    t, e = 200, 5
    vn = vd.clone()
    vn[0, 1, t, e] = float("nan")
    o_n, S_n = T.linattn_forward(qd, kd, vn, ed, chunk, mask)
    torch.cuda.synchronize()
    if mask == O.MASK_TOKEN_CAUSAL:
        first = (t // 64) * 64
    elif mask == O.MASK_UPDATE_THEN_APPLY:
        first = (t // chunk) * chunk
    else:
        first = (t // chunk + 1) * chunk
    nan = torch.isnan(o_n[0, 1].float())
    want = torch.zeros_like(nan)
    want[first:, e] = True
    assert torch.equal(nan, want), (int(nan.sum()), int(want.sum()))
    keep = ~want
    assert torch.equal(o_n[0, 1][keep], o_ref[0, 1][keep]) and torch.equal(o_n[0, 0], o_ref[0, 0])
    assert torch.isnan(S_n[0, 1, e]).all() and not torch.isnan(S_n[0, 1, :e]).any()
    assert torch.equal(S_n[0, 0], S_ref[0, 0])
