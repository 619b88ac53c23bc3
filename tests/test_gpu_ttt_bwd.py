"""GPU parity of ttt_backward (through the C ABI) against the fp64 oracle of the backward of the
layer whose inner loop trains W2 alone by plain GD.

Tolerances are the forward's: relative L2 <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs, over
every gradient as a whole, per (batch, head), per chunk of token rows, and 5x that per row."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import synth
import linear_attention_chunk_amd as T
from gpu_util import assert_close, bulk_ttt_inputs, dev, full_ttt_inputs, host, say

pytestmark = pytest.mark.gpu

TOL = {False: 1e-5, True: 2e-2}


def pack(W1, W3, W2):
    """[..., m, d], [..., m, d], [..., d, m] -> [..., 3 d m] (the library's weight block layout)."""
    lead = W1.shape[:-2]
    return np.concatenate([W1.reshape(*lead, -1), W3.reshape(*lead, -1), W2.reshape(*lead, -1)], axis=-1)


def split(W, d, m):
    dm = d * m
    return W[..., :dm].reshape(*W.shape[:-1], m, d), W[..., dm:2 * dm].reshape(*W.shape[:-1], m, d), \
        W[..., 2 * dm:].reshape(*W.shape[:-1], d, m)


def run(seed, B, H, N, d, m, chunk, mask, bf16, flags=None, inner=1, ascent=False, per_batch=False, dW_out=True,
        want_dW0=True, momentum=0.0, rule=O.UPD_GD):
    say(f"ttt_backward case B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} bf16={bf16} flags={flags} inner{inner} "
        f"ascent{ascent} per_batch={per_batch} dW_out={dW_out} want_dW0={want_dW0} momentum={momentum} rule={rule}")
    (q, k, v, eta, W0), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(seed, B, H, N, d, m, bf16)
    if per_batch:  # a different weight block for every (batch, head)
        Ws = [np.zeros((B, H) + w.shape[1:], np.float32) for w in (W1, W3, W2)]
        for b in range(B):
            for h in range(H):
                for i, w in enumerate(synth.head_weights(seed * 100 + b, h, d, m)):
                    Ws[i][b, h] = w
        W1, W3, W2 = Ws
        W0 = dev(pack(W1, W3, W2))
    dO, dWo = synth.make_ttt_grads(seed, B, H, N, d, m, bf16)
    dWo = dWo if dW_out else None
    dt = torch.bfloat16 if bf16 else torch.float32
    got = T.ttt_backward(q, k, v, eta, W0, dev(dO, dt), chunk, mask, m_h=m,
                         dW_out=None if dWo is None else dev(pack(*dWo)), want_dW0=want_dW0, update_chunks=flags,
                         inner_steps=inner, ascent=ascent, momentum=momentum, update_rule=rule)
    torch.cuda.synchronize()
    ref = O.ttt_lastlayer_backward_ref(hq, hk, hv, he, W1, W3, W2, chunk, mask, dO, dWo, flags, inner, ascent,
                                       momentum=momentum, rule=rule)
    tol = TOL[bf16]
    if N == 0:
        for g, r in zip(got[:4], ref[:4]):
            assert tuple(g.shape) == r.shape and g.numel() == 0
    else:
        for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert_close(host(g), r, tol, name, chunk)
        assert_close(host(got[3]), ref[3], tol, "deta")
    if want_dW0:
        assert tuple(got[4].shape) == tuple(W0.shape)
        for name, g, r in zip(("dW1", "dW3", "dW2"), split(host(got[4]), d, m), ref[4]):
            assert_close(g, r, tol, name)
    else:
        assert got[4] is None
    return got, ref


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask", [O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY])
def test_masks_ragged(mask, bf16):
    # 3 chunks of 96 and a tail of 20; m = 160 leaves partial feature, state and weight-gradient
    # tiles, d = 64 a partial dq / dk tile
    run(1, 1, 2, 308, 64, 160, 96, mask, bf16)


@pytest.mark.parametrize("bf16", [False, True])
def test_full_mask(bf16):
    run(2, 1, 2, 150, 64, 96, 150, O.MASK_FULL, bf16)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("flags,inner,ascent", [([1, 0, 1, 1], 1, False), ([0, 1, 1, 0], 3, True)])
def test_strided_inner_ascent(flags, inner, ascent, bf16):
    got, _ = run(3, 1, 2, 308, 64, 160, 96, O.MASK_STRIDED, bf16, flags=flags, inner=inner, ascent=ascent)
    # chunks that do not update give zero dv and deta
    for c, f in enumerate(flags):
        if not f:
            assert torch.count_nonzero(got[2][:, :, 96 * c:96 * (c + 1)]).item() == 0
            assert torch.count_nonzero(got[3][:, :, 96 * c:96 * (c + 1)]).item() == 0


MOMENTUM_CASES = [
    # mask, chunk, strided flags, inner steps, ascent, momentum
    (O.MASK_APPLY_THEN_UPDATE, 96, None, 1, False, 0.9),
    (O.MASK_UPDATE_THEN_APPLY, 96, None, 2, True, 0.5),
    (O.MASK_STRIDED, 96, [1, 0, 1, 1], 1, False, 0.9),
    (O.MASK_STRIDED, 96, [0, 1, 1, 0], 3, True, 0.7),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,chunk,flags,inner,ascent,mom", MOMENTUM_CASES)
def test_momentum(mask, chunk, flags, inner, ascent, mom, bf16):
    # the W2 steps through a momentum that starts from zero (the reverse scan walks the momentum
    # recurrence transposed); N = 308 leaves a ragged last chunk, m = 160 partial tiles
    run(11, 1, 2, 308, 64, 160, chunk, mask, bf16, flags=flags, inner=inner, ascent=ascent, momentum=mom)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,chunk,flags,inner,ascent,mom", MOMENTUM_CASES)
def test_momentum_fused_pass(mask, chunk, flags, inner, ascent, mom, bf16, monkeypatch):
    # the same with the forward states rebuilt by the linear attention's fused update-and-scan pass
    # (which these shapes alone would not pick): W2 per head as the entry state, the momentum, the
    # repeats and the sign of the steps
    monkeypatch.setenv("TTT_LIN_PASS", "fused")
    run(11, 1, 2, 308, 64, 160, chunk, mask, bf16, flags=flags, inner=inner, ascent=ascent, momentum=mom)


L2_CASES = [
    # mask, chunk, strided flags, inner steps, ascent, momentum
    (O.MASK_APPLY_THEN_UPDATE, 96, None, 1, False, 0.0),
    (O.MASK_UPDATE_THEN_APPLY, 96, None, 2, True, 0.0),
    (O.MASK_APPLY_THEN_UPDATE, 96, None, 1, False, 0.9),
    (O.MASK_STRIDED, 96, [0, 1, 1, 0], 3, False, 0.5),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,chunk,flags,inner,ascent,mom", L2_CASES)
def test_l2_norm(mask, chunk, flags, inner, ascent, mom, bf16):
    # Variant 1 without Muon: W2's rows L2-normalized after every step (the row-wise scans, forward
    # and transposed); m = 160 gives W2 rows that span two 128-wide float4 groups per lane
    run(12, 1, 2, 308, 64, 160, chunk, mask, bf16, flags=flags, inner=inner, ascent=ascent, momentum=mom,
        rule=O.UPD_GD_L2)


def test_l2_norm_full_mask_per_batch_weights():
    run(13, 2, 2, 150, 64, 96, 150, O.MASK_FULL, True, per_batch=True, rule=O.UPD_GD_L2)
    run(13, 2, 2, 150, 64, 96, 150, O.MASK_FULL, False, rule=O.UPD_GD_L2, momentum=0.9)


@pytest.mark.parametrize("bf16", [False, True])
def test_update_then_apply_inner_steps(bf16):
    run(4, 1, 1, 200, 64, 96, 64, O.MASK_UPDATE_THEN_APPLY, bf16, inner=2)


@pytest.mark.parametrize("bf16", [False, True])
def test_weight_layouts(bf16):
    # per-head weights: the gradient sums the batch's scans; per-(batch, head) weights: one each
    run(5, 3, 2, 260, 64, 128, 128, O.MASK_APPLY_THEN_UPDATE, bf16)
    run(6, 2, 2, 260, 64, 128, 128, O.MASK_APPLY_THEN_UPDATE, bf16, per_batch=True)


def test_wide_heads_and_token_parts():
    # d = 128, m = 384: three 128-row weight-gradient tiles, several feature tiles; the weight
    # gradient splits its 2 * 3 * 1100 token positions into parts
    run(7, 3, 1, 1100, 128, 384, 256, O.MASK_APPLY_THEN_UPDATE, True)
    run(8, 1, 2, 1100, 128, 384, 512, O.MASK_UPDATE_THEN_APPLY, False, per_batch=True)


def test_defaults_and_optional_outputs():
    run(9, 1, 2, 200, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, dW_out=False)
    run(9, 1, 2, 200, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, dW_out=False, want_dW0=False)


def test_empty_sequence():
    # N = 0: no token gradients; dW0 is the batch sum of dW_out (zero without it)
    for dwo in (True, False):
        for pb in (False, True):
            run(10, 2, 2, 0, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, per_batch=pb, dW_out=dwo)


def test_full_size_sampled():
    # the LaCT-LLM layer's shape (B=8, H=4, N=32768, d=384, m=768, chunk 2048, bf16) with
    # per-(batch, head) weights; two slices come from the seeded generator and are compared with
    # the oracle (their weight-gradient blocks included), the others are filled on the device
    B, H, N, d, m, chunk = 8, 4, 32768, 384, 768, 2048
    say(f"ttt_backward full-size case B{B} H{H} N{N} d{d} m{m} b{chunk}")
    picks = [(0, 0), (7, 3)]
    q, k, v, eta, W0h, ex, Wh = bulk_ttt_inputs(12, B, H, N, d, m, True, exact=picks)
    W0 = W0h[None].expand(B, H, -1).contiguous()
    g = torch.Generator(device="cuda")
    g.manual_seed(777)
    dO = (torch.randn((B, H, N, d), generator=g, device="cuda") / np.sqrt(d)).to(torch.bfloat16)
    dWo = torch.randn((B, H, 3 * d * m), generator=g, device="cuda") / np.sqrt(d)
    hg = {}
    for (b, h) in picks:
        dos, dws = synth.layer_grad_slice(12, b, h, N, d, m, True)
        dO[b, h] = dev(dos, torch.bfloat16)
        dWo[b, h] = dev(pack(*dws))
        hg[(b, h)] = (dos, dws)
    got = T.ttt_backward(q, k, v, eta, W0, dO, chunk, O.MASK_APPLY_THEN_UPDATE, m_h=m, dW_out=dWo)
    torch.cuda.synchronize()
    for (b, h) in picks:
        qs, ks, vs, es = ex[(b, h)]
        dos, dws = hg[(b, h)]
        say(f"  oracle slice ({b}, {h})")
        ref = O.ttt_lastlayer_backward_scan_ref(qs, ks, vs, es, Wh[0][h], Wh[1][h], Wh[2][h], chunk,
                                                O.MASK_APPLY_THEN_UPDATE, dos, dws)
        for name, gg, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert_close(host(gg[b, h]), r, TOL[True], f"{name}[{b},{h}]", chunk)
        assert_close(host(got[3][b, h])[None], ref[3][None], TOL[True], f"deta[{b},{h}]")
        for name, gg, r in zip(("dW1", "dW3", "dW2"), split(host(got[4][b, h]), d, m), ref[4]):
            assert_close(gg, r, TOL[True], f"{name}[{b},{h}]")
    for t in got:
        assert torch.isfinite(t).all()
