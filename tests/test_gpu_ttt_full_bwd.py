"""GPU parity of ttt_backward with all three fast weights learning (last_layer_only = 0; GD or
GD + L2, with or without momentum), through the C ABI, against the fp64 oracle of the recurrence's
backward.

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
    lead = W1.shape[:-2]
    return np.concatenate([W1.reshape(*lead, -1), W3.reshape(*lead, -1), W2.reshape(*lead, -1)], axis=-1)


def split(W, d, m):
    dm = d * m
    return W[..., :dm].reshape(*W.shape[:-1], m, d), W[..., dm:2 * dm].reshape(*W.shape[:-1], m, d), \
        W[..., 2 * dm:].reshape(*W.shape[:-1], d, m)


def run(seed, B, H, N, d, m, chunk, mask, bf16, rule=O.UPD_GD_L2, flags=None, inner=1, ascent=False, momentum=0.0,
        per_batch=False, dW_out=True, want_dW0=True, last=False):
    say(f"full ttt_backward case B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} bf16={bf16} rule={rule} flags={flags} "
        f"inner{inner} ascent{ascent} momentum={momentum} per_batch={per_batch} dW_out={dW_out} want_dW0={want_dW0} "
        f"last={last}")
    (q, k, v, eta, W0), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(seed, B, H, N, d, m, bf16)
    if per_batch:
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
                         inner_steps=inner, ascent=ascent, momentum=momentum, update_rule=rule, last_layer_only=last)
    torch.cuda.synchronize()
    ref = O.ttt_backward_ref(hq, hk, hv, he, W1, W3, W2, chunk, mask, dO, dWo, flags, inner, ascent, momentum, rule,
                             last)
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
@pytest.mark.parametrize("rule", [O.UPD_GD, O.UPD_GD_L2])
@pytest.mark.parametrize("mask", [O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY])
def test_masks_rules_ragged(mask, rule, bf16):
    # 3 chunks of 96 and a tail of 20; m = 160 leaves partial hidden-unit tiles, d = 64 a partial
    # column tile
    run(1, 1, 2, 308, 64, 160, 96, mask, bf16, rule=rule)


@pytest.mark.parametrize("bf16", [False, True])
def test_full_mask(bf16):
    run(2, 1, 2, 150, 64, 96, 150, O.MASK_FULL, bf16)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("flags,inner,ascent", [([1, 0, 1, 1], 1, False), ([0, 0, 1, 0], 3, True)])
def test_strided_inner_ascent(flags, inner, ascent, bf16):
    # chunks that do not update read the weights of the next update (a query range of several
    # chunks); several inner steps collect dk, dv and deta over the chunk's steps
    got, _ = run(3, 1, 2, 308, 64, 160, 96, O.MASK_STRIDED, bf16, flags=flags, inner=inner, ascent=ascent)
    for c, f in enumerate(flags):
        if not f:
            assert torch.count_nonzero(got[1][:, :, 96 * c:96 * (c + 1)]).item() == 0
            assert torch.count_nonzero(got[3][:, :, 96 * c:96 * (c + 1)]).item() == 0


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,rule,inner,mom", [(O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, 1, 0.9),
                                                 (O.MASK_UPDATE_THEN_APPLY, O.UPD_GD, 2, 0.5)])
def test_momentum(mask, rule, inner, mom, bf16):
    run(4, 1, 2, 308, 64, 160, 96, mask, bf16, rule=rule, inner=inner, momentum=mom)


MUON_CASES = [
    # mask, rule, strided flags, inner steps, ascent, momentum, W2 alone
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, None, 1, False, 0.9, False),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON, None, 2, True, 0.0, False),
    (O.MASK_STRIDED, O.UPD_MUON_L2, [0, 1, 1, 0], 1, False, 0.5, False),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, None, 1, False, 0.9, True),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, None, 1, False, 0.9, True),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,rule,flags,inner,ascent,mom,last", MUON_CASES)
def test_muon(mask, rule, flags, inner, ascent, mom, last, bf16):
    # Newton-Schulz walked back in fp32 on every update (five steps); m = 160 > d = 64 makes W1, W3
    # tall and W2 wide
    run(14, 1, 2, 308, 64, 160, 96, mask, bf16, rule=rule, flags=flags, inner=inner, ascent=ascent, momentum=mom,
        last=last)


@pytest.mark.parametrize("bf16", [False, True])
def test_weight_layouts(bf16):
    # per-head weights: the gradient sums the batch's scans; per-(batch, head) weights: one each
    run(5, 3, 2, 260, 64, 128, 128, O.MASK_APPLY_THEN_UPDATE, bf16)
    run(6, 2, 2, 260, 64, 128, 128, O.MASK_APPLY_THEN_UPDATE, bf16, per_batch=True)


def test_wide_heads():
    # d = 128, m = 384: three hidden-unit tiles, several token tiles per chunk and weight-gradient
    # token parts
    run(7, 2, 1, 1100, 128, 384, 512, O.MASK_APPLY_THEN_UPDATE, True)
    run(8, 1, 2, 700, 128, 384, 256, O.MASK_UPDATE_THEN_APPLY, False, per_batch=True)


def test_defaults_and_optional_outputs():
    run(9, 1, 2, 200, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, dW_out=False)
    run(9, 1, 2, 200, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, dW_out=False, want_dW0=False)


def test_empty_sequence():
    for pb in (False, True):
        run(10, 2, 2, 0, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, per_batch=pb)


def test_full_size_sampled():
    # the LaCT-LLM layer's shape (B=8, H=4, N=32768, d=384, m=768, chunk 2048, bf16, GD + L2) with
    # per-(batch, head) weights; two slices come from the seeded generator and are compared with the
    # oracle (their weight-gradient blocks included), the others are filled on the device
    B, H, N, d, m, chunk = 8, 4, 32768, 384, 768, 2048
    say(f"full ttt_backward full-size case B{B} H{H} N{N} d{d} m{m} b{chunk}")
    picks = [(0, 0), (7, 3)]
    q, k, v, eta, W0h, ex, Wh = bulk_ttt_inputs(12, B, H, N, d, m, True, exact=picks)
    W0 = W0h[None].expand(B, H, -1).contiguous()
    g = torch.Generator(device="cuda")
    g.manual_seed(778)
    dO = (torch.randn((B, H, N, d), generator=g, device="cuda") / np.sqrt(d)).to(torch.bfloat16)
    dWo = torch.randn((B, H, 3 * d * m), generator=g, device="cuda") / np.sqrt(d)
    hg = {}
    for (b, h) in picks:
        dos, dws = synth.layer_grad_slice(12, b, h, N, d, m, True)
        dO[b, h] = dev(dos, torch.bfloat16)
        dWo[b, h] = dev(pack(*dws))
        hg[(b, h)] = (dos, dws)
    got = T.ttt_backward(q, k, v, eta, W0, dO, chunk, O.MASK_APPLY_THEN_UPDATE, m_h=m, dW_out=dWo,
                         update_rule=O.UPD_GD_L2, last_layer_only=False)
    torch.cuda.synchronize()
    for (b, h) in picks:
        qs, ks, vs, es = ex[(b, h)]
        dos, dws = hg[(b, h)]
        say(f"  oracle slice ({b}, {h})")
        ref = O.ttt_backward_scan_ref(qs, ks, vs, es, Wh[0][h], Wh[1][h], Wh[2][h], chunk, O.MASK_APPLY_THEN_UPDATE,
                                      dos, dws, rule=O.UPD_GD_L2)
        for name, gg, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert_close(host(gg[b, h]), r, TOL[True], f"{name}[{b},{h}]", chunk)
        assert_close(host(got[3][b, h])[None], ref[3][None], TOL[True], f"deta[{b},{h}]")
        for name, gg, r in zip(("dW1", "dW3", "dW2"), split(host(got[4][b, h]), d, m), ref[4]):
            assert_close(gg, r, TOL[True], f"{name}[{b},{h}]")
    for t in got:
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask,rule,mom,inner,last", [(O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, 0.0, 1, False),
                                                      (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, 0.9, 2, False),
                                                      (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, 0.5, 1, True)])
def test_training_record(mask, rule, mom, inner, last, bf16):
    # the training pair: ttt_forward_record's o and W_out are ttt_forward's, and the backward from the
    # record is ttt_backward's, bit for bit (the same kernels in the same order)
    say(f"training record case mask{mask} rule{rule} momentum{mom} inner{inner} last={last} bf16={bf16}")
    B, H, N, d, m, chunk = 2, 2, 308, 64, 160, 96
    (q, k, v, eta, W0), _ = full_ttt_inputs(15, B, H, N, d, m, bf16)
    dO, dWo = synth.make_ttt_grads(15, B, H, N, d, m, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    kw = dict(m_h=m, momentum=mom, inner_steps=inner, last_layer_only=last)
    o, W, rec = T.ttt_forward_record(q, k, v, eta, W0, chunk, mask, rule, **kw)
    o_ref, W_ref = T.ttt_forward(q, k, v, eta, W0, chunk, mask, rule, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(W, W_ref)
    args = (q, k, v, eta, W0, dev(dO, dt), chunk, mask)
    bkw = dict(m_h=m, dW_out=dev(pack(*dWo)), momentum=mom, inner_steps=inner, update_rule=rule, last_layer_only=last)
    a = T.ttt_backward(*args, **bkw)
    b = T.ttt_backward(*args, record=rec, **bkw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("bf16", [False, True])
def test_muon_orientations_and_small_shapes(bf16):
    # d > m makes W1, W3 wide and W2 tall (the other side of every Newton-Schulz product); a 48-token
    # chunk leaves single partial tiles; d = m = 32 is the smallest head
    run(16, 1, 2, 200, 128, 64, 48, O.MASK_APPLY_THEN_UPDATE, bf16, rule=O.UPD_MUON_L2, momentum=0.9)
    run(17, 1, 2, 130, 32, 32, 64, O.MASK_UPDATE_THEN_APPLY, bf16, rule=O.UPD_MUON, inner=2)
    run(18, 1, 2, 130, 128, 64, 130, O.MASK_FULL, bf16, rule=O.UPD_GD_L2, momentum=0.5)


@pytest.mark.parametrize("bf16", [False, True])
def test_muon_full_step_tiles(bf16):
    # d and m multiples of 128: the walk back's step tiles all lie inside their matrices and run the
    # full-tile workgroups (one LDS stage); W1, W3 tall and W2 wide, then the other way round
    run(22, 1, 2, 300, 128, 256, 128, O.MASK_APPLY_THEN_UPDATE, bf16, rule=O.UPD_MUON_L2, momentum=0.9)
    run(23, 1, 1, 256, 256, 128, 128, O.MASK_UPDATE_THEN_APPLY, bf16, rule=O.UPD_MUON)


def test_muon_weight_layouts_and_empty():
    run(19, 2, 2, 260, 64, 128, 128, O.MASK_APPLY_THEN_UPDATE, True, rule=O.UPD_MUON_L2, momentum=0.9,
        per_batch=True)
    run(20, 3, 2, 260, 64, 128, 128, O.MASK_UPDATE_THEN_APPLY, False, rule=O.UPD_MUON, momentum=0.9)
    run(21, 2, 2, 0, 64, 96, 64, O.MASK_APPLY_THEN_UPDATE, True, rule=O.UPD_MUON_L2, momentum=0.9)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rule,mom", [(O.UPD_GD, 0.0), (O.UPD_GD_L2, 0.9)])
def test_training_record_last_layer(rule, mom, bf16):
    # W2 alone by GD: the pair walks the recurrence back (with W1, W3 frozen), where ttt_backward
    # goes through linear attention over phi; both against the oracle
    say(f"training record, last layer, rule{rule} momentum{mom} bf16={bf16}")
    B, H, N, d, m, chunk = 1, 2, 308, 64, 160, 96
    (q, k, v, eta, W0), (hq, hk, hv, he, W1, W3, W2) = full_ttt_inputs(22, B, H, N, d, m, bf16)
    dO, dWo = synth.make_ttt_grads(22, B, H, N, d, m, bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    kw = dict(m_h=m, momentum=mom, last_layer_only=True)
    _, _, rec = T.ttt_forward_record(q, k, v, eta, W0, chunk, O.MASK_APPLY_THEN_UPDATE, rule, **kw)
    got = T.ttt_backward(q, k, v, eta, W0, dev(dO, dt), chunk, O.MASK_APPLY_THEN_UPDATE, dW_out=dev(pack(*dWo)),
                         update_rule=rule, record=rec, **kw)
    torch.cuda.synchronize()
    ref = O.ttt_lastlayer_backward_ref(hq, hk, hv, he, W1, W3, W2, chunk, O.MASK_APPLY_THEN_UPDATE, dO, dWo,
                                       momentum=mom, rule=rule)
    tol = TOL[bf16]
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_close(host(g), r, tol, name, chunk)
    assert_close(host(got[3]), ref[3], tol, "deta")
    for name, g, r in zip(("dW1", "dW3", "dW2"), split(host(got[4]), d, m), ref[4]):
        assert_close(g, r, tol, name)
