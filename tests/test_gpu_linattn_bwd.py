"""GPU parity of linattn_backward (through the C ABI) against the fp64 oracle of the backward.

Tolerances are the forward's: relative L2 <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs, over
every gradient as a whole, per (batch, head), per chunk of token rows, and 5x that per row."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import synth
import linear_attention_chunk_amd as T
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

TOL = {False: 1e-5, True: 2e-2}


def run(seed, B, H, N, dk, dv, chunk, mask, bf16, S0=True, dS_out=True, flags=None, want_dS0=True):
    say(f"linattn_backward case B{B} H{H} N{N} dk{dk} dv{dv} b{chunk} mask{mask} bf16={bf16} "
        f"S0={S0} dS_out={dS_out} flags={flags}")
    q, k, v, eta = synth.make_linattn_inputs(seed, B, H, N, dk, dv, bf16)
    dO, dSo = synth.make_linattn_grads(seed, B, H, N, dk, dv, bf16)
    s0 = None
    if S0:
        rng = np.random.default_rng(seed + 99)
        s0 = (rng.standard_normal((B, H, dv, dk)) * 0.1).astype(np.float32)
    dSo = dSo if dS_out else None
    dt = torch.bfloat16 if bf16 else torch.float32
    got = T.linattn_backward(dev(q, dt), dev(k, dt), dev(v, dt), dev(eta), dev(dO, dt), chunk, mask,
                             S0=None if s0 is None else dev(s0), dS_out=None if dSo is None else dev(dSo),
                             update_chunks=flags, want_dS0=want_dS0)
    torch.cuda.synchronize()
    ref = O.linattn_backward_ref(q, k, v, eta, chunk, mask, dO, s0, dSo, flags)
    tol = TOL[bf16]
    if N == 0:  # nothing per token
        for g, r in zip(got[:4], ref[:4]):
            assert tuple(g.shape) == r.shape and g.numel() == 0
    else:
        for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert_close(host(g), r, tol, name, chunk)
        assert_close(host(got[3]), ref[3], tol, "deta")
    if want_dS0:
        assert_close(host(got[4]), ref[4], tol, "dS0")
    else:
        assert got[4] is None
    return got, ref


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mask", [O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY])
def test_masks_ragged(mask, bf16):
    # chunks of 80 tokens leave a partial 128-row tile in every chunk; N = 300 leaves a ragged last chunk
    run(1, 1, 3, 300, 64, 96, 80, mask, bf16)


@pytest.mark.parametrize("bf16", [False, True])
def test_full_mask(bf16):
    run(2, 2, 1, 150, 32, 64, 150, O.MASK_FULL, bf16)
    # a chunk longer than the sequence is the same single chunk
    run(2, 1, 1, 150, 32, 64, 400, O.MASK_FULL, bf16, S0=False)


@pytest.mark.parametrize("bf16", [False, True])
def test_strided(bf16):
    # dk, dv and deta are exactly zero over the chunks that do not update
    got, _ = run(5, 1, 2, 700, 64, 64, 128, O.MASK_STRIDED, bf16, flags=[1, 0, 1, 1, 0, 1])
    for g in got[1:3]:
        assert torch.count_nonzero(g[:, :, 128:256]).item() == 0
        assert torch.count_nonzero(g[:, :, 512:640]).item() == 0
    assert torch.count_nonzero(got[3][:, :, 128:256]).item() == 0
    # all-zero flags: only dq and dS0 are not zero
    got, _ = run(6, 1, 1, 300, 64, 64, 128, O.MASK_STRIDED, bf16, flags=[0, 0, 0])
    for g in got[1:4]:
        assert torch.count_nonzero(g).item() == 0


@pytest.mark.parametrize("bf16", [False, True])
def test_wide_heads(bf16):
    # d_v = 384 spans three 128-column tiles (deta from per-tile partials); d_k = 320 leaves a partial
    # one; N = 1100 leaves a ragged last chunk
    run(8, 1, 2, 1100, 320, 384, 512, O.MASK_APPLY_THEN_UPDATE, bf16)
    run(9, 1, 1, 600, 96, 160, 256, O.MASK_UPDATE_THEN_APPLY, bf16, S0=False)


PASS_CASES = [
    # seed, B, H, N, d_k, d_v, chunk, mask, strided flags
    (21, 1, 3, 300, 64, 96, 80, O.MASK_APPLY_THEN_UPDATE, None),
    (22, 1, 3, 300, 64, 96, 80, O.MASK_UPDATE_THEN_APPLY, None),
    (23, 2, 1, 150, 32, 64, 150, O.MASK_FULL, None),
    (24, 1, 2, 700, 64, 64, 128, O.MASK_STRIDED, [1, 0, 1, 1, 0, 1]),
    (25, 1, 2, 1024, 128, 128, 256, O.MASK_APPLY_THEN_UPDATE, None),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", PASS_CASES)
def test_fused_and_split_passes(case, bf16, monkeypatch):
    # the forward states rebuilt by the fused update-and-scan pass and by the two-pass one: each
    # against the oracle, and the two bit for bit
    seed, B, H, N, dk, dv, chunk, mask, flags = case
    got = {}
    for p in ("fused", "split"):
        monkeypatch.setenv("TTT_LIN_PASS", p)
        say(f"pass {p}")
        got[p], _ = run(seed, B, H, N, dk, dv, chunk, mask, bf16, flags=flags)
    for a, b in zip(got["fused"], got["split"]):
        assert torch.equal(a, b)


def test_small_chunks_and_defaults():
    # many small chunks (each a partial tile); no S0, no dS_out, no dS0 requested
    run(7, 1, 2, 200, 64, 64, 16, O.MASK_APPLY_THEN_UPDATE, True, S0=False, dS_out=False, want_dS0=False)
    run(7, 1, 2, 200, 64, 64, 16, O.MASK_UPDATE_THEN_APPLY, False, dS_out=False)


def test_empty_sequence():
    # N = 0: no token gradients, dS0 = dS_out (or zero without it)
    for dso in (True, False):
        got, ref = run(10, 2, 2, 0, 64, 32, 64, O.MASK_APPLY_THEN_UPDATE, True, dS_out=dso)
        assert got[0].numel() == 0


@pytest.mark.parametrize("bf16", [True])
def test_full_size_sampled(bf16):
    # the linear-attention workload (B=4, H=16, N=8192, chunk 256, d_k = d_v = 128) on the device,
    # with three (batch, head) slices drawn from the seeded generator and compared with the oracle;
    # the rest are filled on the device with the same distributions
    B, H, N, d, chunk = 4, 16, 8192, 128, 256
    say(f"linattn_backward full-size case B{B} H{H} N{N} d{d} b{chunk}")
    dt = torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    s = 1.0 / np.sqrt(d)
    q, k, v, dO = ((torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(dt) for _ in range(4))
    eta = (0.05 * torch.sigmoid(torch.randn((B, H, N), generator=g, device="cuda"))).float()
    dSo = torch.randn((B, H, d, d), generator=g, device="cuda") * s
    picks = [(0, 0), (1, 7), (3, 15)]
    ex = {}
    for (b, h) in picks:
        qs, ks, vs, es = synth.slice_inputs(11, b, h, N, d, d, "sigmoid", 0.05, True)
        dos, dss = synth.grad_slice(11, b, h, N, d, d, True)
        q[b, h], k[b, h], v[b, h], eta[b, h] = dev(qs, dt), dev(ks, dt), dev(vs, dt), dev(es)
        dO[b, h], dSo[b, h] = dev(dos, dt), dev(dss)
        ex[(b, h)] = (qs, ks, vs, es, dos, dss)
    got = T.linattn_backward(q, k, v, eta, dO, chunk, O.MASK_APPLY_THEN_UPDATE, dS_out=dSo)
    torch.cuda.synchronize()
    for (b, h), (qs, ks, vs, es, dos, dss) in ex.items():
        ref = O.linattn_backward_scan_ref(qs, ks, vs, es, np.zeros((d, d)), chunk, O.MASK_APPLY_THEN_UPDATE, dos, dss)
        for name, gg, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            assert_close(host(gg[b, h]), r, TOL[bf16], f"{name}[{b},{h}]", chunk)
        assert_close(host(got[3][b, h])[None], ref[3][None], TOL[bf16], f"deta[{b},{h}]")
        assert_close(host(got[4][b, h]), ref[4], TOL[bf16], f"dS0[{b},{h}]")
    for t in got:
        assert torch.isfinite(t).all()
