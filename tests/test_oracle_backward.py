"""Pins of the backward of chunked linear attention (CPU only), each against an independent route:
central finite differences of L = sum dO . o + <dS_out, S_out> through the forward oracle, and
torch's autograd in float64 through a forward written here with torch operations."""
import numpy as np
import pytest

import oracle as O


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def problem(seed, N=11, dk=3, dv=4):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((2, N, dk))
    v = rng.standard_normal((N, dv))
    eta = rng.standard_normal(N)
    S0 = rng.standard_normal((dv, dk))
    dO = rng.standard_normal((N, dv))
    dSo = rng.standard_normal((dv, dk))
    return q, k, v, eta, S0, dO, dSo


def loss(q, k, v, eta, S0, chunk, mask, dO, dSo, upd):
    o, S = O.linattn_scan_ref(q, k, v, eta, S0, chunk, mask, upd)
    return float(np.sum(dO * o) + np.sum(dSo * S))


MASKS = [(O.MASK_APPLY_THEN_UPDATE, 3, None), (O.MASK_UPDATE_THEN_APPLY, 4, None), (O.MASK_FULL, 11, None),
         (O.MASK_STRIDED, 3, [1, 0, 1, 1])]


@pytest.mark.parametrize("mask,chunk,upd", MASKS)
def test_backward_matches_finite_differences(mask, chunk, upd):
    q, k, v, eta, S0, dO, dSo = problem(60 + mask)
    dq, dk, dv, de, dS0 = O.linattn_backward_scan_ref(q, k, v, eta, S0, chunk, mask, dO, dSo, upd)
    args = [q, k, v, eta, S0]
    h = 1e-6
    for which, g in zip(range(5), (dq, dk, dv, de, dS0)):
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(*args[which].shape):
            a = [x.copy() for x in args]
            a[which][idx] += h
            lp = loss(*a, chunk, mask, dO, dSo, upd)
            a[which][idx] -= 2 * h
            lm = loss(*a, chunk, mask, dO, dSo, upd)
            fd[idx] = (lp - lm) / (2 * h)
        assert rel(g, fd) < 1e-7, which


@pytest.mark.parametrize("mask,chunk,upd", MASKS)
def test_backward_matches_torch_autograd(mask, chunk, upd):
    torch = pytest.importorskip("torch")
    q, k, v, eta, S0, dO, dSo = problem(70 + mask, N=13, dk=5, dv=6)
    if mask == O.MASK_FULL:
        chunk = 13
    if upd is not None:
        upd = [1, 0, 1, 1, 0]
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, eta, S0)]
    tq, tk, tv, te, ts = t
    # the forward again, written with torch operations: each chunk applies its state, then (or
    # first, under update-then-apply) adds its own update
    post = mask in (O.MASK_UPDATE_THEN_APPLY, O.MASK_FULL)
    S, outs = ts, []
    for j, lo in enumerate(range(0, 13, chunk)):
        hi = min(lo + chunk, 13)
        dS = (te[lo:hi, None] * tv[lo:hi]).T @ tk[lo:hi]
        if mask == O.MASK_STRIDED and not upd[j]:
            dS = torch.zeros_like(dS)
        if post:
            S = S + dS
        outs.append(tq[lo:hi] @ S.T)
        if not post:
            S = S + dS
    L = (torch.cat(outs) * torch.tensor(dO)).sum() + (S * torch.tensor(dSo)).sum()
    L.backward()
    got = O.linattn_backward_scan_ref(q, k, v, eta, S0, chunk, mask, dO, dSo, upd)
    for g, x in zip(got, t):
        assert rel(g, x.grad.numpy()) < 1e-12


def test_backward_batched_wrapper_and_defaults():
    rng = np.random.default_rng(80)
    B, H, N, dk, dv = 2, 3, 9, 3, 4
    q, k = rng.standard_normal((2, B, H, N, dk))
    v, dO = rng.standard_normal((2, B, H, N, dv))
    eta = rng.standard_normal((B, H, N))
    S0 = rng.standard_normal((B, H, dv, dk))
    dSo = rng.standard_normal((B, H, dv, dk))
    res = O.linattn_backward_ref(q, k, v, eta, 4, O.MASK_APPLY_THEN_UPDATE, dO, S0, dSo)
    for b in range(B):
        for h in range(H):
            one = O.linattn_backward_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], S0[b, h], 4,
                                              O.MASK_APPLY_THEN_UPDATE, dO[b, h], dSo[b, h])
            for a, bb in zip(res, one):
                assert rel(a[b, h], bb) == 0.0
    # no S0 is a zero state (it does not enter the gradients of q, k, v, eta under these masks except
    # through dq), no dS_out is a zero output gradient
    r0 = O.linattn_backward_ref(q, k, v, eta, 4, O.MASK_APPLY_THEN_UPDATE, dO)
    r1 = O.linattn_backward_ref(q, k, v, eta, 4, O.MASK_APPLY_THEN_UPDATE, dO, np.zeros_like(S0), np.zeros_like(dSo))
    for a, bb in zip(r0, r1):
        assert rel(a, bb) == 0.0


def test_backward_empty_sequence():
    # no tokens: S_out = S0, so dS0 = dS_out (zero without it) and every token gradient is empty
    rng = np.random.default_rng(81)
    q, k = np.zeros((2, 0, 3))
    v = dO = np.zeros((0, 4))
    eta = np.zeros(0)
    S0, dSo = rng.standard_normal((2, 4, 3))
    for mask in (O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY):
        dq, dk, dv, de, dS0 = O.linattn_backward_scan_ref(q, k, v, eta, S0, 5, mask, dO, dSo)
        assert dq.shape == (0, 3) and dk.shape == (0, 3) and dv.shape == (0, 4) and de.shape == (0,)
        assert np.array_equal(dS0, dSo)
        assert np.array_equal(O.linattn_backward_scan_ref(q, k, v, eta, S0, 5, mask, dO)[4], np.zeros((4, 3)))
