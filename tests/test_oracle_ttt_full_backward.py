"""Pins of the backward of the TTT-KVB chunk recurrence (GD, GD + L2, Muon with and without the
norm, with and without momentum; all three weights learning or W2 alone), CPU only.

Each pin takes a route other than the chain rule the oracle writes out: central finite differences
through the forward recurrence (ttt_scan_ref), torch's float64 autograd through a recurrence written
here with the inner gradient itself taken by autograd (a double backward), and the last-layer
backward, derived separately through the linear-attention reading."""
import numpy as np
import pytest

import oracle as O


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def problem(seed, N=9, d=3, m=4, scale=0.3):
    # without the norm a SwiGLU fast weight trained by GD grows quickly: its cases take small eta
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal((3, N, d))
    eta = scale * rng.standard_normal(N)
    W1, W3 = rng.standard_normal((2, m, d))
    W2 = rng.standard_normal((d, m))
    dO = rng.standard_normal((N, d))
    dWo = (rng.standard_normal((m, d)), rng.standard_normal((m, d)), rng.standard_normal((d, m)))
    return [q, k, v, eta, W1, W3, W2], dO, dWo


def fd_grads(args, f, h=1e-6):
    out = []
    for w in range(len(args)):
        fd = np.zeros_like(args[w])
        for idx in np.ndindex(*args[w].shape):
            a = [x.copy() for x in args]
            a[w][idx] += h
            lp = f(a)
            a[w][idx] -= 2 * h
            fd[idx] = (lp - f(a)) / (2 * h)
        out.append(fd)
    return out


def test_swiglu_apply_backward_matches_finite_differences():
    args, dO, _ = problem(1, N=5)
    q, W1, W3, W2 = args[0], args[4], args[5], args[6]
    got = O.swiglu_apply_backward(W1, W3, W2, q, dO)
    fd = fd_grads([q, W1, W3, W2], lambda a: float(np.sum(dO * O.swiglu_apply(a[1], a[2], a[3], a[0]))))
    for g, r in zip(got, fd):
        assert rel(g, r) < 1e-8


def test_chunk_gradients_backward_matches_finite_differences():
    # <Gb, chunk_gradients(W, K, V, eta)> differentiated numerically in every input
    rng = np.random.default_rng(2)
    args, _, Gb = problem(2, N=6)
    k, v, eta, W1, W3, W2 = args[1], args[2], args[3], args[4], args[5], args[6]
    got = O.chunk_gradients_backward(W1, W3, W2, k, v, eta, *Gb)

    def f(a):
        G = O.chunk_gradients(a[0], a[1], a[2], a[3], a[4], a[5])
        return float(sum(np.sum(x * y) for x, y in zip(G, Gb)))
    fd = fd_grads([W1, W3, W2, k, v, eta], f)
    for i, (g, r) in enumerate(zip(got, fd)):
        assert rel(g, r) < 1e-8, i


@pytest.mark.parametrize("shape", [(3, 5), (6, 4), (4, 4)])
def test_newton_schulz_backward_matches_finite_differences(shape):
    # wide, tall (run transposed) and square matrices through five cubic steps and the start's scaling
    rng = np.random.default_rng(7 + shape[0])
    U = rng.standard_normal(shape)
    G = rng.standard_normal(shape)
    got = O.newton_schulz_backward(U, 5, G)
    fd = fd_grads([U], lambda a: float(np.sum(G * O.newton_schulz(a[0], 5))))[0]
    assert rel(got, fd) < 1e-7
    # zero steps: only the scaling U / (|U| + eps)
    got0 = O.newton_schulz_backward(U, 0, G)
    fd0 = fd_grads([U], lambda a: float(np.sum(G * O.newton_schulz(a[0], 0))))[0]
    assert rel(got0, fd0) < 1e-7


def loss(a, chunk, mask, dO, dWo, upd, steps, ascent, beta, rule, last):
    o, W, _ = O.ttt_scan_ref(*a, chunk, mask, rule, momentum=beta, last_layer_only=last, update_chunks=upd,
                             inner_steps=steps, ascent=ascent)
    return float(np.sum(dO * o) + sum(np.sum(g * w) for g, w in zip(dWo, W)))


CASES = [
    # mask, chunk, strided flags, inner steps, ascent, momentum, rule
    (O.MASK_APPLY_THEN_UPDATE, 3, None, 1, False, 0.0, O.UPD_GD),
    (O.MASK_UPDATE_THEN_APPLY, 4, None, 1, False, 0.0, O.UPD_GD),
    (O.MASK_FULL, 9, None, 2, False, 0.0, O.UPD_GD),
    (O.MASK_STRIDED, 2, [1, 0, 1, 1, 0], 1, True, 0.0, O.UPD_GD),
    (O.MASK_APPLY_THEN_UPDATE, 3, None, 1, False, 0.0, O.UPD_GD_L2),
    (O.MASK_UPDATE_THEN_APPLY, 4, None, 2, True, 0.5, O.UPD_GD_L2),
    (O.MASK_FULL, 9, None, 1, False, 0.0, O.UPD_GD_L2),
    (O.MASK_STRIDED, 2, [0, 1, 1, 0, 1], 2, False, 0.9, O.UPD_GD_L2),
    (O.MASK_APPLY_THEN_UPDATE, 2, None, 2, False, 0.5, O.UPD_GD),
]


# Muon (five Newton-Schulz steps on the momentum or the gradient), with and without the norm, all
# three weights learning (last = False) or W2 alone
CASES_MUON = [
    (O.MASK_APPLY_THEN_UPDATE, 3, None, 1, False, 0.0, O.UPD_MUON_L2, False),
    (O.MASK_UPDATE_THEN_APPLY, 4, None, 2, True, 0.9, O.UPD_MUON_L2, False),
    (O.MASK_STRIDED, 2, [0, 1, 1, 0, 1], 1, False, 0.5, O.UPD_MUON, False),
    (O.MASK_FULL, 9, None, 1, False, 0.0, O.UPD_MUON, False),
    (O.MASK_APPLY_THEN_UPDATE, 2, None, 2, False, 0.9, O.UPD_MUON_L2, True),
    (O.MASK_UPDATE_THEN_APPLY, 3, None, 1, True, 0.0, O.UPD_MUON, True),
]


@pytest.mark.parametrize("mask,chunk,upd,steps,ascent,beta,rule,last",
                         [c + (False,) for c in CASES] + CASES_MUON)
def test_backward_matches_finite_differences(mask, chunk, upd, steps, ascent, beta, rule, last):
    # Muon's output has unit scale whatever the gradient's, so its cases take small eta too
    args, dO, dWo = problem(30 + mask + 7 * steps + rule, scale=0.3 if rule == O.UPD_GD_L2 else 0.03)
    got = O.ttt_backward_scan_ref(*args, chunk, mask, dO, dWo, upd, steps, ascent, beta, rule, last)
    fd = fd_grads(args, lambda a: loss(a, chunk, mask, dO, dWo, upd, steps, ascent, beta, rule, last))
    # Muon normalizes its input, so a small eta meets large curvature: central differences with
    # h = 1e-6 are good to about 1e-6 there (the double-autograd pin below is exact)
    tol = 1e-5 if rule in (O.UPD_MUON, O.UPD_MUON_L2) else 1e-7
    for i, (g, r) in enumerate(zip(list(got[:4]) + list(got[4]), fd)):
        assert rel(g, r) < tol, i


@pytest.mark.parametrize("mask,chunk,upd,steps,ascent,beta,rule", CASES[3:7])
def test_last_layer_only_matches_the_last_layer_backward(mask, chunk, upd, steps, ascent, beta, rule):
    # the last-layer backward is derived through linear attention over phi(q), phi(k); this one
    # through the chain rule of the recurrence with W1 and W3 frozen
    args, dO, dWo = problem(60 + mask)
    a = O.ttt_backward_scan_ref(*args, chunk, mask, dO, dWo, upd, steps, ascent, beta, rule, last_layer_only=True)
    b = O.ttt_lastlayer_backward_scan_ref(*args, chunk, mask, dO, dWo, upd, steps, ascent, momentum=beta, rule=rule)
    for x, y in zip(list(a[:4]) + list(a[4]), list(b[:4]) + list(b[4])):
        assert rel(x, y) < 1e-12


@pytest.mark.parametrize("mask,chunk,upd,beta,norm,muon", [(O.MASK_APPLY_THEN_UPDATE, 4, None, 0.0, False, False),
                                                           (O.MASK_UPDATE_THEN_APPLY, 5, None, 0.0, True, False),
                                                           (O.MASK_STRIDED, 3, [0, 1, 1, 0, 1], 0.9, True, False),
                                                           (O.MASK_APPLY_THEN_UPDATE, 4, None, 0.6, False, False),
                                                           (O.MASK_APPLY_THEN_UPDATE, 4, None, 0.9, True, True),
                                                           (O.MASK_UPDATE_THEN_APPLY, 5, None, 0.0, False, True)])
def test_backward_matches_double_autograd(mask, chunk, upd, beta, norm, muon):
    torch = pytest.importorskip("torch")
    N, d, m = 13, 4, 6
    args, dO, dWo = problem(80 + mask, N, d, m)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in args]
    tq, tk, tv, te = t[:4]

    def f(W, x):  # rows of the SwiGLU fast weight over rows of x
        return (torch.nn.functional.silu(x @ W[0].T) * (x @ W[1].T)) @ W[2].T

    def ns(U):  # five cubic Newton-Schulz steps on the side with the smaller Gram matrix
        X = U.T if U.shape[0] > U.shape[1] else U
        X = X / (torch.sqrt((X * X).sum()) + 1e-7)
        for _ in range(5):
            X = 1.5 * X - 0.5 * (X @ X.T) @ X
        return X.T if U.shape[0] > U.shape[1] else X

    post = mask == O.MASK_UPDATE_THEN_APPLY
    W, outs = list(t[4:]), []
    M = [torch.zeros_like(x) for x in W]
    for j, lo in enumerate(range(0, N, chunk)):
        hi = min(lo + chunk, N)
        if not post:
            outs.append(f(W, tq[lo:hi]))
        if upd is None or upd[j]:
            inner = -(te[lo:hi, None] * f(W, tk[lo:hi]) * tv[lo:hi]).sum()  # sum eta_i L(f(k_i), v_i)
            g = torch.autograd.grad(inner, W, create_graph=True)
            for i in range(3):
                M[i] = beta * M[i] + g[i]
                W[i] = W[i] - (ns(M[i]) if muon else M[i])
                if norm:  # rows to unit norm over the input dimension (eps never binds here)
                    W[i] = W[i] / torch.clamp(torch.sqrt((W[i] * W[i]).sum(dim=1, keepdim=True)), min=1e-6)
        if post:
            outs.append(f(W, tq[lo:hi]))
    L = (torch.cat(outs) * torch.tensor(dO)).sum() + sum((w * torch.tensor(g)).sum() for w, g in zip(W, dWo))
    L.backward()
    rule = (O.UPD_MUON_L2 if norm else O.UPD_MUON) if muon else (O.UPD_GD_L2 if norm else O.UPD_GD)
    got = O.ttt_backward_scan_ref(*args, chunk, mask, dO, dWo, upd, 1, False, beta, rule)
    for g, x in zip(list(got[:4]) + list(got[4]), t):
        assert rel(g, x.grad.numpy()) < 1e-12


def test_row_norm_floor():
    # a row whose norm is below the floor is divided by the floor, so its transpose is g / eps
    X = np.array([[3e-7, -4e-7], [3.0, 4.0]])
    g = np.array([[1.0, 2.0], [1.0, 2.0]])
    r = O.ttt_ref._row_norm_transpose(X, g)
    assert np.allclose(r[0], g[0] / O.ttt_ref.ROW_NORM_EPS)
    y = X[1] / 5.0
    assert np.allclose(r[1], (g[1] - y * (y @ g[1])) / 5.0)


def test_batched_wrapper():
    rng = np.random.default_rng(120)
    B, H, N, d, m = 2, 3, 7, 3, 5
    q, k, v, dO = rng.standard_normal((4, B, H, N, d))
    eta = 0.3 * rng.standard_normal((B, H, N))
    W1, W3 = rng.standard_normal((2, H, m, d))
    W2 = rng.standard_normal((H, d, m))
    dWo = (rng.standard_normal((B, H, m, d)), rng.standard_normal((B, H, m, d)), rng.standard_normal((B, H, d, m)))
    res = O.ttt_backward_ref(q, k, v, eta, W1, W3, W2, 3, O.MASK_APPLY_THEN_UPDATE, dO, dWo, rule=O.UPD_GD_L2)
    Wb = [np.broadcast_to(x[None], (B,) + x.shape).copy() for x in (W1, W3, W2)]
    rb = O.ttt_backward_ref(q, k, v, eta, *Wb, 3, O.MASK_APPLY_THEN_UPDATE, dO, dWo, rule=O.UPD_GD_L2)
    for b in range(B):
        for h in range(H):
            one = O.ttt_backward_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], W1[h], W3[h], W2[h], 3,
                                          O.MASK_APPLY_THEN_UPDATE, dO[b, h], tuple(x[b, h] for x in dWo),
                                          rule=O.UPD_GD_L2)
            for a, a2, o in zip(res[:4], rb[:4], one[:4]):
                assert rel(a[b, h], o) == 0.0 and rel(a2[b, h], o) == 0.0
            for i in range(3):
                assert rel(rb[4][i][b, h], one[4][i]) == 0.0
    for i in range(3):
        assert rel(res[4][i], rb[4][i].sum(axis=0)) < 1e-14


def test_without_updates_is_the_static_swiglu_layer():
    args, dO, _ = problem(130, N=8)
    dq, dk, dv, de, dW = O.ttt_backward_scan_ref(*args, 4, O.MASK_STRIDED, dO, None, [0, 0])
    assert not dk.any() and not dv.any() and not de.any()
    ref = O.swiglu_apply_backward(args[4], args[5], args[6], args[0], dO)
    assert rel(dq, ref[0]) < 1e-14
    for a, b in zip(dW, ref[1:]):
        assert rel(a, b) < 1e-14


def test_empty_sequence():
    args, _, dWo = problem(140)
    z = np.zeros((0, 3))
    dq, dk, dv, de, dW = O.ttt_backward_scan_ref(z, z, z, np.zeros(0), *args[4:], 4, O.MASK_APPLY_THEN_UPDATE, z,
                                                 dWo, rule=O.UPD_GD_L2)
    assert dq.shape == (0, 3) and de.shape == (0,)
    for a, b in zip(dW, dWo):
        assert np.array_equal(a, b)
