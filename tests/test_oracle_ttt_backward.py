"""Pins of the backward of the TTT-KVB layer with frozen W1, W3 (last layer only, plain GD), CPU only.

Each pin takes a route that does not go through the linear-attention reading the oracle is written
from: central finite differences through the chunk recurrence (ttt_scan_ref, which updates W2 with
the SwiGLU chunk gradients), and torch's autograd in float64 through a recurrence written here whose
inner gradient is itself taken by autograd (a double backward)."""
import numpy as np
import pytest

import oracle as O


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def problem(seed, N=9, d=3, m=4):
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal((3, N, d))
    eta = rng.standard_normal(N)
    W1, W3 = rng.standard_normal((2, m, d))
    W2 = rng.standard_normal((d, m))
    dO = rng.standard_normal((N, d))
    dWo = (rng.standard_normal((m, d)), rng.standard_normal((m, d)), rng.standard_normal((d, m)))
    return q, k, v, eta, W1, W3, W2, dO, dWo


def loss(q, k, v, eta, W1, W3, W2, chunk, mask, dO, dWo, upd, steps, ascent, beta=0.0, rule=O.UPD_GD):
    # the recurrence with momentum starting from zero; its final momentum is not part of the loss
    o, W, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, rule, momentum=beta, last_layer_only=True,
                             update_chunks=upd, inner_steps=steps, ascent=ascent)
    return float(np.sum(dO * o) + sum(np.sum(g * w) for g, w in zip(dWo, W)))


CASES = [(O.MASK_APPLY_THEN_UPDATE, 3, None, 1, False, 0.0), (O.MASK_UPDATE_THEN_APPLY, 4, None, 1, False, 0.0),
         (O.MASK_FULL, 9, None, 1, False, 0.0), (O.MASK_STRIDED, 2, [1, 0, 1, 1, 0], 1, False, 0.0),
         (O.MASK_APPLY_THEN_UPDATE, 4, None, 2, True, 0.0), (O.MASK_UPDATE_THEN_APPLY, 3, None, 3, False, 0.0),
         # momentum (W2 <- W2 - M, M <- beta M + g): every order, several steps, ascent, skipped chunks
         (O.MASK_APPLY_THEN_UPDATE, 2, None, 1, False, 0.9), (O.MASK_UPDATE_THEN_APPLY, 3, None, 2, True, 0.5),
         (O.MASK_FULL, 9, None, 3, False, 0.7), (O.MASK_STRIDED, 2, [0, 1, 1, 0, 1], 2, False, 0.9)]
# the L2 norm after each step (Variant 1 without Muon), alone and with momentum
CASES_L2 = [(O.MASK_APPLY_THEN_UPDATE, 3, None, 1, False, 0.0), (O.MASK_UPDATE_THEN_APPLY, 4, None, 2, True, 0.0),
            (O.MASK_FULL, 9, None, 1, False, 0.0), (O.MASK_STRIDED, 2, [1, 0, 1, 1, 0], 1, False, 0.0),
            (O.MASK_APPLY_THEN_UPDATE, 2, None, 1, False, 0.9), (O.MASK_UPDATE_THEN_APPLY, 3, None, 3, True, 0.5),
            (O.MASK_STRIDED, 2, [0, 1, 1, 0, 1], 2, False, 0.9)]


@pytest.mark.parametrize("mask,chunk,upd,steps,ascent,beta,rule",
                         [c + (O.UPD_GD,) for c in CASES] + [c + (O.UPD_GD_L2,) for c in CASES_L2])
def test_layer_backward_matches_finite_differences(mask, chunk, upd, steps, ascent, beta, rule):
    args = list(problem(90 + mask + 7 * steps + int(10 * beta) + 5 * rule))
    dO, dWo = args[7], args[8]
    args = args[:7]
    got = O.ttt_lastlayer_backward_scan_ref(*args, chunk, mask, dO, dWo, upd, steps, ascent, momentum=beta, rule=rule)
    grads = list(got[:4]) + list(got[4])
    h = 1e-6
    for which, g in enumerate(grads):
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(*args[which].shape):
            a = [x.copy() for x in args]
            a[which][idx] += h
            lp = loss(*a, chunk, mask, dO, dWo, upd, steps, ascent, beta, rule)
            a[which][idx] -= 2 * h
            lm = loss(*a, chunk, mask, dO, dWo, upd, steps, ascent, beta, rule)
            fd[idx] = (lp - lm) / (2 * h)
        assert rel(g, fd) < 1e-6, which


def test_momentum_zero_matches_the_linear_path():
    # beta = 0 through the momentum recurrence equals the plain path (which scales eta by the steps)
    args = list(problem(150))
    dO, dWo = args[7], args[8]
    a = O.ttt_lastlayer_backward_scan_ref(*args[:7], 3, O.MASK_APPLY_THEN_UPDATE, dO, dWo, None, 2, True)
    b = O.ttt_ref._recurrent_state_backward  # the recurrent path run directly with beta = 0 on the same features
    W1, W3 = args[4], args[5]
    phi = lambda x: O.silu(x @ W1.T) * (x @ W3.T)
    got = b(phi(args[0]), phi(args[1]), args[2], args[3], args[6], 3, O.MASK_APPLY_THEN_UPDATE, dO, dWo[2], None, 2,
            -1.0, 0.0, False)
    ref = O.linattn_backward_scan_ref(phi(args[0]), phi(args[1]), args[2], -2.0 * args[3], args[6], 3,
                                      O.MASK_APPLY_THEN_UPDATE, dO, dWo[2])
    for i, (x, y) in enumerate(zip(got, ref)):
        y = -2.0 * y if i == 3 else y
        assert rel(x, y) < 1e-12, i
    assert rel(a[2], got[2]) < 1e-12


@pytest.mark.parametrize("mask,chunk,upd,beta", [(O.MASK_APPLY_THEN_UPDATE, 4, None, 0.0),
                                                 (O.MASK_UPDATE_THEN_APPLY, 5, None, 0.0),
                                                 (O.MASK_STRIDED, 3, [0, 1, 1, 0, 1], 0.0),
                                                 (O.MASK_APPLY_THEN_UPDATE, 4, None, 0.9),
                                                 (O.MASK_STRIDED, 3, [1, 0, 1, 1, 0], 0.6)])
@pytest.mark.parametrize("norm", [False, True])
def test_layer_backward_matches_double_autograd(mask, chunk, upd, beta, norm):
    torch = pytest.importorskip("torch")
    N, d, m = 13, 4, 6
    q, k, v, eta, W1, W3, W2, dO, dWo = problem(110 + mask, N, d, m)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, eta, W1, W3, W2)]
    tq, tk, tv, te, t1, t3, t2 = t

    def f(W2_, x):  # rows of the SwiGLU fast weight over rows of x
        return (torch.nn.functional.silu(x @ t1.T) * (x @ t3.T)) @ W2_.T

    post = mask == O.MASK_UPDATE_THEN_APPLY
    W, outs, M = t2, [], torch.zeros_like(t2)
    for j, lo in enumerate(range(0, N, chunk)):
        hi = min(lo + chunk, N)
        if not post:
            outs.append(f(W, tq[lo:hi]))
        if upd is None or upd[j]:
            inner = -(te[lo:hi, None] * f(W, tk[lo:hi]) * tv[lo:hi]).sum()  # sum eta_i L(f(k_i), v_i)
            g, = torch.autograd.grad(inner, W, create_graph=True)
            M = beta * M + g
            W = W - M
            if norm:  # rows to unit norm over the input dimension (eps never binds here)
                W = W / torch.clamp(torch.sqrt((W * W).sum(dim=1, keepdim=True)), min=1e-6)
        if post:
            outs.append(f(W, tq[lo:hi]))
    L = (torch.cat(outs) * torch.tensor(dO)).sum()
    L = L + (t1 * torch.tensor(dWo[0])).sum() + (t3 * torch.tensor(dWo[1])).sum() + (W * torch.tensor(dWo[2])).sum()
    L.backward()
    got = O.ttt_lastlayer_backward_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, dO, dWo, upd, momentum=beta,
                                            rule=O.UPD_GD_L2 if norm else O.UPD_GD)
    for g, x in zip(list(got[:4]) + list(got[4]), t):
        assert rel(g, x.grad.numpy()) < 1e-12


def test_layer_backward_batched_wrapper():
    rng = np.random.default_rng(120)
    B, H, N, d, m = 2, 3, 7, 3, 5
    q, k, v, dO = rng.standard_normal((4, B, H, N, d))
    eta = rng.standard_normal((B, H, N))
    W1, W3 = rng.standard_normal((2, H, m, d))
    W2 = rng.standard_normal((H, d, m))
    dWo = (rng.standard_normal((B, H, m, d)), rng.standard_normal((B, H, m, d)), rng.standard_normal((B, H, d, m)))
    res = O.ttt_lastlayer_backward_ref(q, k, v, eta, W1, W3, W2, 3, O.MASK_APPLY_THEN_UPDATE, dO, dWo)
    # per-(batch, head) weights: each scan on its own; per-head weights: the same, summed over the batch
    Wb = [np.broadcast_to(x[None], (B,) + x.shape).copy() for x in (W1, W3, W2)]
    rb = O.ttt_lastlayer_backward_ref(q, k, v, eta, *Wb, 3, O.MASK_APPLY_THEN_UPDATE, dO, dWo)
    for b in range(B):
        for h in range(H):
            one = O.ttt_lastlayer_backward_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], W1[h], W3[h], W2[h], 3,
                                                    O.MASK_APPLY_THEN_UPDATE, dO[b, h], tuple(x[b, h] for x in dWo))
            for a, a2, o in zip(res[:4], rb[:4], one[:4]):
                assert rel(a[b, h], o) == 0.0 and rel(a2[b, h], o) == 0.0
            for i in range(3):
                assert rel(rb[4][i][b, h], one[4][i]) == 0.0
    for i in range(3):
        assert rel(res[4][i], rb[4][i].sum(axis=0)) < 1e-14


def test_layer_backward_without_updates_is_the_static_mlp():
    # no chunk updates: o = f_W0(q) for every token, so k, v and eta get no gradient and the weight
    # gradients are those of a fixed SwiGLU layer, whose W2 gradient is dO^T phi(q)
    q, k, v, eta, W1, W3, W2, dO, _ = problem(130, N=8)
    dq, dk, dv, de, (dW1, dW3, dW2) = O.ttt_lastlayer_backward_scan_ref(q, k, v, eta, W1, W3, W2, 4, O.MASK_STRIDED,
                                                                         dO, None, [0, 0])
    assert not dk.any() and not dv.any() and not de.any()
    phi = O.silu(q @ W1.T) * (q @ W3.T)
    assert rel(dW2, dO.T @ phi) < 1e-14


def test_layer_backward_empty_sequence():
    rng = np.random.default_rng(140)
    z = np.zeros((0, 3))
    W1, W3 = rng.standard_normal((2, 4, 3))
    W2 = rng.standard_normal((3, 4))
    dWo = (rng.standard_normal((4, 3)), rng.standard_normal((4, 3)), rng.standard_normal((3, 4)))
    dq, dk, dv, de, dW = O.ttt_lastlayer_backward_scan_ref(z, z, z, np.zeros(0), W1, W3, W2, 4,
                                                           O.MASK_APPLY_THEN_UPDATE, z, dWo)
    assert dq.shape == dk.shape == dv.shape == (0, 3) and de.shape == (0,)
    for a, b in zip(dW, dWo):
        assert np.array_equal(a, b)
