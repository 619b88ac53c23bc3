"""Pins of the fp64 oracle against what the pages and mathematics fix (CPU only).

Every expected value here is computed by a route independent of the oracle's own formulas:
per-token scalar loops of Eq. (3), central finite differences of the Eq. (2)/(4) loss, the SVD
of the matrix for Newton-Schulz, and the closed forms of the linear and last-layer reductions
(TTT-as-LA Thm. 5.2/5.3, App. H).  A dropped term, a flipped sign, a wrong index or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# independent helpers (scalar loops, finite differences, SVD)

def f_token(W1, W3, W2, x):
    """f_W(x) = W2 [SiLU(W1 x) o (W3 x)] by explicit loops (LaCT notes Eq. (3))."""
    m, d = W1.shape
    hid = []
    for r in range(m):
        a = sum(W1[r, c] * x[c] for c in range(d))
        u = sum(W3[r, c] * x[c] for c in range(d))
        hid.append(a / (1.0 + math.exp(-a)) * u)
    return np.array([sum(W2[e, r] * hid[r] for r in range(m)) for e in range(W2.shape[0])])


def chunk_loss(W1, W3, W2, K, V, eta):
    """sum_i eta_i * L(f_W(k_i), v_i) with L = -f^T v (LaCT notes Eqs. (2), (4))."""
    tot = 0.0
    for i in range(K.shape[0]):
        f = f_token(W1, W3, W2, K[i])
        tot += eta[i] * (-float(np.dot(f, V[i])))
    return tot


def fd_gradients(W1, W3, W2, K, V, eta, h=1e-5):
    Ws = [W1.copy(), W3.copy(), W2.copy()]
    grads = []
    for wi in range(3):
        g = np.zeros_like(Ws[wi])
        for idx in np.ndindex(*Ws[wi].shape):
            old = Ws[wi][idx]
            Ws[wi][idx] = old + h
            lp = chunk_loss(*Ws, K, V, eta)
            Ws[wi][idx] = old - h
            lm = chunk_loss(*Ws, K, V, eta)
            Ws[wi][idx] = old
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads  # G1, G3, G2


def ns_via_svd(U, iters, eps=1e-7):
    """Newton-Schulz written on the singular values: U = P diag(s) Q^T, and the cubic
    x <- 1.5 x - 0.5 x^3 acts on each normalised singular value separately."""
    P, s, Qt = np.linalg.svd(U, full_matrices=False)
    x = s / (np.sqrt(np.sum(s * s)) + eps)
    for _ in range(iters):
        x = 1.5 * x - 0.5 * x ** 3
    return (P * x) @ Qt


def rownorm_loops(W, eps=1e-6):
    out = np.empty_like(W)
    for r in range(W.shape[0]):
        n = math.sqrt(sum(float(w) * float(w) for w in W[r]))
        out[r] = W[r] / max(n, eps)
    return out


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def tiny_problem(seed, N=8, d=4, m=6, eta_scale=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, d)) / math.sqrt(d)
    k = rng.standard_normal((N, d)) / math.sqrt(d)
    v = rng.standard_normal((N, d)) / math.sqrt(d)
    eta = eta_scale * np.log1p(np.exp(rng.standard_normal(N)))
    W1 = rng.standard_normal((m, d)) / math.sqrt(d)
    W3 = rng.standard_normal((m, d)) / math.sqrt(d)
    W2 = rng.standard_normal((d, m)) / math.sqrt(d)
    return q, k, v, eta, W1, W3, W2


# ----------------------------------------------------------------------------------------------
# Eq. (3) forward and Eqs. (2)/(4) gradients

def test_swiglu_apply_matches_scalar_loops():
    q, k, v, eta, W1, W3, W2 = tiny_problem(1)
    got = O.swiglu_apply(W1, W3, W2, q)
    want = np.stack([f_token(W1, W3, W2, x) for x in q])
    assert rel(got, want) < 1e-13


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chunk_gradients_match_finite_differences(seed):
    q, k, v, eta, W1, W3, W2 = tiny_problem(seed, N=5)
    eta = eta - 0.1  # includes negative rates (gradient ascent is allowed)
    G1, G3, G2 = O.chunk_gradients(W1, W3, W2, k, v, eta)
    F1, F3, F2 = fd_gradients(W1, W3, W2, k, v, eta)
    assert rel(G1, F1) < 1e-7
    assert rel(G3, F3) < 1e-7
    assert rel(G2, F2) < 1e-7


def test_last_layer_gradient_closed_form():
    """TTT-as-LA App. E.2: the last layer's gradient is -phi(K)^T (eta V), phi = SiLU(W1 k) o W3 k."""
    q, k, v, eta, W1, W3, W2 = tiny_problem(3)
    phi = np.stack([[a / (1 + math.exp(-a)) * u for a, u in zip(W1 @ x, W3 @ x)] for x in k])
    want = -(eta[:, None] * v).T @ phi
    assert rel(O.chunk_gradients(W1, W3, W2, k, v, eta)[2], want) < 1e-13


# ----------------------------------------------------------------------------------------------
# Newton-Schulz (Eq. (6))

def test_newton_schulz_converges_to_polar_factor():
    rng = np.random.default_rng(7)
    P, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    Q, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    s = np.linspace(1.0, 2.5, 6)
    U = (P * s) @ Q[:6]
    want = P @ Q[:6]
    assert rel(O.newton_schulz(U, 100), want) < 1e-10
    assert rel(O.newton_schulz(U.T, 100), want.T) < 1e-10


@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (7, 7)])
def test_newton_schulz_five_steps_on_singular_values(shape):
    rng = np.random.default_rng(11)
    U = rng.standard_normal(shape)
    assert rel(O.newton_schulz(U, 5), ns_via_svd(U, 5)) < 1e-12
    assert rel(O.newton_schulz(U, 1), ns_via_svd(U, 1)) < 1e-13


def test_newton_schulz_invariants():
    rng = np.random.default_rng(5)
    U = rng.standard_normal((6, 10))
    base = O.newton_schulz(U, 5)
    assert rel(O.newton_schulz(3.7 * U, 5), base) < 1e-6  # eps makes scale invariance approximate
    assert rel(O.newton_schulz(-U, 5), -base) < 1e-14
    assert rel(O.newton_schulz(U.T, 5), base.T) < 1e-13
    P, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    Q, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    assert rel(O.newton_schulz(P @ U @ Q, 5), P @ base @ Q) < 1e-12
    assert np.all(O.newton_schulz(np.zeros((3, 4)), 5) == 0.0)


# ----------------------------------------------------------------------------------------------
# L2-Normalize (Eq. (5))

def test_l2_normalize_rows_definition():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((5, 7))
    got = O.l2_normalize_rows(W)
    assert rel(got, rownorm_loops(W)) < 1e-14
    assert np.allclose(np.linalg.norm(got, axis=1), 1.0, atol=1e-14)
    assert rel(O.l2_normalize_rows(got), got) < 1e-14
    # columns are not normalised
    assert not np.allclose(np.linalg.norm(got, axis=0), 1.0)


# ----------------------------------------------------------------------------------------------
# an independent stepper: FD gradients + SVD Newton-Schulz + loop row norms, following the
# order of the mask (LaCT notes section 1.1, Eq. (10))

def stepper(q, k, v, eta, W1, W3, W2, chunk, mask, rule, ns_iters=5, beta=0.0, last_only=False,
            upd=None, M0=None):
    W = [W1.copy(), W3.copy(), W2.copy()]
    M = [np.zeros_like(x) for x in W] if M0 is None else [x.copy() for x in M0]
    N = q.shape[0]
    o = np.zeros((N, W2.shape[0]))
    for j, lo in enumerate(range(0, N, chunk)):
        hi = min(lo + chunk, N)
        first = mask in (O.MASK_APPLY_THEN_UPDATE, O.MASK_STRIDED)
        if first:
            o[lo:hi] = np.stack([f_token(*W, x) for x in q[lo:hi]])
        if mask != O.MASK_STRIDED or upd[j]:
            G = fd_gradients(*W, k[lo:hi], v[lo:hi], eta[lo:hi])
            for i in ([2] if last_only else [0, 1, 2]):
                U = G[i]
                if beta:
                    M[i] = beta * M[i] + G[i]
                    U = M[i]
                if rule in (O.UPD_MUON_L2, O.UPD_MUON):
                    U = ns_via_svd(U, ns_iters)
                W[i] = W[i] - U
                if rule in (O.UPD_GD_L2, O.UPD_MUON_L2):
                    W[i] = rownorm_loops(W[i])
        if not first:
            o[lo:hi] = np.stack([f_token(*W, x) for x in q[lo:hi]])
    return o, W, M


CASES = [
    # (mask, rule, beta, last_only, chunk)
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, 0.0, False, 3),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON_L2, 0.9, False, 3),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, 0.0, False, 4),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_GD_L2, 0.0, False, 3),
    (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, 0.0, True, 3),
    (O.MASK_STRIDED, O.UPD_MUON_L2, 0.0, False, 3),
    (O.MASK_FULL, O.UPD_GD_L2, 0.0, False, 8),
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, 0.5, False, 3),
]


@pytest.mark.parametrize("mask,rule,beta,last_only,chunk", CASES)
def test_scan_matches_independent_stepper(mask, rule, beta, last_only, chunk):
    q, k, v, eta, W1, W3, W2 = tiny_problem(21, N=8)
    upd = [1, 1, 0] if mask == O.MASK_STRIDED else None
    o, W, M = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, rule, 5, beta, last_only, upd)
    o2, W2s, M2 = stepper(q, k, v, eta, W1, W3, W2, chunk, mask, rule, 5, beta, last_only, upd)
    assert rel(o, o2) < 1e-6
    for a, b in zip(W, W2s):
        assert rel(a, b) < 1e-6
    if beta:
        for a, b in zip(M, M2):
            assert rel(a, b) < 1e-6


def test_first_chunk_apply_then_update_uses_initial_weights():
    q, k, v, eta, W1, W3, W2 = tiny_problem(4, N=8)
    o, _, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    want = np.stack([f_token(W1, W3, W2, x) for x in q[:4]])
    assert rel(o[:4], want) < 1e-13


def test_l2_rows_unit_after_update():
    q, k, v, eta, W1, W3, W2 = tiny_problem(6, N=8)
    _, W, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    assert np.allclose(np.linalg.norm(W[0], axis=1), 1.0, atol=1e-14)  # W1 rows over d
    assert np.allclose(np.linalg.norm(W[1], axis=1), 1.0, atol=1e-14)  # W3 rows over d
    assert np.allclose(np.linalg.norm(W[2], axis=1), 1.0, atol=1e-14)  # W2 rows over m


# ----------------------------------------------------------------------------------------------
# closed forms of the reductions (TTT-as-LA Thm. 5.2 / 5.3, App. H)

def visible(t, s, chunk, mask, upd=None):
    """Does token s's key/value reach token t's output under the mask?"""
    ct, cs = t // chunk, s // chunk
    if mask == O.MASK_FULL:
        return True
    if mask == O.MASK_TOKEN_CAUSAL:
        return s <= t
    if mask == O.MASK_UPDATE_THEN_APPLY:
        return cs <= ct
    if mask == O.MASK_APPLY_THEN_UPDATE:
        return cs < ct
    if mask == O.MASK_STRIDED:
        return cs < ct and bool(upd[cs])
    raise ValueError


@pytest.mark.parametrize("mask,chunk,N", [
    (O.MASK_APPLY_THEN_UPDATE, 4, 13), (O.MASK_UPDATE_THEN_APPLY, 4, 13), (O.MASK_TOKEN_CAUSAL, 4, 13),
    (O.MASK_FULL, 13, 13), (O.MASK_STRIDED, 4, 16), (O.MASK_APPLY_THEN_UPDATE, 1, 6),
])
def test_linear_model_closed_form(mask, chunk, N):
    """o_t = S0 q_t + sum_{s visible} eta_s v_s (k_s . q_t)  (Thm. 5.2; LA-to-TTT causal form)."""
    rng = np.random.default_rng(N + chunk + mask)
    dk, dv = 3, 5
    q = rng.standard_normal((N, dk))
    k = rng.standard_normal((N, dk))
    v = rng.standard_normal((N, dv))
    eta = rng.standard_normal(N)
    S0 = rng.standard_normal((dv, dk))
    upd = [1, 0, 1, 0] if mask == O.MASK_STRIDED else None
    o, S = O.linattn_scan_ref(q, k, v, eta, S0, chunk, mask, upd)
    for t in range(N):
        want = [sum(S0[e, c] * q[t, c] for c in range(dk)) for e in range(dv)]
        for s in range(N):
            if visible(t, s, chunk, mask, upd):
                dot = sum(k[s, c] * q[t, c] for c in range(dk))
                for e in range(dv):
                    want[e] += eta[s] * v[s, e] * dot
        assert rel(o[t], np.array(want)) < 1e-12
    # final state sums every updating chunk
    Sw = S0.copy()
    for s in range(N):
        if mask != O.MASK_STRIDED or upd[s // chunk]:
            Sw += eta[s] * np.outer(v[s], k[s])
    assert rel(S, Sw) < 1e-12


def test_linear_full_mask_is_bidirectional_attention_form():
    rng = np.random.default_rng(9)
    N, d = 10, 4
    q, k, v = rng.standard_normal((3, N, d))
    eta = rng.random(N)
    S0 = rng.standard_normal((d, d))
    o, _ = O.linattn_scan_ref(q, k, v, eta, S0, N, O.MASK_FULL)
    assert rel(o, q @ S0.T + (q @ k.T) @ (eta[:, None] * v)) < 1e-13


def test_linear_sign_flip_negates_accumulated_term():
    """TTT-as-LA Sec. 5.2: gradient ascent flips the sign of the effective value."""
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((3, 12, 4))
    eta = rng.random(12)
    S0 = rng.standard_normal((4, 4))
    o1, _ = O.linattn_scan_ref(q, k, v, eta, S0, 4, O.MASK_APPLY_THEN_UPDATE)
    o2, _ = O.linattn_scan_ref(q, k, v, -eta, S0, 4, O.MASK_APPLY_THEN_UPDATE)
    base = q @ S0.T
    assert rel(o1 - base, -(o2 - base)) < 1e-13


def phi_rows(W1, W3, X):
    return np.stack([[a / (1 + math.exp(-a)) * u for a, u in zip(W1 @ x, W3 @ x)] for x in X])


@pytest.mark.parametrize("mask", [O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY, O.MASK_FULL])
@pytest.mark.parametrize("beta", [0.0, 0.9])
def test_last_layer_gd_momentum_parallel_form(mask, beta):
    """Static kernel phi, plain GD on the last layer with chunk momentum: the masked parallel form
    O = phi(Q) W2^T + sum_{i <= J(t)} c(J, i) (phi(Q) phi(K_i)^T) diag(eta_i) V_i with
    c(J, i) = sum_{j=i..J} beta^(j-i)  (TTT-as-LA Thm. 5.3 / App. H, written per chunk)."""
    N, chunk = 12, 4
    if mask == O.MASK_FULL:
        chunk = N
    q, k, v, eta, W1, W3, W2 = tiny_problem(30, N=N)
    o, W, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, O.UPD_GD, 5, beta, True)
    PQ, PK = phi_rows(W1, W3, q), phi_rows(W1, W3, k)
    want = PQ @ W2.T
    for t in range(N):
        J = t // chunk - (1 if mask == O.MASK_APPLY_THEN_UPDATE else 0)
        for s in range(N):
            i = s // chunk
            if i <= J:
                c = sum(beta ** (j - i) for j in range(i, J + 1))
                want[t] += c * eta[s] * np.dot(PQ[t], PK[s]) * v[s]
    assert rel(o, want) < 1e-12
    assert rel(W[0], W1) == 0.0 and rel(W[1], W3) == 0.0  # only the last layer moves


def test_weight_norm_breaks_parallel_form():
    """Negative control, TTT-as-LA App. I.2: with L2-Normalize the state is not a sum over history."""
    N, chunk = 12, 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(31, N=N, eta_scale=2.0)
    o, _, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, 5,
                             0.0, True)
    PQ, PK = phi_rows(W1, W3, q), phi_rows(W1, W3, k)
    par = PQ @ W2.T
    for t in range(N):
        for s in range(N):
            if s // chunk < t // chunk:
                par[t] += eta[s] * np.dot(PQ[t], PK[s]) * v[s]
    assert rel(o, par) > 1e-2


def test_full_mask_all_layers_gd_is_update_then_apply():
    """Thm. 5.1 with one chunk: o = W2' phi'(q), where W' = W - G and G is the chunk gradient
    (taken here by finite differences)."""
    q, k, v, eta, W1, W3, W2 = tiny_problem(32, N=6)
    o, W, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, 6, O.MASK_FULL, O.UPD_GD)
    G1, G3, G2 = fd_gradients(W1, W3, W2, k, v, eta)
    want = np.stack([f_token(W1 - G1, W3 - G3, W2 - G2, x) for x in q])
    assert rel(o, want) < 1e-8


# ----------------------------------------------------------------------------------------------
# order relations, chaining, degenerate cases

def test_update_then_apply_is_apply_then_update_shifted_by_one_chunk():
    """Both orders share the W_j sequence; UTA reads W_j for chunk j, ATU reads it for chunk j+1."""
    N, chunk = 12, 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(33, N=N)
    o_uta, W_uta, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, O.MASK_UPDATE_THEN_APPLY, O.UPD_GD_L2)
    q_shift = np.concatenate([np.zeros((chunk, q.shape[1])), q[:-chunk]])
    o_atu, W_atu, _ = O.ttt_scan_ref(q_shift, k, v, eta, W1, W3, W2, chunk, O.MASK_APPLY_THEN_UPDATE,
                                     O.UPD_GD_L2)
    assert rel(o_atu[chunk:], o_uta[:-chunk]) < 1e-13
    for a, b in zip(W_uta, W_atu):
        assert rel(a, b) < 1e-14


@pytest.mark.parametrize("rule,beta", [(O.UPD_GD_L2, 0.0), (O.UPD_MUON_L2, 0.9)])
def test_two_calls_equal_one(rule, beta):
    N, chunk = 12, 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(34, N=N)
    mask = O.MASK_APPLY_THEN_UPDATE
    o, W, M = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, rule, 5, beta)
    oa, Wa, Ma = O.ttt_scan_ref(q[:8], k[:8], v[:8], eta[:8], W1, W3, W2, chunk, mask, rule, 5, beta)
    ob, Wb, Mb = O.ttt_scan_ref(q[8:], k[8:], v[8:], eta[8:], *Wa, chunk, mask, rule, 5, beta, M=Ma)
    assert rel(np.concatenate([oa, ob]), o) < 1e-14
    for a, b in zip(Wb, W):
        assert rel(a, b) < 1e-14


def test_strided_degenerate_flags():
    N, chunk = 12, 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(35, N=N)
    o_all, W_all, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, O.MASK_STRIDED, O.UPD_GD_L2,
                                     update_chunks=[1, 1, 1])
    o_atu, W_atu, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    assert rel(o_all, o_atu) == 0.0
    o_none, W_none, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, O.MASK_STRIDED, O.UPD_GD_L2,
                                       update_chunks=[0, 0, 0])
    assert rel(o_none, np.stack([f_token(W1, W3, W2, x) for x in q])) < 1e-13
    assert rel(W_none[2], W2) == 0.0


def test_zero_eta_leaves_weights_unchanged_under_gd():
    q, k, v, eta, W1, W3, W2 = tiny_problem(36, N=8)
    o, W, _ = O.ttt_scan_ref(q, k, v, 0 * eta, W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD)
    assert rel(W[0], W1) == 0.0 and rel(W[2], W2) == 0.0
    assert rel(o, np.stack([f_token(W1, W3, W2, x) for x in q])) < 1e-13


def test_forward_ref_batches_match_scans():
    q, k, v, eta, W1, W3, W2 = tiny_problem(37, N=8)
    Q = np.stack([np.stack([q, k]), np.stack([v, q])])
    K = np.stack([np.stack([k, v]), np.stack([q, k])])
    V = np.stack([np.stack([v, q]), np.stack([k, v])])
    E = np.stack([np.stack([eta, eta[::-1]]), np.stack([eta * 2, eta])])
    Ws = [np.stack([W, W * 0.5]) for W in (W1, W3, W2)]
    o, W, _ = O.ttt_forward_ref(Q, K, V, E, *Ws, 4, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    for b in range(2):
        for h in range(2):
            ob, Wb, _ = O.ttt_scan_ref(Q[b, h], K[b, h], V[b, h], E[b, h], Ws[0][h], Ws[1][h], Ws[2][h], 4,
                                       O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
            assert rel(o[b, h], ob) == 0.0


def test_eq1_intensity_table():
    with open(os.path.join(GOLDEN, "eq1_intensity.json")) as f:
        g = json.load(f)
    for row in g["rows"]:
        assert abs(O.gemm_intensity(row["h"], row["b"]) - row["r"]) <= g["rounding"]


# ----------------------------------------------------------------------------------------------
# inner-loop variants: several gradient steps per chunk (TTT-as-LA Sec. 4.1) and gradient ascent
# (TTT-as-LA Sec. 4.2; Sec. 5.2 states that ascent only flips the sign of the step, +eta for -eta)

@pytest.mark.parametrize("rule,beta,last", [(O.UPD_GD, 0.0, False), (O.UPD_GD_L2, 0.0, False),
                                            (O.UPD_MUON_L2, 0.9, False), (O.UPD_MUON, 0.5, True)])
def test_ascent_is_descent_with_negated_eta(rule, beta, last):
    """The chunk gradient is linear in eta and the Newton-Schulz polynomial is odd, so an ascent
    step with eta is a descent step with -eta, for every rule, with momentum; exactly, since every
    operation commutes with the sign."""
    q, k, v, eta, W1, W3, W2 = tiny_problem(40, N=12)
    for mask in (O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY):
        oa, Wa, Ma = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, 4, mask, rule, 3, beta, last, ascent=True)
        od, Wd, Md = O.ttt_scan_ref(q, k, v, -eta, W1, W3, W2, 4, mask, rule, 3, beta, last)
        assert rel(oa, od) == 0.0
        for a, b in zip(Wa + Ma, Wd + Md):
            assert np.array_equal(a, b)
        o_desc, W_desc, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, 4, mask, rule, 3, beta, last)
        assert rel(Wa[2], W_desc[2]) > 1e-3  # and it is not descent


@pytest.mark.parametrize("rule,beta", [(O.UPD_GD, 0.0), (O.UPD_GD_L2, 0.0), (O.UPD_MUON_L2, 0.9)])
def test_inner_steps_equal_repeated_chunks(rule, beta):
    """n inner steps on one chunk take the path of n consecutive chunks that hold the same tokens,
    one step each: every step's gradient is taken at the weights the previous step left (a step
    that reused the first gradient, or a loop that ran once, would differ)."""
    c = 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(41, N=c)
    rep = lambda x, n: np.concatenate([x] * n)
    for n in (2, 3):
        _, Wi, Mi = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, c, O.MASK_UPDATE_THEN_APPLY, rule, 3, beta,
                                   inner_steps=n)
        _, Wr, Mr = O.ttt_scan_ref(rep(q, n), rep(k, n), rep(v, n), rep(eta, n), W1, W3, W2, c,
                                   O.MASK_UPDATE_THEN_APPLY, rule, 3, beta)
        for a, b in zip(Wi + Mi, Wr + Mr):
            assert rel(a, b) < 1e-14
        _, W1step, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, c, O.MASK_UPDATE_THEN_APPLY, rule, 3, beta)
        assert rel(Wi[2], W1step[2]) > 1e-4


def test_last_layer_gd_inner_steps_scale_eta():
    """With W2 alone updated under plain GD, its chunk gradient -sum_i eta_i v_i h(k_i)^T does not
    depend on W2 (TTT-as-LA Thm. 5.1), so n inner steps are one step with n eta: a closed form.
    The apply order is checked through the outputs of both orders."""
    q, k, v, eta, W1, W3, W2 = tiny_problem(42, N=12)
    for mask in (O.MASK_APPLY_THEN_UPDATE, O.MASK_UPDATE_THEN_APPLY):
        on, Wn, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, 4, mask, O.UPD_GD, last_layer_only=True,
                                   inner_steps=3)
        o1, W1s, _ = O.ttt_scan_ref(q, k, v, 3 * eta, W1, W3, W2, 4, mask, O.UPD_GD, last_layer_only=True)
        assert rel(on, o1) < 1e-13
        assert rel(Wn[2], W1s[2]) < 1e-13
        assert rel(Wn[0], W1) == 0.0 and rel(Wn[1], W3) == 0.0


# ----------------------------------------------------------------------------------------------
# the batched wrappers: every (batch, head) slice with its own state, each against an independent
# route (brute-force sums for the linear model, the finite-difference stepper for the layer)

@pytest.mark.parametrize("mask,chunk,N", [
    (O.MASK_APPLY_THEN_UPDATE, 4, 13), (O.MASK_UPDATE_THEN_APPLY, 3, 13), (O.MASK_TOKEN_CAUSAL, 4, 11),
    (O.MASK_FULL, 9, 9), (O.MASK_STRIDED, 4, 14),
])
def test_linattn_forward_ref_slices_closed_form(mask, chunk, N):
    """linattn_forward_ref over B x H slices, each with its own S0 and d_k != d_v, against
    o_t = S0[b,h] q_t + sum_{s visible} eta_s v_s (k_s . q_t) per slice (Thm. 5.2), and its final
    states against S0[b,h] + sum over updating chunks of eta_s v_s k_s^T."""
    B, H, dk, dv = 2, 3, 3, 5
    rng = np.random.default_rng(100 + 7 * mask + N)
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    eta = rng.standard_normal((B, H, N))
    S0 = rng.standard_normal((B, H, dv, dk))
    upd = [1, 0, 1, 1] if mask == O.MASK_STRIDED else None
    o, S = O.linattn_forward_ref(q, k, v, eta, chunk, mask, S0, upd)
    assert o.shape == (B, H, N, dv) and S.shape == (B, H, dv, dk)
    for b in range(B):
        for h in range(H):
            for t in range(N):
                want = [sum(S0[b, h, e, c] * q[b, h, t, c] for c in range(dk)) for e in range(dv)]
                for s_ in range(N):
                    if visible(t, s_, chunk, mask, upd):
                        dot = sum(k[b, h, s_, c] * q[b, h, t, c] for c in range(dk))
                        for e in range(dv):
                            want[e] += eta[b, h, s_] * v[b, h, s_, e] * dot
                assert rel(o[b, h, t], np.array(want)) < 1e-12, (b, h, t)
            Sw = S0[b, h].copy()
            for s_ in range(N):
                if mask != O.MASK_STRIDED or upd[s_ // chunk]:
                    Sw += eta[b, h, s_] * np.outer(v[b, h, s_], k[b, h, s_])
            assert rel(S[b, h], Sw) < 1e-12, (b, h)
    # without S0 the state starts at zero; `slices` computes only the listed slices
    o0, S0_ = O.linattn_forward_ref(q, k, v, eta, chunk, mask, None, upd, slices=[(1, 2)])
    o1, _ = O.linattn_forward_ref(q[1:, 2:], k[1:, 2:], v[1:, 2:], eta[1:, 2:], chunk, mask,
                                  np.zeros((1, 1, dv, dk)), upd)
    assert rel(o0[1, 2], o1[0, 0]) == 0.0
    assert not o0[0].any() and not o0[1, :2].any() and not S0_[0].any()


@pytest.mark.parametrize("rule,beta,mask", [(O.UPD_GD_L2, 0.0, O.MASK_APPLY_THEN_UPDATE),
                                            (O.UPD_MUON_L2, 0.9, O.MASK_UPDATE_THEN_APPLY),
                                            (O.UPD_GD, 0.5, O.MASK_APPLY_THEN_UPDATE)])
def test_forward_ref_per_batch_weights_and_momentum(rule, beta, mask):
    """ttt_forward_ref with W0 given per (batch, head) and a non-zero starting momentum M per
    (batch, head): each slice against the independent finite-difference stepper started from that
    slice's own W0 and M; `slices` computes only the listed slices."""
    B, H, N, chunk = 2, 2, 8, 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(40, N=N)
    rng = np.random.default_rng(41)
    Q = np.stack([np.stack([q, k]), np.stack([v, q])])
    K = np.stack([np.stack([k, v]), np.stack([q, k])])
    V = np.stack([np.stack([v, q]), np.stack([k, v])])
    E = np.stack([np.stack([eta, eta[::-1]]), np.stack([eta * 2, eta])])
    Ws = [np.stack([np.stack([W * (1 + 0.1 * (2 * b + h)) for h in range(H)]) for b in range(B)])
          for W in (W1, W3, W2)]
    M = tuple(0.05 * rng.standard_normal(W.shape) for W in Ws)
    o, W, Mo = O.ttt_forward_ref(Q, K, V, E, *Ws, chunk, mask, rule, 5, beta, M=M)
    for b in range(B):
        for h in range(H):
            o2, W2s, M2 = stepper(Q[b, h], K[b, h], V[b, h], E[b, h], Ws[0][b, h], Ws[1][b, h], Ws[2][b, h], chunk,
                                  mask, rule, 5, beta, M0=[x[b, h] for x in M])
            assert rel(o[b, h], o2) < 1e-6, (b, h)
            for i in range(3):
                assert rel(W[i][b, h], W2s[i]) < 1e-6, (b, h, i)
                if beta:
                    assert rel(Mo[i][b, h], M2[i]) < 1e-6, (b, h, i)
    o1, W1s, _ = O.ttt_forward_ref(Q, K, V, E, *Ws, chunk, mask, rule, 5, beta, M=M, slices=[(1, 0)])
    assert rel(o1[1, 0], o[1, 0]) == 0.0 and rel(W1s[2][1, 0], W[2][1, 0]) == 0.0
    assert not o1[0].any() and not o1[1, 1].any() and not W1s[0][0].any()


@pytest.mark.parametrize("mask,beta,upd", [(O.MASK_APPLY_THEN_UPDATE, 0.9, None), (O.MASK_UPDATE_THEN_APPLY, 0.0, None),
                                           (O.MASK_STRIDED, 0.9, [1, 0, 1, 1])])
def test_last_layer_muon_parallel_form(mask, beta, upd):
    """Variant 2 of the paper's ablation (Sec. 6.1 Steps 1-2, Table 2): only W2 learns, Muon and
    momentum stay, no weight norm.  The chunk gradient of W2 is -phi(K)^T (eta V) (App. E.2): it
    depends on the frozen features and on v, never on W2, so the recurrence is a parallel prefix over
    chunks (Sec. 6.2): every chunk's gradient up front, the momentum as a linear scan, Muon on each
    chunk's momentum, W2 as W2_0 minus the prefix sum of those.  Built here from the finite-difference
    gradient, a loop momentum and the SVD form of Newton-Schulz, it must equal the oracle's recurrence;
    Muon applied to each chunk's outer product before the sum (App. E.3 read literally) must not,
    because Muon is not additive."""
    N, chunk = 12, 4
    q, k, v, eta, W1, W3, W2 = tiny_problem(42, N=N)
    o, W, _ = O.ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, O.UPD_MUON, 5, beta, True, upd)
    nch = N // chunk
    updates = [mask != O.MASK_STRIDED or upd[j] for j in range(nch)]
    G = [fd_gradients(W1, W3, W2, k[j * chunk:(j + 1) * chunk], v[j * chunk:(j + 1) * chunk],
                      eta[j * chunk:(j + 1) * chunk])[2] for j in range(nch)]
    # the gradient does not depend on W2 (so the chunk gradients can all be taken up front)
    G_other = fd_gradients(W1, W3, 3.0 * W2 + 1.0, k[:chunk], v[:chunk], eta[:chunk])[2]
    assert rel(G_other, G[0]) < 1e-7
    Mx, U = np.zeros_like(W2), []
    for j in range(nch):
        if updates[j]:
            Mx = beta * Mx + G[j]
            U.append(ns_via_svd(Mx, 5))
        else:
            U.append(np.zeros_like(W2))
    PQ = phi_rows(W1, W3, q)
    want = np.zeros_like(o)
    for t in range(N):
        j = t // chunk
        seen = j + (1 if mask == O.MASK_UPDATE_THEN_APPLY else 0)   # chunks whose update t sees
        W2_t = W2 - sum((U[i] for i in range(seen)), np.zeros_like(W2))
        want[t] = W2_t @ PQ[t]
    assert rel(o, want) < 1e-6
    assert rel(W[2], W2 - sum(U, np.zeros_like(W2))) < 1e-6
    # negative control: Muon of each chunk's own outer product, summed (E.3 taken literally)
    lit = W2.copy()
    for j in range(nch):
        if updates[j]:
            lit = lit - ns_via_svd(G[j], 5)
    if beta:
        assert rel(lit, W[2]) > 1e-3


# ----------------------------------------------------------------------------------------------
# per-chunk rates outside the optimizer step (TTT-as-LA App. E.1, written per chunk in App. H)

def stepper_chunk_rates(q, k, v, lr, alpha, W1, W3, W2, chunk, mask, rule, last_only=False, upd=None, ns=5):
    """The chunk recurrence of App. H.2 (with Muon per App. E.3) from independent pieces: finite-
    difference gradients with every token weighted 1, the momentum step dW = g + alpha_j dW, the SVD
    form of Newton-Schulz, W - lr_j Opt(dW), loop row norms."""
    W = [W1.copy(), W3.copy(), W2.copy()]
    M = [np.zeros_like(x) for x in W]
    N = q.shape[0]
    o = np.zeros((N, W2.shape[0]))
    for j, lo in enumerate(range(0, N, chunk)):
        hi = min(lo + chunk, N)
        first = mask in (O.MASK_APPLY_THEN_UPDATE, O.MASK_STRIDED)
        if first:
            o[lo:hi] = np.stack([f_token(*W, x) for x in q[lo:hi]])
        if mask != O.MASK_STRIDED or upd[j]:
            G = fd_gradients(*W, k[lo:hi], v[lo:hi], np.ones(hi - lo))
            for i in ([2] if last_only else [0, 1, 2]):
                M[i] = G[i] if alpha is None else alpha[j] * M[i] + G[i]
                U = ns_via_svd(M[i], ns) if rule in (O.UPD_MUON_L2, O.UPD_MUON) else M[i]
                W[i] = W[i] - lr[j] * U
                if rule in (O.UPD_GD_L2, O.UPD_MUON_L2):
                    W[i] = rownorm_loops(W[i])
        if not first:
            o[lo:hi] = np.stack([f_token(*W, x) for x in q[lo:hi]])
    return o, W, M


@pytest.mark.parametrize("mask,rule,with_alpha,last_only", [
    (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, True, False), (O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, True, False),
    (O.MASK_STRIDED, O.UPD_MUON, True, True), (O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, False, False),
])
def test_chunk_rates_match_independent_stepper(mask, rule, with_alpha, last_only):
    q, k, v, _, W1, W3, W2 = tiny_problem(50, N=9)
    rng = np.random.default_rng(51)
    lr = 0.1 + 0.3 * rng.random(3)
    alpha = np.array([0.7, 0.0, 0.9]) if with_alpha else None   # alpha_j = 0 restarts the momentum
    upd = [1, 0, 1] if mask == O.MASK_STRIDED else None
    o, W, M = O.ttt_scan_ref(q, k, v, lr, W1, W3, W2, 3, mask, rule, 5, 0.0, last_only, upd, chunk_rates=True,
                             chunk_alpha=alpha)
    o2, W2s, M2 = stepper_chunk_rates(q, k, v, lr, alpha, W1, W3, W2, 3, mask, rule, last_only, upd)
    assert rel(o, o2) < 1e-6
    for a, b in zip(W, W2s):
        assert rel(a, b) < 1e-6


@pytest.mark.parametrize("mask", [O.MASK_UPDATE_THEN_APPLY, O.MASK_APPLY_THEN_UPDATE])
def test_chunk_rates_parallel_form_mask_c(mask):
    """App. H.1: with only the last layer learning by GD, per-chunk rates eta_j and momentum alpha_j,
    O = Phi(Q) W_0 + sum over chunks i <= t of C_ti Phi(Q_t) Phi(K_i)^T V_i with
    C_ti = sum_{j=i..t} eta_j prod_{s=i+1..j} alpha_s (update-then-apply: chunk t sees its own update;
    apply-then-update: the mask shifted by one chunk)."""
    N, chunk = 12, 3
    q, k, v, _, W1, W3, W2 = tiny_problem(52, N=N)
    rng = np.random.default_rng(53)
    nch = N // chunk
    lr = 0.1 + rng.random(nch)
    alpha = 0.2 + 0.7 * rng.random(nch)
    o, W, _ = O.ttt_scan_ref(q, k, v, lr, W1, W3, W2, chunk, mask, O.UPD_GD, 5, 0.0, True, chunk_rates=True,
                             chunk_alpha=alpha)
    PQ, PK = phi_rows(W1, W3, q), phi_rows(W1, W3, k)

    def C(t, i):
        return sum(lr[j] * np.prod([alpha[s] for s in range(i + 1, j + 1)]) for j in range(i, t + 1))

    want = PQ @ W2.T
    for p in range(N):
        t = p // chunk - (1 if mask == O.MASK_APPLY_THEN_UPDATE else 0)
        for s in range(N):
            i = s // chunk
            if i <= t:
                want[p] += C(t, i) * np.dot(PQ[p], PK[s]) * v[s]
    assert rel(o, want) < 1e-12


def test_chunk_rates_equal_token_rates_for_gd_at_constant_rates_but_not_for_muon():
    """With GD (and the weight norm), a constant per-chunk rate c and momentum beta equal the
    per-token form with every eta_i = c and momentum beta: c G inside the momentum or c outside it
    give the same step.  With Muon they differ: Newton-Schulz removes the scale of its input, so the
    per-token rates only weigh tokens against each other while eta_j outside sets the step size."""
    q, k, v, _, W1, W3, W2 = tiny_problem(54, N=8)
    c, beta = 0.37, 0.8
    for rule in (O.UPD_GD, O.UPD_GD_L2):
        a = O.ttt_scan_ref(q, k, v, np.full(8, c), W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, rule, 5, beta)
        b = O.ttt_scan_ref(q, k, v, np.full(2, c), W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, rule, 5, 0.0,
                           chunk_rates=True, chunk_alpha=np.full(2, beta))
        assert rel(a[0], b[0]) < 1e-12
    a = O.ttt_scan_ref(q, k, v, np.full(8, c), W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, 5, beta)
    b = O.ttt_scan_ref(q, k, v, np.full(2, c), W1, W3, W2, 4, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, 5, 0.0,
                       chunk_rates=True, chunk_alpha=np.full(2, beta))
    assert rel(a[1][2], b[1][2]) > 1e-2
    # the per-chunk Muon step is eta_j times a scale-free update: doubling eta doubles W - W0
    b2 = O.ttt_scan_ref(q, k, v, np.full(2, 2 * c), W1, W3, W2, 8, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, 5, 0.0,
                        True, chunk_rates=True)
    b1 = O.ttt_scan_ref(q, k, v, np.full(2, c), W1, W3, W2, 8, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, 5, 0.0,
                        True, chunk_rates=True)
    assert rel(b2[1][2] - W2, 2 * (b1[1][2] - W2)) < 1e-12
