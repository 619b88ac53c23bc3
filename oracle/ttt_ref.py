"""Plain fp64 CPU oracle for the large-chunk TTT-KVB layer and its linear reduction.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this module: only the
tests, the smoke check and the CPU-baseline leg of the benchmark do.  It shares no code with the
HIP library and imports nothing from it.

Sources (cited by title and equation; "LaCT notes" is the PaperTrace page
"5.2.1 LaCT and TTT-E2E", "TTT-as-LA" is the paper "Test-Time Training with KV Binding Is
Secretly Linear Attention", "LA-to-TTT" is the blog post "From Linear Attention to Test-Time
Training"):

* chunk update g = grad_W sum_i eta_i L(f_W(k_i), v_i) ........ LaCT notes, Eq. (2)
* apply o_i = f_W(q_i), all queries of a chunk share one W ...... LaCT notes, text after Eq. (2)
* f_W(x) = W2 [SiLU(W1 x) o (W3 x)], bias-free SwiGLU ........... LaCT notes, Eq. (3)
* L(f_W(k), v) = -f_W(k)^T v ..................................... LaCT notes, Eq. (4);
                                                                   TTT-as-LA, App. E.2
* W <- L2-Normalize(W - g), along the input dimension ........... LaCT notes, Eq. (5)
* W <- L2-Normalize(W - Muon(g)), Newton-Schulz, per matrix ..... LaCT notes, Eq. (6)
* momentum M <- beta M + sum_i eta_i grad L_i, Muon applied to M  LaCT notes, text after Eq. (6)
* the four update/apply orders and their masks ................... LaCT notes, section 1.1
* apply-then-update recurrence O_j, G_j, W_j ..................... LaCT notes, Eq. (10)
* linear bias-free fast weight + GD = linear attention ........... TTT-as-LA, Thm. 5.2 and
                                                                   Sec. 6.1 Step 6; LA-to-TTT,
                                                                   "Causal Linear Attention"
* several inner-loop gradient steps per chunk (inference time) ... TTT-as-LA, Sec. 4.1
* the backward of the linear reduction (outer-loop gradients) ..... TTT-as-LA, Sec. 6.2 and Fig. 4
                                                                   (training with the parallel form)
* the backward of the layer with frozen W1, W3 (last layer only, GD, momentum, the L2 norm):
  the state's recurrence transposed over phi(q), phi(k), then phi's chain rule  TTT-as-LA, Thm. 5.2-5.3,
                                                                   Sec. 6.1-6.2
* the backward of the chunk recurrence (every rule, momentum, all three weights learning or W2
  alone): reverse mode over the steps, each through the norm's transpose, W - U or W - Muon(U)
  (Newton-Schulz walked back), the momentum and the chunk gradient differentiated once more
  (SiLU'' included) ................................................ TTT-as-LA, Sec. 6.2; LaCT notes,
                                                                   Eqs. (2)-(6) and section 1.1
* gradient ascent in the inner loop: the step's sign flips ....... TTT-as-LA, Sec. 4.2 and 5.2
* per-chunk rates outside the optimizer step: momentum dW_j = g_j + alpha_j dW_{j-1} over the
  chunk gradient g_j (unit token weights), W <- W - eta_j Opt(dW_j) .. TTT-as-LA, App. E.1 (per token)
                                                                   and App. H.1-H.2 (per chunk),
                                                                   App. E.3 (with Muon)

Readings taken where the pages are silent or garbled (each is also listed in the design notes):

* orientation: W1, W3 are m x d (gate, up), W2 is d x m (down); tokens are rows, so a chunk's
  outputs are rows of f applied to rows of Q;
* mask "chunk = whole sequence" is taken as update-then-apply with one chunk (the only reading
  that mixes tokens bidirectionally); STRIDED is apply-then-update that skips the update on
  chunks whose flag is 0;
* L2-Normalize scales each row (one output unit over its input dimension) to unit norm,
  w / max(||w||_2, 1e-6); W0 is used as given;
* Muon is the cubic Newton-Schulz polar iteration X <- 1.5 X - 0.5 (X X^T) X, started from
  U / (||U||_F + 1e-7) and run on the side with the smaller Gram matrix;
* eta sits inside the gradient sum (before Muon); the gradient is a sum (not a mean) over the
  chunk; momentum is per chunk with M0 = 0 and no dampening;
* a partial last chunk (N not a multiple of the chunk) simply holds fewer tokens;
* n inner steps on a chunk repeat the whole update n times, each from the gradient at the current
  W (momentum and Muon included, one momentum step per inner step); ascent adds the gradient
  instead of subtracting it, everything else unchanged;
* per-chunk rates (App. E.1 written per chunk as in H.1): eta_j and alpha_j belong to each (batch,
  head) and chunk; the chunk gradient weighs every token by 1; the momentum step is taken on every
  updating chunk (alpha_j = 0 restarts it from g_j); Muon, when the rule has it, acts on dW_j before
  eta_j scales it; the weight norm, when the rule has it, follows W - eta_j Opt(dW_j).

Parity status: every function here is pinned by the CPU tests (finite differences, closed forms
of the linear and last-layer reductions, the SVD polar factor, invariants).  The full SwiGLU
L2 / Muon recurrences have no closed form; they are pinned through their separately pinned parts.
"""
from __future__ import annotations

import numpy as np

# mask orders (LaCT notes, section 1.1)
MASK_FULL = 0                # chunk = whole sequence, update then apply -> bidirectional
MASK_UPDATE_THEN_APPLY = 1   # block-causal, own chunk visible
MASK_APPLY_THEN_UPDATE = 2   # only earlier chunks visible (Eq. (10), language modelling)
MASK_STRIDED = 3             # update on flagged chunks only, apply on all
MASK_TOKEN_CAUSAL = 4        # linear model only: every token sees itself and all earlier tokens

# update rules
UPD_GD = 0        # W <- W - U (no normalisation)
UPD_GD_L2 = 1     # Eq. (5)
UPD_MUON_L2 = 2   # Eq. (6)
UPD_MUON = 3      # W <- W - Muon(U), no weight norm (TTT-as-LA Table 2, Variant 2 recurrence)

ROW_NORM_EPS = 1e-6
NS_EPS = 1e-7


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """SiLU(a) = a * sigmoid(a)."""
    return x * sigmoid(x)


def swiglu_apply(W1, W3, W2, X):
    """Rows of f_W(X) for the bias-free SwiGLU fast weight, LaCT notes Eq. (3).

    X is [n, d]; W1, W3 are [m, d]; W2 is [d, m].  Returns [n, d].
    """
    A = X @ W1.T
    C = X @ W3.T
    return (silu(A) * C) @ W2.T


def chunk_gradients(W1, W3, W2, K, V, eta):
    """Gradients of sum_i eta_i * (-f_W(k_i)^T v_i) w.r.t. W1, W3, W2 (LaCT notes Eqs. (2)-(4)).

    The loss derivative w.r.t. f_W(k_i) is -eta_i v_i (TTT-as-LA App. E.2); the rest is the
    chain rule through W2, the product and the SiLU.  Returns (G1, G3, G2) with the shapes of
    (W1, W3, W2).
    """
    A = K @ W1.T                   # [b, m] pre-activation of the gate
    C = K @ W3.T                   # [b, m] up projection
    s = sigmoid(A)
    Hk = A * s * C                 # hidden features of the keys
    Df = -eta[:, None] * V         # dLoss/df(k_i), [b, d]
    G2 = Df.T @ Hk                 # [d, m]
    DH = Df @ W2                   # dLoss/dH, [b, m]
    dsilu = s * (1.0 + A * (1.0 - s))
    G1 = (DH * C * dsilu).T @ K    # [m, d]
    G3 = (DH * A * s).T @ K        # [m, d]
    return G1, G3, G2


def l2_normalize_rows(W, eps=ROW_NORM_EPS):
    """L2-Normalize of LaCT notes Eq. (5): each row (an output unit over its inputs) to unit norm."""
    n = np.sqrt(np.sum(W * W, axis=1, keepdims=True))
    return W / np.maximum(n, eps)


def newton_schulz(U, iters, eps=NS_EPS):
    """Muon(U) of LaCT notes Eq. (6): the cubic Newton-Schulz approximation of the polar factor.

    X0 = U / (||U||_F + eps); then `iters` times X <- 1.5 X - 0.5 (X X^T) X on the side whose Gram
    matrix is smaller (U is transposed first when it has more rows than columns, and back after).
    """
    U = _f64(U)
    tr = U.shape[0] > U.shape[1]
    X = U.T if tr else U
    X = X / (np.sqrt(np.sum(X * X)) + eps)
    for _ in range(iters):
        X = 1.5 * X - 0.5 * ((X @ X.T) @ X)
    return X.T if tr else X


def chunk_bounds(N, chunk):
    """Token ranges [lo, hi) of the chunks; the last one may be shorter."""
    return [(lo, min(lo + chunk, N)) for lo in range(0, N, chunk)]


def _weight_update(W, G, Mx, rule, ns_iters, momentum, lr=None, alpha=None):
    """One fast-weight update of one matrix: optional momentum, optional Muon, W - U, optional norm.
    With per-chunk rates (lr is not None): the momentum step dW = G + alpha dW is always taken when
    alpha is given (alpha None: dW = G), and the step is W - lr Opt(dW)."""
    U = G
    if lr is not None:
        if alpha is not None:
            Mx = alpha * Mx + G
            U = Mx
    elif momentum != 0.0:
        Mx = momentum * Mx + G
        U = Mx
    if rule in (UPD_MUON_L2, UPD_MUON):
        U = newton_schulz(U, ns_iters)
    W = W - (U if lr is None else lr * U)
    if rule in (UPD_GD_L2, UPD_MUON_L2):
        W = l2_normalize_rows(W)
    return W, Mx


def ttt_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, rule, ns_iters=5, momentum=0.0,
                 last_layer_only=False, update_chunks=None, M=None, inner_steps=1, ascent=False,
                 chunk_rates=False, chunk_alpha=None):
    """One (batch, head) scan of the TTT-KVB layer.

    q, k, v [N, d]; eta [N]; W1, W3 [m, d]; W2 [d, m]; M optional (M1, M3, M2) momentum state.
    Returns (o [N, d], (W1, W3, W2), (M1, M3, M2)).  The apply/update order per chunk follows
    LaCT notes section 1.1 and Eq. (10).  An updating chunk takes ``inner_steps`` gradient steps
    (TTT-as-LA Sec. 4.1); ``ascent`` steps along +g instead of -g (TTT-as-LA Sec. 4.2).
    chunk_rates: eta is [number of chunks], one rate per chunk applied outside the optimizer step,
    the chunk gradient weighs its tokens by 1, and chunk_alpha ([number of chunks] or None) holds
    the per-chunk momentum factors (TTT-as-LA App. E.1, H.1-H.2, E.3); ``momentum`` is then unused.
    """
    q, k, v, eta = _f64(q), _f64(k), _f64(v), _f64(eta)
    W = [_f64(W1).copy(), _f64(W3).copy(), _f64(W2).copy()]
    N, d = q.shape
    if M is None:
        Ms = [np.zeros_like(W[0]), np.zeros_like(W[1]), np.zeros_like(W[2])]
    else:
        Ms = [_f64(x).copy() for x in M]
    o = np.zeros((N, W[2].shape[0]))
    bounds = chunk_bounds(N, chunk)
    if mask == MASK_FULL and len(bounds) > 1:
        raise ValueError("MASK_FULL needs chunk >= N")
    if mask == MASK_TOKEN_CAUSAL:
        raise ValueError("MASK_TOKEN_CAUSAL is defined for the linear model only")
    for j, (lo, hi) in enumerate(bounds):
        update = True
        if mask == MASK_STRIDED:
            update = bool(update_chunks[j])
        apply_first = mask in (MASK_APPLY_THEN_UPDATE, MASK_STRIDED)
        if apply_first:
            o[lo:hi] = swiglu_apply(W[0], W[1], W[2], q[lo:hi])
        if update:
            for _ in range(inner_steps):
                w_tok = np.ones(hi - lo) if chunk_rates else eta[lo:hi]
                G = chunk_gradients(W[0], W[1], W[2], k[lo:hi], v[lo:hi], w_tok)
                if ascent:
                    G = tuple(-g for g in G)
                which = (2,) if last_layer_only else (0, 1, 2)
                for i in which:
                    if chunk_rates:
                        a_j = None if chunk_alpha is None else float(chunk_alpha[j])
                        W[i], Ms[i] = _weight_update(W[i], G[i], Ms[i], rule, ns_iters, 0.0, float(eta[j]), a_j)
                    else:
                        W[i], Ms[i] = _weight_update(W[i], G[i], Ms[i], rule, ns_iters, momentum)
        if not apply_first:
            o[lo:hi] = swiglu_apply(W[0], W[1], W[2], q[lo:hi])
    return o, tuple(W), tuple(Ms)


def ttt_forward_ref(q, k, v, eta, W1, W3, W2, chunk, mask, rule, ns_iters=5, momentum=0.0,
                    last_layer_only=False, update_chunks=None, M=None, slices=None, inner_steps=1,
                    ascent=False, chunk_rates=False, chunk_alpha=None):
    """The TTT-KVB layer over [B, H, N, d] inputs; every (batch, head) scan is independent.

    W1, W3, W2 are per head ([H, ...]) or per (batch, head) ([B, H, ...]).  M, if given, is a
    tuple of three [B, H, ...] momentum arrays.  ``slices`` restricts the work to a list of
    (b, h) pairs (the other outputs stay zero).  Returns (o, (W1, W3, W2), (M1, M3, M2)) with
    [B, H, ...] weight and momentum stacks.  With chunk_rates, eta and chunk_alpha are
    [B, H, number of chunks].
    """
    B, H, N, d = q.shape
    m = W1.shape[-2]
    o = np.zeros((B, H, N, d))
    Wo = [np.zeros((B, H, m, d)), np.zeros((B, H, m, d)), np.zeros((B, H, d, m))]
    Mo = [np.zeros_like(x) for x in Wo]
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        ws = [x[h] if x.ndim == 3 else x[b, h] for x in (W1, W3, W2)]
        Mi = None if M is None else tuple(x[b, h] for x in M)
        ob, Wb, Mb = ttt_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], *ws, chunk, mask, rule,
                                  ns_iters, momentum, last_layer_only, update_chunks, Mi, inner_steps,
                                  ascent, chunk_rates, None if chunk_alpha is None else chunk_alpha[b, h])
        o[b, h] = ob
        for i in range(3):
            Wo[i][b, h] = Wb[i]
            Mo[i][b, h] = Mb[i]
    return o, tuple(Wo), tuple(Mo)


def linattn_scan_ref(q, k, v, eta, S0, chunk, mask, update_chunks=None):
    """One (batch, head) scan of the linear fast weight trained by plain GD on the dot-product loss.

    With f_S(x) = S x (S is d_v x d_k), L = -(S k)^T v gives grad = -v k^T, so one chunk's GD step
    is S <- S + sum_i eta_i v_i k_i^T (TTT-as-LA Thm. 5.2, Sec. 6.1 Step 6).  The apply/update
    order per chunk is the same as the SwiGLU layer's; MASK_TOKEN_CAUSAL is the one-token-chunk
    update-then-apply limit (LA-to-TTT, "Causal Linear Attention").  Returns (o, S).
    """
    q, k, v, eta = _f64(q), _f64(k), _f64(v), _f64(eta)
    S = _f64(S0).copy()
    N = q.shape[0]
    o = np.zeros((N, S.shape[0]))
    if mask == MASK_TOKEN_CAUSAL:
        chunk = 1
        mask = MASK_UPDATE_THEN_APPLY
    bounds = chunk_bounds(N, chunk)
    if mask == MASK_FULL and len(bounds) > 1:
        raise ValueError("MASK_FULL needs chunk >= N")
    for j, (lo, hi) in enumerate(bounds):
        update = True if mask != MASK_STRIDED else bool(update_chunks[j])
        apply_first = mask in (MASK_APPLY_THEN_UPDATE, MASK_STRIDED)
        if apply_first:
            o[lo:hi] = q[lo:hi] @ S.T
        if update:
            S = S + (eta[lo:hi, None] * v[lo:hi]).T @ k[lo:hi]
        if not apply_first:
            o[lo:hi] = q[lo:hi] @ S.T
    return o, S


def linattn_forward_ref(q, k, v, eta, chunk, mask, S0=None, update_chunks=None, slices=None):
    """Linear attention over [B, H, N, d] inputs.  S0 is [B, H, d_v, d_k] or None (zeros)."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, N, dv))
    S = np.zeros((B, H, dv, dk))
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        s0 = np.zeros((dv, dk)) if S0 is None else S0[b, h]
        o[b, h], S[b, h] = linattn_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], s0, chunk, mask,
                                            update_chunks)
    return o, S


def gemm_intensity(h, b):
    """LaCT notes Eq. (1): FLOP per byte of an h x h bf16 weight times a b x h chunk."""
    return (2.0 * h * h * b) / (2.0 * h * h + 4.0 * h * b)


def linattn_backward_scan_ref(q, k, v, eta, S0, chunk, mask, dO, dS_out=None, update_chunks=None):
    """Gradients of one (batch, head) scan of chunked linear attention (linattn_scan_ref) under the
    chunked masks, for the loss L = sum_t dO_t . o_t + <dS_out, S_out>.

    Written from the forward's structure: chunk c's queries see the state S_c (S0 plus the updates
    of the chunks before it, or up to it under update-then-apply and the one-chunk FULL mask), so
    dq_t = S_c^T dO_t and D_c = sum_{t in c} dO_t q_t^T is the gradient of S_c.  The update of
    chunk j, dS_j = sum_s eta_s v_s k_s^T, reaches every S_c that includes it and S_out, so its
    gradient is R_j = sum of those D_c plus dS_out, and dv_s = eta_s R_j k_s, dk_s = eta_s R_j^T v_s,
    deta_s = v_s . (R_j k_s); chunks that do not update give zero.  dS0 = sum_c D_c + dS_out.
    Returns (dq, dk, dv, deta, dS0).
    """
    q, k, v, eta, dO = (_f64(x) for x in (q, k, v, eta, dO))
    if mask == MASK_TOKEN_CAUSAL:
        raise ValueError("the backward covers the chunked masks")
    S = _f64(S0).copy()
    N = q.shape[0]
    bounds = chunk_bounds(N, chunk)
    if mask == MASK_FULL and len(bounds) > 1:
        raise ValueError("MASK_FULL needs chunk >= N")
    post = mask in (MASK_UPDATE_THEN_APPLY, MASK_FULL)
    upd = [mask != MASK_STRIDED or bool(update_chunks[j]) for j in range(len(bounds))]
    # forward states each chunk's queries see
    Sc = []
    for j, (lo, hi) in enumerate(bounds):
        dS = (eta[lo:hi, None] * v[lo:hi]).T @ k[lo:hi] if upd[j] else 0.0
        if post:
            S = S + dS
        Sc.append(S.copy())
        if not post:
            S = S + dS
    dq = np.zeros_like(q)
    D = []
    for j, (lo, hi) in enumerate(bounds):
        dq[lo:hi] = dO[lo:hi] @ Sc[j]
        D.append(dO[lo:hi].T @ q[lo:hi])
    dSo = np.zeros_like(S) if dS_out is None else _f64(dS_out)   # (no tokens: S_out = S0)
    dk, dv, deta = np.zeros_like(k), np.zeros_like(v), np.zeros_like(eta)
    for j, (lo, hi) in enumerate(bounds):
        if not upd[j]:
            continue
        seen_by = range(j, len(bounds)) if post else range(j + 1, len(bounds))
        R = dSo + sum((D[c] for c in seen_by), np.zeros_like(dSo))
        u = k[lo:hi] @ R.T                       # R_j k_s, one row per token
        dv[lo:hi] = eta[lo:hi, None] * u
        dk[lo:hi] = eta[lo:hi, None] * (v[lo:hi] @ R)
        deta[lo:hi] = np.sum(v[lo:hi] * u, axis=1)
    dS0 = dSo + sum(D, np.zeros_like(dSo))
    return dq, dk, dv, deta, dS0


def linattn_backward_ref(q, k, v, eta, chunk, mask, dO, S0=None, dS_out=None, update_chunks=None, slices=None):
    """linattn_backward_scan_ref over [B, H, N, d] inputs; S0 and dS_out are [B, H, d_v, d_k] or None."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    out = [np.zeros((B, H, N, dk)), np.zeros((B, H, N, dk)), np.zeros((B, H, N, dv)), np.zeros((B, H, N)),
           np.zeros((B, H, dv, dk))]
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        s0 = np.zeros((dv, dk)) if S0 is None else S0[b, h]
        dso = None if dS_out is None else dS_out[b, h]
        res = linattn_backward_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], s0, chunk, mask, dO[b, h], dso,
                                        update_chunks)
        for o_, r in zip(out, res):
            o_[b, h] = r
    return tuple(out)


def _recurrent_state_backward(phq, phk, v, eta, S0, chunk, mask, dO, dS_out, update_chunks, reps, sign, beta, norm):
    """The linear-attention part of the layer's backward when W2's steps carry momentum or end in
    the L2 norm (the state walked chunk by chunk).

    Forward, per updating chunk and step (reps steps): m <- beta m + sign dS_c, x = S + m, and S <- x,
    or S <- L2-Normalize(x) row by row (norm; LaCT notes Eq. (5)), with dS_c = sum eta v phi(k)^T and
    m starting at zero (m is minus the momentum M of M <- beta M + g, W2 <- [norm](W2 - M); LaCT notes,
    text after Eq. (6)).  Backward: the chunks' queries see S_c, so dphi(q)_t = S_c^T dO_t and
    D_c = sum_t dO_t phi(q)_t^T is S_c's gradient; the recurrence is then walked transposed from the
    last chunk: with gS and gm the gradients of S and m after a step, the step's norm sends gS back
    to gx = (gS - y (y . gS)) / |x| per row (y = S after the step; gS / eps where |x| <= eps), its
    update receives g = gm + gx, and gm <- beta g, gS <- gx before it.  The final momentum is not part
    of the loss.  Returns (dphi(q), dphi(k), dv, deta, dS0).
    """
    N = phq.shape[0]
    bounds = chunk_bounds(N, chunk)
    post = mask in (MASK_UPDATE_THEN_APPLY, MASK_FULL)
    upd = [mask != MASK_STRIDED or bool(update_chunks[j]) for j in range(len(bounds))]
    S, m = _f64(S0).copy(), np.zeros_like(_f64(S0))
    Sc, steps = [], {}  # steps[j]: (y, |x| per row) of each of chunk j's steps

    def update(j, dS):
        nonlocal S, m
        steps[j] = []
        for _ in range(reps):
            m = beta * m + sign * dS
            x = S + m
            if norm:
                n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
                S = x / np.maximum(n, ROW_NORM_EPS)
                steps[j].append((S.copy(), n))
            else:
                S = x

    for j, (lo, hi) in enumerate(bounds):
        dS = (eta[lo:hi, None] * v[lo:hi]).T @ phk[lo:hi]
        if post and upd[j]:
            update(j, dS)
        Sc.append(S.copy())
        if not post and upd[j]:
            update(j, dS)
    dphq = np.zeros_like(phq)
    D = []
    for j, (lo, hi) in enumerate(bounds):
        dphq[lo:hi] = dO[lo:hi] @ Sc[j]
        D.append(dO[lo:hi].T @ phq[lo:hi])
    gS = np.zeros_like(S) if dS_out is None else _f64(dS_out).copy()
    gm = np.zeros_like(S)
    R = [None] * len(bounds)
    for j in reversed(range(len(bounds))):
        if post:
            gS = gS + D[j]
        if upd[j]:
            Rj = np.zeros_like(S)
            for r in reversed(range(reps)):
                if norm:
                    y, n = steps[j][r]
                    gx = np.where(n > ROW_NORM_EPS, (gS - y * np.sum(y * gS, axis=1, keepdims=True)) / np.maximum(n, ROW_NORM_EPS),
                                  gS / ROW_NORM_EPS)
                else:
                    gx = gS
                g = gm + gx
                Rj = Rj + g
                gm = beta * g
                gS = gx
            R[j] = sign * Rj          # the gradient of dS_j
        if not post:
            gS = gS + D[j]
    dphk, dv, deta = np.zeros_like(phk), np.zeros_like(v), np.zeros_like(eta)
    for j, (lo, hi) in enumerate(bounds):
        if upd[j]:
            u = phk[lo:hi] @ R[j].T
            dv[lo:hi] = eta[lo:hi, None] * u
            dphk[lo:hi] = eta[lo:hi, None] * (v[lo:hi] @ R[j])
            deta[lo:hi] = np.sum(v[lo:hi] * u, axis=1)
    return dphq, dphk, dv, deta, gS


def ttt_lastlayer_backward_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, dO, dW_out=None, update_chunks=None,
                                    inner_steps=1, ascent=False, momentum=0.0, rule=UPD_GD):
    """Gradients of one (batch, head) scan of the TTT-KVB layer whose inner loop trains W2 alone by
    GD (ttt_scan_ref with last_layer_only, rule UPD_GD or UPD_GD_L2), for the loss
    L = sum_t dO_t . o_t + <dW1_out, W1> + <dW3_out, W3> + <dW2_out, W2_out>.

    With W1 and W3 frozen, phi(x) = SiLU(W1 x) o (W3 x) is fixed, the chunk gradient of W2 is
    -sum eta v phi(k)^T, and the layer is chunked linear attention with queries phi(q), keys
    phi(k), values v and state W2 (TTT-as-LA, Thm. 5.2-5.3 and Sec. 6.1 Steps 1-6); its outer-loop
    gradients (TTT-as-LA, Sec. 6.2) are those of linear attention (linattn_backward_scan_ref),
    followed by the chain rule through phi.  inner_steps repeats an update that does not depend on
    W2, and ascent flips its sign: without momentum or norm both scale eta.  With momentum (starting
    from zero, its final state outside the loss) or the L2 norm (UPD_GD_L2: Variant 1 of TTT-as-LA
    Sec. 6.1 without Muon) the state part is _recurrent_state_backward.  dW_out is
    None or (dW1, dW3, dW2) of the shapes of (W1, W3, W2).  Returns (dq, dk, dv, deta, (dW1, dW3, dW2)).
    """
    q, k, v, eta, dO = (_f64(x) for x in (q, k, v, eta, dO))
    W1, W3, W2 = _f64(W1), _f64(W3), _f64(W2)
    sign, reps = (-1.0 if ascent else 1.0), max(int(inner_steps), 1)
    A = {"q": q @ W1.T, "k": k @ W1.T}
    C = {"q": q @ W3.T, "k": k @ W3.T}
    phi = {s: silu(A[s]) * C[s] for s in ("q", "k")}
    dW2o = None if dW_out is None else dW_out[2]
    if rule not in (UPD_GD, UPD_GD_L2):
        raise ValueError("the backward covers W2 learning alone by GD, with or without the L2 norm")
    if momentum == 0.0 and rule == UPD_GD:
        f = sign * reps
        dphq, dphk, dv, deta, dW2 = linattn_backward_scan_ref(phi["q"], phi["k"], v, f * eta, W2, chunk, mask, dO,
                                                              dW2o, update_chunks)
        deta = f * deta
    else:
        dphq, dphk, dv, deta, dW2 = _recurrent_state_backward(phi["q"], phi["k"], v, eta, W2, chunk, mask, dO, dW2o,
                                                              update_chunks, reps, sign, float(momentum),
                                                              rule == UPD_GD_L2)
    dW1 = np.zeros_like(W1) if dW_out is None else _f64(dW_out[0]).copy()
    dW3 = np.zeros_like(W3) if dW_out is None else _f64(dW_out[1]).copy()
    dx = {}
    for s, x, dphi in (("q", q, dphq), ("k", k, dphk)):
        sg = sigmoid(A[s])
        dA = dphi * C[s] * sg * (1.0 + A[s] * (1.0 - sg))   # d SiLU(a)/da = s (1 + a (1 - s))
        dC = dphi * A[s] * sg
        dx[s] = dA @ W1 + dC @ W3
        dW1 += dA.T @ x
        dW3 += dC.T @ x
    return dx["q"], dx["k"], dv, deta, (dW1, dW3, dW2)


def ttt_lastlayer_backward_ref(q, k, v, eta, W1, W3, W2, chunk, mask, dO, dW_out=None, update_chunks=None,
                               inner_steps=1, ascent=False, slices=None, momentum=0.0, rule=UPD_GD):
    """ttt_lastlayer_backward_scan_ref over [B, H, N, d] inputs.  W1, W3, W2 are per head ([H, ...])
    or per (batch, head) ([B, H, ...]); the weight gradients take the same shape (per-head weights
    sum over the batch).  dW_out is None or three [B, H, ...] arrays (the W_out the layer returns
    is per (batch, head)).  Returns (dq, dk, dv, deta, (dW1, dW3, dW2))."""
    B, H, N, d = q.shape
    per_head = W1.ndim == 3
    dq, dk, dv = np.zeros((B, H, N, d)), np.zeros((B, H, N, d)), np.zeros((B, H, N, d))
    deta = np.zeros((B, H, N))
    dW = [np.zeros(x.shape) for x in (W1, W3, W2)]
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        ws = [x[h] if per_head else x[b, h] for x in (W1, W3, W2)]
        dwo = None if dW_out is None else tuple(x[b, h] for x in dW_out)
        r = ttt_lastlayer_backward_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], *ws, chunk, mask, dO[b, h], dwo,
                                            update_chunks, inner_steps, ascent, momentum, rule)
        dq[b, h], dk[b, h], dv[b, h], deta[b, h] = r[:4]
        for i in range(3):
            if per_head:
                dW[i][h] += r[4][i]
            else:
                dW[i][b, h] = r[4][i]
    return dq, dk, dv, deta, tuple(dW)


def _row_norm_transpose(X, g, eps=ROW_NORM_EPS):
    """The transpose of L2-Normalize's Jacobian at X (rows over the input dimension), applied to a
    gradient g of its output: (g - y (y . g)) / |x| with y = x / |x| where |x| > eps, g / eps where
    the floor binds (LaCT notes, Eq. (5))."""
    n = np.sqrt(np.sum(X * X, axis=1, keepdims=True))
    y = X / np.maximum(n, eps)
    big = n > eps
    return np.where(big, (g - y * np.sum(y * g, axis=1, keepdims=True)) / np.where(big, n, 1.0), g / eps)


def newton_schulz_backward(U, iters, G, eps=NS_EPS):
    """The gradient with respect to U of <G, newton_schulz(U, iters)> (LaCT notes, Eq. (6)): the
    iteration run again, then walked back.  One cubic step X' = 1.5 X - 0.5 (X X^T) X takes a
    gradient G of X' to 1.5 G - 0.5 [(G X^T + X G^T) X + (X X^T) G]; the start X0 = U / (|U| + eps)
    takes G to G / (|U| + eps) - <G, U> U / ((|U| + eps)^2 |U|) (the second term is absent at U = 0).
    A U with more rows than columns is handled transposed, as the forward does."""
    U, G = _f64(U), _f64(G)
    tr = U.shape[0] > U.shape[1]
    X = U.T if tr else U
    G = G.T if tr else G
    n = np.sqrt(np.sum(X * X))
    Xs = [X / (n + eps)]
    for _ in range(iters):
        Xk = Xs[-1]
        Xs.append(1.5 * Xk - 0.5 * ((Xk @ Xk.T) @ Xk))
    for k in range(iters - 1, -1, -1):
        Xk = Xs[k]
        G = 1.5 * G - 0.5 * ((G @ Xk.T + Xk @ G.T) @ Xk + (Xk @ Xk.T) @ G)
    dX = G / (n + eps)
    if n > 0:
        dX = dX - (np.sum(G * X) / ((n + eps) ** 2 * n)) * X
    return dX.T if tr else dX


def swiglu_apply_backward(W1, W3, W2, X, dO):
    """Gradients of sum dO . f_W(X) (LaCT notes, Eq. (3)): returns (dX, dW1, dW3, dW2)."""
    A, C = X @ W1.T, X @ W3.T
    s = sigmoid(A)
    dH = dO @ W2                                   # [n, m]
    dA = dH * C * s * (1.0 + A * (1.0 - s))        # SiLU'(a) = s (1 + a (1 - s))
    dC = dH * A * s
    return dA @ W1 + dC @ W3, dA.T @ X, dC.T @ X, dO.T @ (A * s * C)


def chunk_gradients_backward(W1, W3, W2, K, V, eta, G1b, G3b, G2b):
    """The transpose of chunk_gradients' derivative: given the gradients (G1b, G3b, G2b) of a loss
    with respect to its outputs (G1, G3, G2), the gradients with respect to its inputs W1, W3, W2,
    K, V, eta (LaCT notes, Eqs. (2)-(4), differentiated once more).  Returns
    (dW1, dW3, dW2, dK, dV, deta).

    With A = K W1^T, C = K W3^T, s = sigmoid(A), H = SiLU(A) C, Df = -eta V and E = Df W2, the
    forward is G2 = Df^T H, G1 = (E C SiLU'(A))^T K, G3 = (E SiLU(A))^T K; every step below is the
    chain rule through one of these, SiLU''(a) = s (1 - s) (2 + a (1 - 2 s)) included."""
    A, C = K @ W1.T, K @ W3.T
    s = sigmoid(A)
    S0 = A * s                                      # SiLU(a)
    S1 = s * (1.0 + A * (1.0 - s))                  # SiLU'(a)
    S2 = s * (1.0 - s) * (2.0 + A * (1.0 - 2.0 * s))  # SiLU''(a)
    Df = -eta[:, None] * V
    H = S0 * C
    E = Df @ W2
    # G1 = (E C S1)^T K and G3 = (E S0)^T K
    dDA, dDC = K @ G1b.T, K @ G3b.T                # gradients of E C S1 and of E S0, [n, m]
    dK = (E * C * S1) @ G1b + (E * S0) @ G3b
    # G2 = Df^T H
    dDf = H @ G2b.T                                 # [n, d]
    dH = Df @ G2b                                   # [n, m]
    # the elementwise products, back to E, C and A
    dE = dDA * C * S1 + dDC * S0
    dC = dDA * E * S1 + dH * S0
    dA = dDA * E * C * S2 + dDC * E * S1 + dH * C * S1
    # E = Df W2, A = K W1^T, C = K W3^T, Df = -eta V
    dDf += dE @ W2.T
    dW2 = Df.T @ dE
    dK += dA @ W1 + dC @ W3
    dW1, dW3 = dA.T @ K, dC.T @ K
    dV = -eta[:, None] * dDf
    deta = -np.sum(V * dDf, axis=1)
    return dW1, dW3, dW2, dK, dV, deta


def ttt_backward_scan_ref(q, k, v, eta, W1, W3, W2, chunk, mask, dO, dW_out=None, update_chunks=None,
                          inner_steps=1, ascent=False, momentum=0.0, rule=UPD_GD, last_layer_only=False, ns_iters=5):
    """Gradients of one (batch, head) scan of the TTT-KVB layer (ttt_scan_ref with any of the four
    rules, all three weights learning unless last_layer_only) for the loss
    L = sum_t dO_t . o_t + <dW1_out, W1_out> + <dW3_out, W3_out> + <dW2_out, W2_out>.

    The outer-loop gradient (TTT-as-LA, Sec. 6.2) of the chunk recurrence (LaCT notes, section 1.1
    and Eqs. (2)-(5)), taken in reverse mode: the forward is run once and keeps every step's weights
    (and, with the norm, every step's W - U); then, from the last step back, the gradient of the
    weights a step produced goes through the norm's transpose, the step W - U (W - Muon(U) with
    newton_schulz_backward), the momentum M <- beta M + g (starting from zero; the final momentum is
    outside the loss) and the chunk gradient g (chunk_gradients_backward), and the queries that read
    a set of weights add the gradient of their outputs (swiglu_apply_backward).  dW_out is None or
    (dW1, dW3, dW2).
    Returns (dq, dk, dv, deta, (dW1, dW3, dW2)) with dW the gradients of W1, W3, W2 on entry.
    """
    q, k, v, eta, dO = (_f64(x) for x in (q, k, v, eta, dO))
    if rule not in (UPD_GD, UPD_GD_L2, UPD_MUON_L2, UPD_MUON):
        raise ValueError("unknown update rule")
    N, d = q.shape
    bounds = chunk_bounds(N, chunk)
    if mask == MASK_FULL and len(bounds) > 1:
        raise ValueError("MASK_FULL needs chunk >= N")
    if mask == MASK_TOKEN_CAUSAL:
        raise ValueError("MASK_TOKEN_CAUSAL is defined for the linear model only")
    sign = -1.0 if ascent else 1.0
    learn = (2,) if last_layer_only else (0, 1, 2)
    norm = rule in (UPD_GD_L2, UPD_MUON_L2)
    muon = rule in (UPD_MUON_L2, UPD_MUON)
    # forward: Ws[t] are the weights before step t; reads[t] the chunks whose queries see Ws[t]
    W = [_f64(W1).copy(), _f64(W3).copy(), _f64(W2).copy()]
    M = [np.zeros_like(x) for x in W]
    Ws, Xs, Us, steps, reads = [], [], [], [], {}
    for j, (lo, hi) in enumerate(bounds):
        update = mask != MASK_STRIDED or bool(update_chunks[j])
        apply_first = mask in (MASK_APPLY_THEN_UPDATE, MASK_STRIDED)
        if apply_first:
            reads.setdefault(len(Ws), []).append(j)
        if update:
            for _ in range(max(int(inner_steps), 1)):
                G = chunk_gradients(W[0], W[1], W[2], k[lo:hi], v[lo:hi], eta[lo:hi])
                Ws.append([x.copy() for x in W])
                X, Ui = [None, None, None], [None, None, None]
                for i in learn:
                    M[i] = momentum * M[i] + sign * G[i]
                    Ui[i] = M[i].copy()
                    X[i] = W[i] - (newton_schulz(M[i], ns_iters) if muon else M[i])
                    W[i] = l2_normalize_rows(X[i]) if norm else X[i]
                Xs.append(X)
                Us.append(Ui)
                steps.append(j)
        if not apply_first:
            reads.setdefault(len(Ws), []).append(j)
    T = len(Ws)
    # reverse
    dq, dk, dv, deta = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(eta)
    dW = [np.zeros_like(x) for x in W] if dW_out is None else [_f64(x).copy() for x in dW_out]
    dM = [np.zeros_like(x) for x in W]
    Wt = W
    for t in range(T, -1, -1):
        if t < T:  # step t took Ws[t] to the weights whose gradient dW now holds
            Wt = Ws[t]
            lo, hi = bounds[steps[t]]
            gG = [np.zeros_like(x) for x in W]  # gradient of the chunk gradient g
            for i in learn:
                gx = _row_norm_transpose(Xs[t][i], dW[i]) if norm else dW[i]  # gradient of X = W - Opt(M)
                # M enters X with a minus sign, through Muon when the rule has it
                dMi = dM[i] + (newton_schulz_backward(Us[t][i], ns_iters, -gx) if muon else -gx)
                gG[i] = sign * dMi
                dM[i] = momentum * dMi
                dW[i] = gx
            r = chunk_gradients_backward(Wt[0], Wt[1], Wt[2], k[lo:hi], v[lo:hi], eta[lo:hi], *gG)
            for i in range(3):
                dW[i] = dW[i] + r[i]
            dk[lo:hi] += r[3]
            dv[lo:hi] += r[4]
            deta[lo:hi] += r[5]
        for j in reads.get(t, []):  # the queries that read the weights of this point
            lo, hi = bounds[j]
            r = swiglu_apply_backward(Wt[0], Wt[1], Wt[2], q[lo:hi], dO[lo:hi])
            dq[lo:hi] += r[0]
            for i in range(3):
                dW[i] = dW[i] + r[1 + i]
    return dq, dk, dv, deta, tuple(dW)


def ttt_backward_ref(q, k, v, eta, W1, W3, W2, chunk, mask, dO, dW_out=None, update_chunks=None, inner_steps=1,
                     ascent=False, momentum=0.0, rule=UPD_GD, last_layer_only=False, slices=None, ns_iters=5):
    """ttt_backward_scan_ref over [B, H, N, d] inputs.  W1, W3, W2 are per head ([H, ...]) or per
    (batch, head) ([B, H, ...]); the weight gradients take the same shape (per-head weights sum over
    the batch).  dW_out is None or three [B, H, ...] arrays.  Returns (dq, dk, dv, deta, (dW1, dW3,
    dW2))."""
    B, H, N, d = q.shape
    per_head = W1.ndim == 3
    dq, dk, dv = np.zeros((B, H, N, d)), np.zeros((B, H, N, d)), np.zeros((B, H, N, d))
    deta = np.zeros((B, H, N))
    dW = [np.zeros(x.shape) for x in (W1, W3, W2)]
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        ws = [x[h] if per_head else x[b, h] for x in (W1, W3, W2)]
        dwo = None if dW_out is None else tuple(x[b, h] for x in dW_out)
        r = ttt_backward_scan_ref(q[b, h], k[b, h], v[b, h], eta[b, h], *ws, chunk, mask, dO[b, h], dwo,
                                  update_chunks, inner_steps, ascent, momentum, rule, last_layer_only, ns_iters)
        dq[b, h], dk[b, h], dv[b, h], deta[b, h] = r[:4]
        for i in range(3):
            if per_head:
                dW[i][h] += r[4][i]
            else:
                dW[i][b, h] = r[4][i]
    return dq, dk, dv, deta, tuple(dW)
