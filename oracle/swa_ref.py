"""Plain fp64 CPU oracle for the sliding-window attention that sits beside the TTT layer in LaCT.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU-baseline
leg, never by the product path; it shares no code with the HIP library.

Source: the PaperTrace page "5.2.1 LaCT and TTT-E2E", section 1.1 (the paragraphs on window
attention) and the remark after Eq. (10).  In language modelling LaCT adds, beside the fast-weight
branch, a sliding-window attention whose window equals the chunk (2048 or 4096 tokens); it shares
Q, K and V with the fast-weight branch and gives Q and K a per-channel scale and shift.  Under the
apply-then-update order of Eq. (10) the fast weights see a chunk only from the next chunk on, and a
causal window as wide as the chunk covers exactly that gap.

Readings where the page is silent (each also listed in the design notes):
* the attention is softmax attention with the usual 1/sqrt(d) scale on the scores;
* "sliding window of w tokens, causal": token t attends to the tokens s with t - w < s <= t
  (itself and the w - 1 before it);
* the per-channel scale and shift are parameters of each head: q' = q * gamma_q + beta_q and
  k' = k * gamma_k + beta_k, channel by channel, applied before the scores; v is used as is;
* heads of the window attention are the fast-weight branch's heads (shared Q, K, V).

Parity status: pinned by the CPU tests (brute-force loops, full causal attention through torch's
own routine when the window covers the sequence, the one-token window, the shift invariance of
softmax, the convex-hull bound).
"""
from __future__ import annotations

import numpy as np


def swa_scan_ref(q, k, v, window, q_scale=None, q_shift=None, k_scale=None, k_shift=None):
    """One (batch, head) slice: q, k, v [N, d]; the per-channel scale/shift vectors [d] or None
    (identity).  Returns o [N, d]."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, d = q.shape
    qs = np.ones(d) if q_scale is None else np.asarray(q_scale, np.float64)
    qb = np.zeros(d) if q_shift is None else np.asarray(q_shift, np.float64)
    ks = np.ones(d) if k_scale is None else np.asarray(k_scale, np.float64)
    kb = np.zeros(d) if k_shift is None else np.asarray(k_shift, np.float64)
    qp = q * qs + qb
    kp = k * ks + kb
    o = np.zeros((N, v.shape[1]))
    for t in range(N):
        lo = max(0, t - window + 1)
        s = (kp[lo:t + 1] @ qp[t]) / np.sqrt(d)
        w = np.exp(s - s.max())
        o[t] = (w / w.sum()) @ v[lo:t + 1]
    return o


def swa_forward_ref(q, k, v, window, q_scale=None, q_shift=None, k_scale=None, k_shift=None, slices=None):
    """[B, H, N, d] inputs; the scale/shift parameters are [H, d] (or None).  ``slices`` restricts the
    work to a list of (b, h) pairs (the other outputs stay zero)."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]))
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    pick = lambda p, h: None if p is None else p[h]
    for b, h in todo:
        o[b, h] = swa_scan_ref(q[b, h], k[b, h], v[b, h], window, pick(q_scale, h), pick(q_shift, h),
                               pick(k_scale, h), pick(k_shift, h))
    return o
