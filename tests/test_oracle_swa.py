"""Pins of the sliding-window attention oracle (CPU only), each against an independent route:
brute-force loops, torch's own scaled-dot-product attention when the window covers the sequence,
the one-token window, softmax's invariance to a per-key-independent shift, and the convex hull."""
import math

import numpy as np
import pytest

import oracle as O


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def problem(seed, N=9, d=3, dv=None):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    q, k = rng.standard_normal((2, N, d))
    v = rng.standard_normal((N, dv))
    gq, gk = 0.5 + rng.random((2, d))
    bq, bk = 0.3 * rng.standard_normal((2, d))
    return q, k, v, gq, bq, gk, bk


def loops(q, k, v, window, gq, bq, gk, bk):
    """Scalar loops of softmax((q' . k') / sqrt(d)) over t - window < s <= t."""
    N, d = q.shape
    out = np.zeros_like(v)
    for t in range(N):
        keys = [s for s in range(N) if t - window < s <= t]
        sc = []
        for s in keys:
            sc.append(sum((q[t, c] * gq[c] + bq[c]) * (k[s, c] * gk[c] + bk[c]) for c in range(d)) / math.sqrt(d))
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = sum(w)
        for j, s in enumerate(keys):
            for e in range(v.shape[1]):
                out[t, e] += w[j] / tot * v[s, e]
    return out


@pytest.mark.parametrize("window", [1, 2, 3, 5, 9, 20])
def test_swa_matches_loops(window):
    q, k, v, gq, bq, gk, bk = problem(window, dv=4)
    got = O.swa_scan_ref(q, k, v, window, gq, bq, gk, bk)
    assert rel(got, loops(q, k, v, window, gq, bq, gk, bk)) < 1e-13


def test_window_covering_the_sequence_is_causal_attention():
    torch = pytest.importorskip("torch")
    q, k, v, gq, bq, gk, bk = problem(11, N=17, d=5)
    got = O.swa_scan_ref(q, k, v, 17, gq, bq, gk, bk)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    want = torch.nn.functional.scaled_dot_product_attention(t(q * gq + bq), t(k * gk + bk), t(v), is_causal=True)
    assert rel(got, want[0, 0].numpy()) < 1e-13
    # and any wider window gives the same
    assert rel(O.swa_scan_ref(q, k, v, 1000, gq, bq, gk, bk), got) == 0.0


def test_one_token_window_returns_v():
    q, k, v, gq, bq, gk, bk = problem(12, N=10)
    assert rel(O.swa_scan_ref(q, k, v, 1, gq, bq, gk, bk), v) < 1e-15


def test_key_shift_does_not_change_the_output_query_shift_does():
    """(q') . (k' + c) = q'.k' + q'.c, and q'.c is the same for every key of one query: softmax drops
    it.  So the key shift never changes the output, while the query shift (which scales with every
    key differently) does; a shift applied to the wrong operand fails one of the two."""
    q, k, v, gq, bq, gk, bk = problem(13, N=12, d=4)
    base = O.swa_scan_ref(q, k, v, 5, gq, bq, gk, None)
    assert rel(O.swa_scan_ref(q, k, v, 5, gq, bq, gk, bk), base) < 1e-13
    assert rel(O.swa_scan_ref(q, k, v, 5, gq, None, gk, bk), base) > 1e-3


def test_outputs_lie_in_the_windows_value_range():
    q, k, v, gq, bq, gk, bk = problem(14, N=15, d=3)
    o = O.swa_scan_ref(q, k, v, 4, gq, bq, gk, bk)
    for t in range(15):
        win = v[max(0, t - 3):t + 1]
        assert (o[t] >= win.min(axis=0) - 1e-12).all() and (o[t] <= win.max(axis=0) + 1e-12).all()


def test_forward_ref_slices_and_per_head_parameters():
    rng = np.random.default_rng(15)
    B, H, N, d = 2, 3, 8, 4
    q, k, v = rng.standard_normal((3, B, H, N, d))
    gq, gk = 0.5 + rng.random((2, H, d))
    bq, bk = rng.standard_normal((2, H, d))
    o = O.swa_forward_ref(q, k, v, 3, gq, bq, gk, bk)
    for b in range(B):
        for h in range(H):
            assert rel(o[b, h], loops(q[b, h], k[b, h], v[b, h], 3, gq[h], bq[h], gk[h], bk[h])) < 1e-13
    o1 = O.swa_forward_ref(q, k, v, 3, gq, bq, gk, bk, slices=[(1, 2)])
    assert rel(o1[1, 2], o[1, 2]) == 0.0 and not o1[0].any()
    # identity parameters (None) are scale 1, shift 0
    assert rel(O.swa_forward_ref(q, k, v, 3), O.swa_forward_ref(q, k, v, 3, np.ones((H, d)), np.zeros((H, d)),
                                                                np.ones((H, d)), np.zeros((H, d)))) == 0.0
