"""Helpers for the GPU parity tests: device inputs from the seeded generators, error metrics."""
import sys

import numpy as np
import torch

import synth


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bulk_ttt_inputs(seed, B, H, N, d, m, bf16, eta_kind="softplus", eta_scale=0.01, exact=None):
    """Device inputs for a whole workload.

    Slices listed in `exact` ((b, h) pairs) come from the seeded generator module and are the ones
    compared with the oracle; the others are filled with the same distributions by torch's seeded
    generator on the device (cheap at full size).  W0 is always the generator's per-head weights.
    Returns (q, k, v, eta, W0 [H, 3dm], host dict of the exact slices, (W1, W3, W2) host).
    """
    dt = torch.bfloat16 if bf16 else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(10_000 + seed)
    s = 1.0 / np.sqrt(d)
    q = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(dt)
    k = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(dt)
    v = (torch.randn((B, H, N, d), generator=g, device="cuda") * s).to(dt)
    raw = torch.randn((B, H, N), generator=g, device="cuda")
    eta = (eta_scale * (torch.nn.functional.softplus(raw) if eta_kind == "softplus" else torch.sigmoid(raw))).float()
    ex = {}
    for (b, h) in (exact or []):
        qs, ks, vs, es = synth.slice_inputs(seed, b, h, N, d, d, eta_kind, eta_scale, bf16)
        q[b, h] = dev(qs, dt)
        k[b, h] = dev(ks, dt)
        v[b, h] = dev(vs, dt)
        eta[b, h] = dev(es)
        ex[(b, h)] = (qs, ks, vs, es)
    W = [np.zeros((H, m, d), np.float32), np.zeros((H, m, d), np.float32), np.zeros((H, d, m), np.float32)]
    for h in range(H):
        W[0][h], W[1][h], W[2][h] = synth.head_weights(seed, h, d, m)
    W0 = dev(np.concatenate([W[0].reshape(H, -1), W[1].reshape(H, -1), W[2].reshape(H, -1)], axis=1))
    return q, k, v, eta, W0, ex, W


def full_ttt_inputs(seed, B, H, N, d, m, bf16, eta_kind="softplus", eta_scale=0.01):
    """Every slice from the seeded generator (small workloads)."""
    q, k, v, eta, W1, W3, W2 = synth.make_ttt_inputs(seed, B, H, N, d, m, bf16, eta_kind, eta_scale)
    dt = torch.bfloat16 if bf16 else torch.float32
    W0 = dev(np.concatenate([W1.reshape(H, -1), W3.reshape(H, -1), W2.reshape(H, -1)], axis=1))
    return (dev(q, dt), dev(k, dt), dev(v, dt), dev(eta), W0), (q, k, v, eta, W1, W3, W2)


# Per-row bound, as a multiple of the relative-L2 tolerance: a row is one token's output vector or
# one row of a weight matrix.  Rounding spreads evenly over the rows, so a healthy result stays
# well inside it, while one wrong row (a chunk edge, the ragged tail, one head) breaks it even
# where the whole-tensor figure would hide it.
ROW_FACTOR = 5.0


def row_rel(a, b):
    """Per-row relative L2 error over the last axis."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def assert_close(g, r, tol, name, chunk=None):
    """Relative L2 of g against r over the whole tensor, per leading slice ([..., rows, cols]: every
    index but the last two), per chunk of rows (if chunk is given) must each be <= tol, and every
    row's relative error <= ROW_FACTOR * tol.  Returns the figures (also printed)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    whole = rel(g, r)
    lead = g.reshape(-1, *g.shape[-2:])
    lr = r.reshape(-1, *r.shape[-2:])
    per_slice = max(rel(a, b) for a, b in zip(lead, lr)) if lead.size else 0.0
    per_chunk = 0.0
    if chunk is not None and g.shape[-2] > 0:
        n = g.shape[-2]
        for lo in range(0, n, chunk):
            for a, b in zip(lead, lr):
                per_chunk = max(per_chunk, rel(a[lo:lo + chunk], b[lo:lo + chunk]))
    per_row = float(row_rel(g, r).max()) if g.size else 0.0
    say(f"    {name}: rel={whole:.3e} worst slice={per_slice:.3e} worst chunk={per_chunk:.3e} "
        f"worst row={per_row:.3e} (tol {tol}, rows {ROW_FACTOR * tol:g})")
    assert whole <= tol, f"{name}: relative L2 {whole} > {tol}"
    assert per_slice <= tol, f"{name}: worst (batch, head) relative L2 {per_slice} > {tol}"
    assert per_chunk <= tol, f"{name}: worst chunk relative L2 {per_chunk} > {tol}"
    assert per_row <= ROW_FACTOR * tol, f"{name}: worst row relative error {per_row} > {ROW_FACTOR * tol}"
    return whole, per_slice, per_chunk, per_row
