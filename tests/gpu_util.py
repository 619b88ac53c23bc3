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
