"""Seeded synthetic inputs for the large-chunk TTT-KVB layer and chunked linear attention.

This module only draws random numbers and rounds them to the storage precision.  It contains
none of the layer's arithmetic, so both the fp64 CPU oracle and the HIP path can be fed from it
without sharing any compute code.

Recipe (per (batch, head) slice, so any slice can be regenerated on its own):
  * ``numpy.random.default_rng([seed, b, h])`` draws, in this order, q, k, v as
    N(0, 1) / sqrt(d) arrays of shape [N, d], then one standard-normal ``eta_raw`` per token;
  * eta = 0.01 * softplus(eta_raw) (LaCT layer workloads) or 0.05 * sigmoid(eta_raw)
    (linear-attention workload); eta is a per-token, per-head learning rate, kept in fp32;
  * the initial fast weights of head h come from ``default_rng([seed, 10**6 + h])``, drawing
    W1 (m x d), W3 (m x d), W2 (d x m) with entries N(0, 1/d), stored fp32;
  * q, k, v are rounded once, round-to-nearest-even, to bfloat16 when the workload runs in bf16;
    the rounded values (held in float32 arrays) are what every consumer sees;
  * the backward's upstream gradients of slice (b, h) come from ``default_rng([seed, b, h, 7])``:
    dO [N, d_v] with entries N(0, 1) / sqrt(d_v) (rounded to bfloat16 for bf16 workloads), then
    dS_out [d_v, d_k] with entries N(0, 1) / sqrt(d_k), kept in fp32;
  * the TTT layer's upstream gradients of slice (b, h) come from ``default_rng([seed, b, h, 8])``:
    dO [N, d] with entries N(0, 1) / sqrt(d) (rounded to bfloat16 for bf16 workloads), then the
    gradients of the returned fast weights dW1 (m x d), dW3 (m x d), dW2 (d x m) with entries
    N(0, 1) / sqrt(d), kept in fp32.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "round_to_bf16",
    "bf16_bits",
    "slice_inputs",
    "head_weights",
    "make_ttt_inputs",
    "make_linattn_inputs",
    "grad_slice",
    "make_linattn_grads",
    "layer_grad_slice",
    "make_ttt_grads",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # add 0x7FFF plus the lowest kept bit, then truncate: the usual RNE for 16 dropped bits
    out = np.right_shift(bits, np.uint32(16))
    np.bitwise_and(out, np.uint32(1), out=out)
    np.add(out, np.uint32(0x7FFF), out=out)
    np.add(out, bits, out=out)
    np.bitwise_and(out, np.uint32(0xFFFF0000), out=out)
    out = out.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def slice_inputs(seed: int, b: int, h: int, N: int, d_k: int, d_v: int | None = None,
                 eta_kind: str = "softplus", eta_scale: float = 0.01, bf16: bool = True):
    """q, k [N, d_k], v [N, d_v] and eta [N] for one (batch, head) slice."""
    d_v = d_k if d_v is None else d_v
    rng = np.random.default_rng([seed, b, h])
    scale = np.float32(np.sqrt(d_k))
    q = np.divide(rng.standard_normal((N, d_k), dtype=np.float32), scale, dtype=np.float32)
    k = np.divide(rng.standard_normal((N, d_k), dtype=np.float32), scale, dtype=np.float32)
    v = np.divide(rng.standard_normal((N, d_v), dtype=np.float32), scale, dtype=np.float32)
    raw = rng.standard_normal(N).astype(np.float32)
    if eta_kind == "softplus":
        eta = (eta_scale * _softplus(raw.astype(np.float64))).astype(np.float32)
    elif eta_kind == "sigmoid":
        eta = (eta_scale * _sigmoid(raw.astype(np.float64))).astype(np.float32)
    elif eta_kind == "const":
        eta = np.full(N, eta_scale, dtype=np.float32)
    else:
        raise ValueError(f"unknown eta_kind {eta_kind!r}")
    if bf16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v, eta


def head_weights(seed: int, h: int, d: int, m: int):
    """Initial fast weights W1 (m x d), W3 (m x d), W2 (d x m) of head h, entries N(0, 1/d), fp32."""
    rng = np.random.default_rng([seed, 10**6 + h])
    s = np.float32(1.0 / np.sqrt(d))
    W1 = (rng.standard_normal((m, d), dtype=np.float32) * s).astype(np.float32)
    W3 = (rng.standard_normal((m, d), dtype=np.float32) * s).astype(np.float32)
    W2 = (rng.standard_normal((d, m), dtype=np.float32) * s).astype(np.float32)
    return W1, W3, W2


def make_ttt_inputs(seed: int, B: int, H: int, N: int, d: int, m: int, bf16: bool = True,
                    eta_kind: str = "softplus", eta_scale: float = 0.01, slices=None):
    """Full [B, H, N, d] q, k, v, [B, H, N] eta and per-head W1, W3, W2 stacks [H, ...].

    ``slices`` optionally restricts generation to a list of (b, h) pairs (others stay zero);
    every generated slice is identical to the one a full generation would give.
    """
    q = np.zeros((B, H, N, d), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    eta = np.zeros((B, H, N), np.float32)
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        q[b, h], k[b, h], v[b, h], eta[b, h] = slice_inputs(seed, b, h, N, d, d, eta_kind, eta_scale, bf16)
    W1 = np.zeros((H, m, d), np.float32)
    W3 = np.zeros((H, m, d), np.float32)
    W2 = np.zeros((H, d, m), np.float32)
    for h in range(H):
        W1[h], W3[h], W2[h] = head_weights(seed, h, d, m)
    return q, k, v, eta, W1, W3, W2


def make_linattn_inputs(seed: int, B: int, H: int, N: int, d_k: int, d_v: int, bf16: bool = True,
                        eta_kind: str = "sigmoid", eta_scale: float = 0.05, slices=None):
    """q, k [B, H, N, d_k], v [B, H, N, d_v], eta [B, H, N] for the linear-attention workload."""
    q = np.zeros((B, H, N, d_k), np.float32)
    k = np.zeros_like(q)
    v = np.zeros((B, H, N, d_v), np.float32)
    eta = np.zeros((B, H, N), np.float32)
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        q[b, h], k[b, h], v[b, h], eta[b, h] = slice_inputs(seed, b, h, N, d_k, d_v, eta_kind, eta_scale, bf16)
    return q, k, v, eta


def grad_slice(seed: int, b: int, h: int, N: int, d_k: int, d_v: int, bf16: bool = True):
    """Upstream gradients of one (batch, head) slice: dO [N, d_v] and dS_out [d_v, d_k] (fp32)."""
    rng = np.random.default_rng([seed, b, h, 7])
    dO = np.divide(rng.standard_normal((N, d_v), dtype=np.float32), np.float32(np.sqrt(d_v)), dtype=np.float32)
    dS = np.divide(rng.standard_normal((d_v, d_k), dtype=np.float32), np.float32(np.sqrt(d_k)), dtype=np.float32)
    if bf16:
        dO = round_to_bf16(dO)
    return dO, dS


def make_linattn_grads(seed: int, B: int, H: int, N: int, d_k: int, d_v: int, bf16: bool = True, slices=None):
    """dO [B, H, N, d_v] and dS_out [B, H, d_v, d_k] (slices not listed stay zero)."""
    dO = np.zeros((B, H, N, d_v), np.float32)
    dS = np.zeros((B, H, d_v, d_k), np.float32)
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        dO[b, h], dS[b, h] = grad_slice(seed, b, h, N, d_k, d_v, bf16)
    return dO, dS


def layer_grad_slice(seed: int, b: int, h: int, N: int, d: int, m: int, bf16: bool = True):
    """Upstream gradients of one (batch, head) slice of the TTT layer: dO [N, d] and the gradients
    of the returned fast weights (dW1 [m, d], dW3 [m, d], dW2 [d, m], fp32)."""
    rng = np.random.default_rng([seed, b, h, 8])
    s = np.float32(np.sqrt(d))
    dO = np.divide(rng.standard_normal((N, d), dtype=np.float32), s, dtype=np.float32)
    dW = tuple(np.divide(rng.standard_normal(shape, dtype=np.float32), s, dtype=np.float32)
               for shape in ((m, d), (m, d), (d, m)))
    if bf16:
        dO = round_to_bf16(dO)
    return dO, dW


def make_ttt_grads(seed: int, B: int, H: int, N: int, d: int, m: int, bf16: bool = True, slices=None):
    """dO [B, H, N, d] and (dW1 [B, H, m, d], dW3 [B, H, m, d], dW2 [B, H, d, m]) (slices not listed
    stay zero)."""
    dO = np.zeros((B, H, N, d), np.float32)
    dW = (np.zeros((B, H, m, d), np.float32), np.zeros((B, H, m, d), np.float32), np.zeros((B, H, d, m), np.float32))
    todo = [(b, h) for b in range(B) for h in range(H)] if slices is None else list(slices)
    for b, h in todo:
        dO[b, h], ws = layer_grad_slice(seed, b, h, N, d, m, bf16)
        for i in range(3):
            dW[i][b, h] = ws[i]
    return dO, dW
