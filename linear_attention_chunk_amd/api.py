"""Thin PyTorch binding of the C ABI: argument checks, output/workspace allocation, the call.

Tensors provide device memory and the stream; every step of the computation runs in libttt.so.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib as C

_DT = {torch.bfloat16: C.TTT_BF16, torch.float32: C.TTT_F32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def pack_weights(W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor) -> torch.Tensor:
    """[..., m, d], [..., m, d], [..., d, m] -> [..., 3*d*m] fp32 blocks [W1 | W3 | W2]."""
    lead = W1.shape[:-2]
    return torch.cat([W1.reshape(*lead, -1), W3.reshape(*lead, -1), W2.reshape(*lead, -1)], dim=-1).float().contiguous()


def unpack_weights(W: torch.Tensor, d: int, m: int):
    """Inverse of pack_weights."""
    dm = d * m
    lead = W.shape[:-1]
    return (W[..., :dm].reshape(*lead, m, d), W[..., dm:2 * dm].reshape(*lead, m, d),
            W[..., 2 * dm:].reshape(*lead, d, m))


def ttt_desc(B, H, N, d_h, m_h, chunk, io_dtype, mask, rule, ns_iters=5, momentum=0.0, last_layer_only=False,
             w0_per_batch=False, update_chunks: Optional[Sequence[int]] = None, inner_steps: int = 1,
             ascent: bool = False, parallel_form: bool = False):
    """A filled TttDesc plus the host buffer that keeps update_chunks alive."""
    flags = None
    if update_chunks is not None:
        flags = (ctypes.c_uint8 * len(update_chunks))(*[1 if f else 0 for f in update_chunks])
    D = C.TttDesc(B, H, N, d_h, m_h, chunk, io_dtype, mask, rule, ns_iters, float(momentum), int(last_layer_only),
                  int(w0_per_batch), ctypes.cast(flags, ctypes.c_void_p) if flags is not None else None,
                  int(inner_steps), int(ascent), int(parallel_form))
    return D, flags


def ttt_workspace_bytes(desc: C.TttDesc) -> int:
    n = ctypes.c_size_t(0)
    C.check(C.lib().ttt_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ttt_forward(q, k, v, eta, W0, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE,
                update_rule: int = C.UPD_GD_L2, *, m_h: Optional[int] = None, ns_iters: int = 5,
                momentum: float = 0.0, last_layer_only: bool = False, update_chunks=None,
                M: Optional[torch.Tensor] = None, want_W: bool = True, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None, inner_steps: int = 1,
                ascent: bool = False, parallel_form: bool = False):
    """The TTT-KVB layer through ttt_forward of libttt.so.

    q, k, v [B, H, N, d] (bf16 or fp32, same dtype); eta [B, H, N] fp32; W0 fp32 [H, 3*d*m] or
    [B, H, 3*d*m] (see pack_weights).  M, if given, is the [B, H, 3*d*m] fp32 momentum, updated
    in place.  parallel_form (last_layer_only with plain GD only) computes the same layer as
    chunked linear attention over the frozen SwiGLU features.  Returns (o, W_out or None).
    """
    B, H, N, d = q.shape
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
        if t.shape != q.shape:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(q.shape)}")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    _need(eta, "eta", torch.float32, dev)
    if tuple(eta.shape) != (B, H, N):
        raise ValueError("eta must be [B, H, N]")
    _need(W0, "W0", torch.float32, dev)
    per_batch = W0.dim() == 3
    if m_h is None:
        m_h = W0.shape[-1] // (3 * d)
    if W0.shape[-1] != 3 * d * m_h or (per_batch and tuple(W0.shape[:2]) != (B, H)) or (
            not per_batch and (W0.dim() != 2 or W0.shape[0] != H)):
        raise ValueError("W0 must be [H, 3*d*m] or [B, H, 3*d*m]")
    D, keep = ttt_desc(B, H, N, d, m_h, chunk, _DT[q.dtype], mask_mode, update_rule, ns_iters, momentum,
                       last_layer_only, per_batch, update_chunks, inner_steps, ascent, parallel_form)
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", q.dtype, dev)
    W_out = torch.empty((B, H, 3 * d * m_h), dtype=torch.float32, device=dev) if want_W else None
    if M is not None:
        _need(M, "M", torch.float32, dev)
    nbytes = ttt_workspace_bytes(D)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = C.lib().ttt_forward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(W0), _ptr(o), _ptr(W_out),
                             _ptr(M), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream_handle(stream))
    del keep
    C.check(st)
    return o, W_out


def linattn_desc(B, H, N, d_k, d_v, chunk, io_dtype, mask, update_chunks=None):
    flags = None
    if update_chunks is not None:
        flags = (ctypes.c_uint8 * len(update_chunks))(*[1 if f else 0 for f in update_chunks])
    D = C.LinattnDesc(B, H, N, d_k, d_v, chunk, io_dtype, mask,
                      ctypes.cast(flags, ctypes.c_void_p) if flags is not None else None)
    return D, flags


def linattn_workspace_bytes(desc: C.LinattnDesc) -> int:
    n = ctypes.c_size_t(0)
    C.check(C.lib().linattn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def linattn_forward(q, k, v, eta, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE, *,
                    S0: Optional[torch.Tensor] = None, update_chunks=None, want_S: bool = True,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Chunked linear attention through linattn_forward of libttt.so.  Returns (o, S_out or None)."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", None, dev)
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape[:3]) != (B, H, N):
        raise ValueError("q, k must be [B, H, N, d_k] and v [B, H, N, d_v]")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    _need(eta, "eta", torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, dev)
    D, keep = linattn_desc(B, H, N, dk, dv, chunk, _DT[q.dtype], mask_mode, update_chunks)
    o = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev) if out is None else out
    S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_S else None
    nbytes = linattn_workspace_bytes(D)
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = C.lib().linattn_forward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(S0), _ptr(o),
                                 _ptr(S_out), _ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                                 _stream_handle(stream))
    del keep
    C.check(st)
    return o, S_out
