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


def _need(t: torch.Tensor, name: str, dtype=None, device=None, shape=None):
    """Checks one tensor argument: exact shape and dtype first, then that it is a contiguous tensor on
    the call's device.  The library writes through these pointers on the device, so every mismatch
    is a ValueError here instead of a fault or wrong results there."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> Optional[torch.Tensor]:
    """The caller's workspace after checks (a contiguous uint8 device tensor of at least nbytes), or a
    new one when none is given."""
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes else None
    _need(ws, "workspace", torch.uint8, device)
    if ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {nbytes}")
    return ws


def _need_bytes(t: torch.Tensor, name: str, nbytes: int, device):
    """A contiguous uint8 device tensor of at least nbytes (a record)."""
    _need(t, name, torch.uint8, device)
    if t.numel() < nbytes:
        raise ValueError(f"{name} holds {t.numel()} bytes, the call needs {nbytes}")


def _flags(update_chunks, N: int, chunk: int, strided: bool, name="update_chunks"):
    """update_chunks must hold a flag for every chunk (the library reads ceil(N / chunk) of them)."""
    if update_chunks is None:
        if strided and N > 0:
            raise ValueError(f"the strided mask needs {name}")
        return
    need = -(-N // chunk) if chunk > 0 else 0
    if len(update_chunks) < need:
        raise ValueError(f"{name} has {len(update_chunks)} flags, the sequence has {need} chunks")


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
             ascent: bool = False, parallel_form: bool = False, chunk_rates: bool = False,
             chunk_momentum: Optional[torch.Tensor] = None):
    """A filled TttDesc plus the host buffer that keeps update_chunks alive."""
    flags = None
    if update_chunks is not None:
        flags = (ctypes.c_uint8 * len(update_chunks))(*[1 if f else 0 for f in update_chunks])
    D = C.TttDesc(B, H, N, d_h, m_h, chunk, io_dtype, mask, rule, ns_iters, float(momentum), int(last_layer_only),
                  int(w0_per_batch), ctypes.cast(flags, ctypes.c_void_p) if flags is not None else None,
                  int(inner_steps), int(ascent), int(parallel_form), int(chunk_rates), _ptr(chunk_momentum))
    return D, flags


def ttt_workspace_bytes(desc: C.TttDesc) -> int:
    n = ctypes.c_size_t(0)
    C.check(C.lib().ttt_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _ttt_prepare(q, k, v, eta, W0, chunk, mask_mode, update_rule, m_h, ns_iters, momentum, last_layer_only,
                 update_chunks, M, want_W, out, inner_steps, ascent, parallel_form, chunk_rates=False,
                 chunk_momentum=None):
    """Argument checks shared by ttt_forward and ttt_forward_noalloc; returns the descriptor, the
    host buffer keeping update_chunks alive, the output and W_out tensors."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B, H, N, d] tensor")
    B, H, N, d = q.shape
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev, q.shape)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    nc = -(-N // chunk)
    _need(eta, "eta", torch.float32, dev, (B, H, nc) if chunk_rates else (B, H, N))
    if chunk_momentum is not None:
        if not chunk_rates:
            raise ValueError("chunk_momentum needs chunk_rates")
        _need(chunk_momentum, "chunk_momentum", torch.float32, dev, (B, H, nc))
    if not isinstance(W0, torch.Tensor) or W0.dim() not in (2, 3):
        raise ValueError("W0 must be [H, 3*d*m] or [B, H, 3*d*m]")
    per_batch = W0.dim() == 3
    if m_h is None:
        m_h = W0.shape[-1] // (3 * d)
    _need(W0, "W0", torch.float32, dev, ((B, H) if per_batch else (H,)) + (3 * d * m_h,))
    _flags(update_chunks, N, chunk, mask_mode == C.MASK_STRIDED)
    wshape = (B, H, 3 * d * m_h)
    if out is not None:
        _need(out, "out", q.dtype, dev, q.shape)
    if M is not None:
        _need(M, "M", torch.float32, dev, wshape)
    D, keep = ttt_desc(B, H, N, d, m_h, chunk, _DT[q.dtype], mask_mode, update_rule, ns_iters, momentum,
                       last_layer_only, per_batch, update_chunks, inner_steps, ascent, parallel_form, chunk_rates,
                       chunk_momentum)
    o = torch.empty_like(q) if out is None else out
    W_out = torch.empty(wshape, dtype=torch.float32, device=dev) if want_W else None
    return D, keep, o, W_out


def ttt_forward(q, k, v, eta, W0, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE,
                update_rule: int = C.UPD_GD_L2, *, m_h: Optional[int] = None, ns_iters: int = 5,
                momentum: float = 0.0, last_layer_only: bool = False, update_chunks=None,
                M: Optional[torch.Tensor] = None, want_W: bool = True, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None, inner_steps: int = 1,
                ascent: bool = False, parallel_form: bool = False, chunk_rates: bool = False,
                chunk_momentum: Optional[torch.Tensor] = None):
    """The TTT-KVB layer through ttt_forward of libttt.so.

    q, k, v [B, H, N, d] (bf16 or fp32, same dtype); eta [B, H, N] fp32; W0 fp32 [H, 3*d*m] or
    [B, H, 3*d*m] (see pack_weights).  M, if given, is the [B, H, 3*d*m] fp32 momentum, updated
    in place.  parallel_form (last_layer_only with plain GD only) computes the same layer as
    chunked linear attention over the frozen SwiGLU features.  chunk_rates: eta is [B, H, chunks], one
    rate per chunk outside the optimizer step, with per-chunk momentum factors chunk_momentum
    [B, H, chunks] (or None).  Returns (o, W_out or None).
    """
    D, keep, o, W_out = _ttt_prepare(q, k, v, eta, W0, chunk, mask_mode, update_rule, m_h, ns_iters, momentum,
                                     last_layer_only, update_chunks, M, want_W, out, inner_steps, ascent,
                                     parallel_form, chunk_rates, chunk_momentum)
    nbytes = ttt_workspace_bytes(D)
    workspace = _workspace(workspace, nbytes, q.device)
    st = C.lib().ttt_forward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(W0), _ptr(o), _ptr(W_out),
                             _ptr(M), _ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                             _stream_handle(stream))
    del keep
    C.check(st)
    return o, W_out


def ttt_record_bytes(desc: C.TttDesc):
    """(record bytes, workspace bytes) of ttt_forward_record for this descriptor."""
    r, w = ctypes.c_size_t(0), ctypes.c_size_t(0)
    C.check(C.lib().ttt_record_bytes(ctypes.byref(desc), ctypes.byref(r), ctypes.byref(w)))
    return r.value, w.value


def ttt_forward_record(q, k, v, eta, W0, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE,
                       update_rule: int = C.UPD_GD_L2, *, m_h: Optional[int] = None, ns_iters: int = 5,
                       momentum: float = 0.0, last_layer_only: bool = False, update_chunks=None,
                       inner_steps: int = 1, ascent: bool = False, out: Optional[torch.Tensor] = None,
                       record: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """The training forward through ttt_forward_record of libttt.so: o and W_out as ttt_forward
    returns them (momentum from zero), and the record that ttt_backward(..., record=) reads instead
    of running the forward again (a uint8 device tensor, allocated here unless given).
    Returns (o, W_out, record)."""
    D, keep, o, W_out = _ttt_prepare(q, k, v, eta, W0, chunk, mask_mode, update_rule, m_h, ns_iters, momentum,
                                     last_layer_only, update_chunks, None, True, out, inner_steps, ascent, False)
    rbytes, wbytes = ttt_record_bytes(D)
    record = _workspace(record, rbytes, q.device)
    workspace = _workspace(workspace, wbytes, q.device)
    st = C.lib().ttt_forward_record(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(W0), _ptr(o),
                                    _ptr(W_out), _ptr(record), ctypes.c_size_t(0 if record is None else record.numel()),
                                    _ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                                    _stream_handle(stream))
    del keep
    C.check(st)
    return o, W_out, record


def ttt_forward_noalloc(q, k, v, eta, W0, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE,
                        update_rule: int = C.UPD_GD_L2, *, m_h: Optional[int] = None, ns_iters: int = 5,
                        momentum: float = 0.0, last_layer_only: bool = False, update_chunks=None,
                        M: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        W_out: Optional[torch.Tensor] = None, stream=None, inner_steps: int = 1,
                        ascent: bool = False, parallel_form: bool = False, chunk_rates: bool = False,
                        chunk_momentum: Optional[torch.Tensor] = None):
    """ttt_forward through ttt_forward_noalloc: the library's static device scratch replaces the
    workspace, and the library allocates nothing.  Pass `out` (and `W_out`, [B, H, 3*d*m] fp32, or
    None to skip the final weights) to keep this wrapper from allocating too.  Returns (o, W_out)."""
    D, keep, o, _ = _ttt_prepare(q, k, v, eta, W0, chunk, mask_mode, update_rule, m_h, ns_iters, momentum,
                                 last_layer_only, update_chunks, M, False, out, inner_steps, ascent, parallel_form,
                                 chunk_rates, chunk_momentum)
    if W_out is not None:
        _need(W_out, "W_out", torch.float32, q.device, (D.B, D.H, 3 * D.d_h * D.m_h))
    st = C.lib().ttt_forward_noalloc(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(W0), _ptr(o),
                                     _ptr(W_out), _ptr(M), _stream_handle(stream))
    del keep
    C.check(st)
    return o, W_out


def ttt_backward_workspace_bytes(desc: C.TttDesc) -> int:
    n = ctypes.c_size_t(0)
    C.check(C.lib().ttt_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ttt_backward(q, k, v, eta, W0, dO, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE, *,
                 m_h: Optional[int] = None, dW_out: Optional[torch.Tensor] = None, want_dW0: bool = True,
                 update_chunks=None, inner_steps: int = 1, ascent: bool = False, momentum: float = 0.0,
                 update_rule: int = C.UPD_GD, last_layer_only: bool = True, ns_iters: int = 5,
                 record: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of ttt_forward (momentum as a forward call without M, i.e. from zero), through
    ttt_backward of libttt.so: with last_layer_only the layer whose inner loop trains W2 alone,
    otherwise the recurrence with all three weights learning; ns_iters as for ttt_forward (Muon).
    record: the record ttt_forward_record wrote for the same inputs (through ttt_backward_record:
    the forward is not run again; W0 is then not read).

    dO [B, H, N, d] is the gradient of o, dW_out ([B, H, 3*d*m] fp32 or None) that of W_out.
    Returns (dq, dk, dv, deta, dW0 or None); dW0 has W0's shape (per-head weights sum over the
    batch)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B, H, N, d] tensor")
    B, H, N, d = q.shape
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dO, "dO")):
        _need(t, n, q.dtype, dev, q.shape)
    _need(eta, "eta", torch.float32, dev, (B, H, N))
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    if not isinstance(W0, torch.Tensor) or W0.dim() not in (2, 3):
        raise ValueError("W0 must be [H, 3*d*m] or [B, H, 3*d*m]")
    per_batch = W0.dim() == 3
    if m_h is None:
        m_h = W0.shape[-1] // (3 * d)
    _need(W0, "W0", torch.float32, dev, ((B, H) if per_batch else (H,)) + (3 * d * m_h,))
    if dW_out is not None:
        _need(dW_out, "dW_out", torch.float32, dev, (B, H, 3 * d * m_h))
    _flags(update_chunks, N, chunk, mask_mode == C.MASK_STRIDED)
    D, keep = ttt_desc(B, H, N, d, m_h, chunk, _DT[q.dtype], mask_mode, update_rule, ns_iters, momentum,
                       bool(last_layer_only), per_batch, update_chunks, inner_steps, ascent)
    if record is not None:
        rbytes, _ = ttt_record_bytes(D)
        _need_bytes(record, "record", rbytes, dev)
        n = ctypes.c_size_t(0)
        C.check(C.lib().ttt_backward_record_workspace_bytes(ctypes.byref(D), ctypes.byref(n)))
        nbytes = n.value
    else:
        nbytes = ttt_backward_workspace_bytes(D)
    workspace = _workspace(workspace, nbytes, dev)
    dq, dkt, dvt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    deta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dW0 = torch.empty_like(W0) if want_dW0 else None
    wsn = ctypes.c_size_t(0 if workspace is None else workspace.numel())
    if record is not None:
        st = C.lib().ttt_backward_record(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(record),
                                         ctypes.c_size_t(record.numel()), _ptr(dO), _ptr(dW_out), _ptr(dq), _ptr(dkt),
                                         _ptr(dvt), _ptr(deta), _ptr(dW0), _ptr(workspace), wsn, _stream_handle(stream))
    else:
        st = C.lib().ttt_backward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(W0), _ptr(dO),
                                  _ptr(dW_out), _ptr(dq), _ptr(dkt), _ptr(dvt), _ptr(deta), _ptr(dW0), _ptr(workspace),
                                  wsn, _stream_handle(stream))
    del keep
    C.check(st)
    return dq, dkt, dvt, deta, dW0


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
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D [B, H, N, d] tensor")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    _need(q, "q", None, dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, N, dv))
    _need(eta, "eta", torch.float32, dev, (B, H, N))
    if S0 is not None:
        _need(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if out is not None:
        _need(out, "out", q.dtype, dev, (B, H, N, dv))
    if mask_mode != C.MASK_TOKEN_CAUSAL and chunk < 1:
        raise ValueError("chunk must be >= 1")
    _flags(update_chunks, N, max(chunk, 1), mask_mode == C.MASK_STRIDED)
    D, keep = linattn_desc(B, H, N, dk, dv, chunk, _DT[q.dtype], mask_mode, update_chunks)
    nbytes = linattn_workspace_bytes(D)
    workspace = _workspace(workspace, nbytes, dev)
    o = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev) if out is None else out
    S_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_S else None
    st = C.lib().linattn_forward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(S0), _ptr(o),
                                 _ptr(S_out), _ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                                 _stream_handle(stream))
    del keep
    C.check(st)
    return o, S_out


def linattn_backward_workspace_bytes(desc: C.LinattnDesc) -> int:
    n = ctypes.c_size_t(0)
    C.check(C.lib().linattn_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def linattn_backward(q, k, v, eta, dO, chunk: int, mask_mode: int = C.MASK_APPLY_THEN_UPDATE, *,
                     S0: Optional[torch.Tensor] = None, dS_out: Optional[torch.Tensor] = None, update_chunks=None,
                     want_dS0: bool = True, workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of linattn_forward under a chunked mask through linattn_backward of libttt.so, for the
    output gradient dO [B, H, N, d_v] and the final-state gradient dS_out ([B, H, d_v, d_k] fp32 or
    None).  Returns (dq, dk, dv, deta, dS0 or None)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dO, "dO")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D [B, H, N, d] tensor")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    _need(q, "q", None, dev)
    _need(k, "k", q.dtype, dev, q.shape)
    _need(v, "v", q.dtype, dev, (B, H, N, dv))
    _need(dO, "dO", q.dtype, dev, (B, H, N, dv))
    _need(eta, "eta", torch.float32, dev, (B, H, N))
    if S0 is not None:
        _need(S0, "S0", torch.float32, dev, (B, H, dv, dk))
    if dS_out is not None:
        _need(dS_out, "dS_out", torch.float32, dev, (B, H, dv, dk))
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    _flags(update_chunks, N, chunk, mask_mode == C.MASK_STRIDED)
    D, keep = linattn_desc(B, H, N, dk, dv, chunk, _DT[q.dtype], mask_mode, update_chunks)
    nbytes = linattn_backward_workspace_bytes(D)
    workspace = _workspace(workspace, nbytes, dev)
    dq = torch.empty_like(q)
    dkt = torch.empty_like(k)
    dvt = torch.empty_like(v)
    deta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dS0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None
    st = C.lib().linattn_backward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(eta), _ptr(S0), _ptr(dO),
                                  _ptr(dS_out), _ptr(dq), _ptr(dkt), _ptr(dvt), _ptr(deta), _ptr(dS0), _ptr(workspace),
                                  ctypes.c_size_t(0 if workspace is None else workspace.numel()),
                                  _stream_handle(stream))
    del keep
    C.check(st)
    return dq, dkt, dvt, deta, dS0


def swa_workspace_bytes(desc: C.SwaDesc) -> int:
    n = ctypes.c_size_t(0)
    C.check(C.lib().swa_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def swa_forward(q, k, v, window: int, *, q_scale: Optional[torch.Tensor] = None, q_shift: Optional[torch.Tensor] = None,
                k_scale: Optional[torch.Tensor] = None, k_shift: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """LaCT's causal sliding-window attention through swa_forward of libttt.so: q, k, v [B, H, N, d]
    (bf16 or fp32); the per-head, per-channel scale / shift parameters are [H, d] fp32 or None.
    Returns o [B, H, N, d]."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B, H, N, d] tensor")
    B, H, N, d = q.shape
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"unsupported io dtype {q.dtype}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev, q.shape)
    for t, n in ((q_scale, "q_scale"), (q_shift, "q_shift"), (k_scale, "k_scale"), (k_shift, "k_shift")):
        if t is not None:
            _need(t, n, torch.float32, dev, (H, d))
    if out is not None:
        _need(out, "out", q.dtype, dev, q.shape)
    if window < 1:
        raise ValueError("window must be >= 1")
    D = C.SwaDesc(B, H, N, d, int(window), _DT[q.dtype])
    workspace = _workspace(workspace, swa_workspace_bytes(D), dev)
    o = torch.empty_like(q) if out is None else out
    st = C.lib().swa_forward(ctypes.byref(D), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(q_shift), _ptr(k_scale),
                             _ptr(k_shift), _ptr(o), _ptr(workspace),
                             ctypes.c_size_t(0 if workspace is None else workspace.numel()), _stream_handle(stream))
    C.check(st)
    return o
