"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point enqueues only kernels and device-to-device copies on the caller's stream, with no
allocation, memset or synchronisation, so a call can be captured once and replayed.  Each case runs
the call eagerly, captures it, then replays it three times with eager work between the replays
(outputs cleared, carried state reset) and checks every replay bit for bit against the eager
result.  The workspaces are allocated before the capture."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import linear_attention_chunk_amd as T
from linear_attention_chunk_amd import _lib as C
from linear_attention_chunk_amd import api as A
from gpu_util import full_ttt_inputs, say

pytestmark = pytest.mark.gpu


def replay_matches_eager(label, call, outs, reset=None, reps=3):
    say(f"graph case {label}")
    if reset:
        reset()
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    if reset:
        reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        call()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outs:
            o.fill_(float("nan"))
        if reset:
            reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"{label}: replay {r}, output {i} differs from the eager call"
    del g


def ttt_case(label, seed, N, d, m, chunk, mask, rule, bf16, momentum=0.0, last=False, parallel=False):
    (q, k, v, eta, W0), _ = full_ttt_inputs(seed, 1, 2, N, d, m, bf16)
    D, keep = T.ttt_desc(1, 2, N, d, m, chunk, C.TTT_BF16 if bf16 else C.TTT_F32, mask, rule, 5, momentum, last,
                         False, None, 1, False, parallel)
    ws = torch.empty(max(1, T.ttt_workspace_bytes(D)), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    W = torch.empty((1, 2, 3 * d * m), dtype=torch.float32, device="cuda")
    M = torch.zeros((1, 2, 3 * d * m), dtype=torch.float32, device="cuda") if momentum else None
    M0 = None if M is None else 0.01 * torch.randn_like(M)
    reset = (lambda: M.copy_(M0)) if M is not None else None

    # through the C ABI directly, so that W_out is a preallocated tensor
    def call_w():
        st = C.lib().ttt_forward(A.ctypes.byref(D), A._ptr(q), A._ptr(k), A._ptr(v),
                                 A._ptr(eta), A._ptr(W0), A._ptr(o), A._ptr(W), A._ptr(M),
                                 A._ptr(ws), A.ctypes.c_size_t(ws.numel()), A._stream_handle(None))
        C.check(st)

    replay_matches_eager(label, call_w, [o, W] + ([M] if M is not None else []), reset)
    del keep


@pytest.mark.parametrize("bf16", [False, True])
def test_layer_recurrence_replays(bf16):
    ttt_case("GD + L2", 1, 308, 64, 160, 96, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, bf16)
    ttt_case("Muon + L2, momentum", 2, 308, 64, 160, 96, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, bf16, momentum=0.9)


@pytest.mark.parametrize("bf16", [False, True])
def test_parallel_forms_replay(bf16):
    ttt_case("parallel form, GD", 3, 308, 64, 160, 96, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, bf16, last=True,
             parallel=True)
    ttt_case("parallel form, Muon", 4, 308, 64, 160, 96, O.MASK_APPLY_THEN_UPDATE, O.UPD_MUON, bf16, momentum=0.9,
             last=True, parallel=True)


def test_linear_attention_and_backwards_replay():
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    B, H, N, d = 2, 2, 700, 64
    q, k, v, dO = ((torch.randn((B, H, N, d), generator=g, device="cuda") / 8).to(torch.bfloat16) for _ in range(4))
    eta = 0.05 * torch.sigmoid(torch.randn((B, H, N), generator=g, device="cuda"))
    o = torch.empty_like(q)
    for mask, chunk in ((O.MASK_APPLY_THEN_UPDATE, 128), (O.MASK_TOKEN_CAUSAL, 1), (O.MASK_UPDATE_THEN_APPLY, 32)):
        D, _ = T.linattn_desc(B, H, N, d, d, chunk, C.TTT_BF16, mask)
        ws = torch.empty(max(1, T.linattn_workspace_bytes(D)), dtype=torch.uint8, device="cuda")
        replay_matches_eager(f"linattn_forward mask{mask} chunk{chunk}",
                             lambda: T.linattn_forward(q, k, v, eta, chunk, mask, out=o, want_S=False, workspace=ws),
                             [o])
    D, _ = T.linattn_desc(B, H, N, d, d, 128, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE)
    wsb = torch.empty(max(1, T.linattn_backward_workspace_bytes(D)), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q) for _ in range(3)] + [torch.empty_like(eta)]

    def lbwd():
        st = C.lib().linattn_backward(A.ctypes.byref(D), *[A._ptr(x) for x in (q, k, v, eta)], None,
                                      A._ptr(dO), None, *[A._ptr(x) for x in outs], None, A._ptr(wsb),
                                      A.ctypes.c_size_t(wsb.numel()), A._stream_handle(None))
        C.check(st)

    replay_matches_eager("linattn_backward", lbwd, outs)
    # the layer's backward (last layer only, plain GD)
    (qt, kt, vt, et, W0), _ = full_ttt_inputs(6, 1, 2, 308, 64, 160, True)
    dOt = torch.randn_like(qt.float()).to(torch.bfloat16)
    Dt, _ = T.ttt_desc(1, 2, 308, 64, 160, 96, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE, C.UPD_GD, 0, 0.0, True)
    wst = torch.empty(max(1, T.ttt_backward_workspace_bytes(Dt)), dtype=torch.uint8, device="cuda")
    touts = [torch.empty_like(qt) for _ in range(3)] + [torch.empty_like(et), torch.empty_like(W0)]

    def tbwd():
        st = C.lib().ttt_backward(A.ctypes.byref(Dt), *[A._ptr(x) for x in (qt, kt, vt, et, W0, dOt)], None,
                                  *[A._ptr(x) for x in touts], A._ptr(wst), A.ctypes.c_size_t(wst.numel()),
                                  A._stream_handle(None))
        C.check(st)

    replay_matches_eager("ttt_backward", tbwd, touts)
    # the backward with all three weights learning (GD + L2, momentum), dW_out given
    Df, _ = T.ttt_desc(1, 2, 308, 64, 160, 96, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE, C.UPD_GD_L2, 0, 0.9)
    wsf = torch.empty(max(1, T.ttt_backward_workspace_bytes(Df)), dtype=torch.uint8, device="cuda")
    dWo = 0.1 * torch.randn((1, 2, W0.shape[-1]), device="cuda")
    fouts = [torch.empty_like(qt) for _ in range(3)] + [torch.empty_like(et), torch.empty_like(W0)]

    def fbwd():
        st = C.lib().ttt_backward(A.ctypes.byref(Df), *[A._ptr(x) for x in (qt, kt, vt, et, W0, dOt, dWo)],
                                  *[A._ptr(x) for x in fouts], A._ptr(wsf), A.ctypes.c_size_t(wsf.numel()),
                                  A._stream_handle(None))
        C.check(st)

    replay_matches_eager("ttt_backward, all weights", fbwd, fouts)
    # and through Muon (Newton-Schulz walked back on every update)
    Df, _ = T.ttt_desc(1, 2, 308, 64, 160, 96, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE, C.UPD_MUON_L2, 5, 0.9)
    wsf = torch.empty(max(1, T.ttt_backward_workspace_bytes(Df)), dtype=torch.uint8, device="cuda")
    replay_matches_eager("ttt_backward, Muon", fbwd, fouts)
    # sliding-window attention
    Ds = C.SwaDesc(1, 2, 308, 64, 96, C.TTT_BF16)
    wss = torch.empty(max(1, T.swa_workspace_bytes(Ds)), dtype=torch.uint8, device="cuda")
    os_ = torch.empty_like(qt)
    replay_matches_eager("swa_forward", lambda: T.swa_forward(qt, kt, vt, 96, out=os_, workspace=wss), [os_])
