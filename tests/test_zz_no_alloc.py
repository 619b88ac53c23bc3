"""ttt_forward_noalloc (through the C ABI) against ttt_forward with a caller-given workspace.

Both run the same kernels on the same inputs, and nothing a call reads from its workspace comes
from an earlier call, so the outputs must agree bit for bit: two calls in a row on the library's
shared scratch, the second with a smaller input and another update rule, then a call too large for
the scratch, which is refused before anything runs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O
import linear_attention_chunk_amd as T
from linear_attention_chunk_amd import _lib as C
from gpu_util import full_ttt_inputs, say

pytestmark = pytest.mark.gpu


def _pair(seed, B, H, N, d, m, chunk, mask, rule, bf16, momentum=0.0, want_W=True, **kw):
    say(f"noalloc case B{B} H{H} N{N} d{d} m{m} b{chunk} mask{mask} rule{rule} mom{momentum} bf16={bf16}")
    (q, k, v, eta, W0), _ = full_ttt_inputs(seed, B, H, N, d, m, bf16)
    M_ref = M_na = None
    if momentum:
        M0 = 0.01 * torch.randn((B, H, 3 * d * m), device="cuda")
        M_ref, M_na = M0.clone(), M0.clone()
    o_ref, W_ref = T.ttt_forward(q, k, v, eta, W0, chunk, mask, rule, m_h=m, momentum=momentum, M=M_ref,
                                 want_W=want_W, **kw)
    o = torch.full_like(q, 7.0)
    W_out = torch.full((B, H, 3 * d * m), 7.0, device="cuda") if want_W else None
    o_na, W_na = T.ttt_forward_noalloc(q, k, v, eta, W0, chunk, mask, rule, m_h=m, momentum=momentum, M=M_na,
                                       out=o, W_out=W_out, **kw)
    torch.cuda.synchronize()
    assert o_na is o and W_na is W_out
    assert torch.equal(o_na, o_ref)
    if want_W:
        assert torch.equal(W_na, W_ref)
    if momentum:
        assert torch.equal(M_na, M_ref)
    return o_ref


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    D, keep = T.ttt_desc(1, 2, 1100, 128, 384, 256, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    assert T.ttt_workspace_bytes(D) <= C.NOALLOC_SCRATCH_BYTES
    # the larger call first, so that the second runs on scratch the first has filled
    _pair(50, 1, 2, 1100, 128, 384, 256, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2, True)
    _pair(51, 1, 1, 300, 64, 160, 96, O.MASK_UPDATE_THEN_APPLY, O.UPD_MUON_L2, True, momentum=0.9)
    # fp32, outputs only; and the parallel form, whose workspace holds other things
    _pair(52, 2, 1, 256, 32, 96, 64, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, False, want_W=False)
    _pair(53, 1, 2, 308, 64, 160, 96, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD, True, momentum=0.9,
          last_layer_only=True, parallel_form=True)


def test_noalloc_refuses_calls_beyond_its_scratch():
    B, H, N, d, m, chunk = 2, 4, 4096, 384, 768, 2048
    D, keep = T.ttt_desc(B, H, N, d, m, chunk, C.TTT_BF16, O.MASK_APPLY_THEN_UPDATE, O.UPD_GD_L2)
    need = T.ttt_workspace_bytes(D)
    assert need > C.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    eta = torch.zeros((B, H, N), device="cuda")
    W0 = torch.zeros((H, 3 * d * m), device="cuda")
    o = torch.full_like(q, 3.0)
    with pytest.raises(C.TttError) as e:
        T.ttt_forward_noalloc(q, q, q, eta, W0, chunk, m_h=m, out=o)
    assert e.value.status == C.TTT_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())   # refused before anything was enqueued
