"""CPU checks of the C ABI: libttt.so loads, exports what include/ttt.h declares, and rejects bad
arguments before touching any device (only argument-validation paths are exercised here)."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_chunk_amd import _lib as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

# fake device addresses: never dereferenced, because every call below fails validation first
P16 = 0x7F0000000000
P16B = 0x7F0100000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_\w+|linattn_\w+|swa_\w+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(C.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    L = C.lib()
    for name in C.EXPORTS:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in C.EXPORTS:
        assert name in syms, name


def test_version_and_status_strings():
    L = C.lib()
    assert L.ttt_abi_version() == 7
    for s in range(5):
        assert L.ttt_status_string(s)
    assert L.ttt_status_string(99) == b"unknown status"


def test_profiler_selection_on_the_host():
    """Selecting kernel classes and reading with nothing recorded touch no device."""
    L = C.lib()
    names = [L.ttt_profile_kernel_name(i).decode() for i in range(C.PROF_KERNELS)]
    assert names[0] == "k_up" and len(set(names)) == C.PROF_KERNELS
    C.profile_select(["k_up", "k_ns_step"])
    C.profile_select(None)
    assert L.ttt_profile_select(0) == C.TTT_OK
    assert L.ttt_profile_select(0xFFFFFFFF) == C.TTT_OK
    assert all(v == (0.0, 0) for v in C.profile_read().values())
    with pytest.raises(KeyError):
        C.profile_select(["no_such_kernel"])


def test_mfma_probe_rejects_before_enqueueing():
    L = C.lib()
    assert L.ttt_probe_mfma_bf16(0, 16, P16, None) == C.TTT_ERR_INVALID_ARGUMENT
    assert L.ttt_probe_mfma_bf16(4, 0, P16, None) == C.TTT_ERR_INVALID_ARGUMENT
    assert L.ttt_probe_mfma_bf16(4, 16, None, None) == C.TTT_ERR_INVALID_ARGUMENT


def desc(**kw):
    base = dict(B=2, H=4, N=256, d_h=64, m_h=128, chunk=64, io_dtype=C.TTT_BF16, mask=C.MASK_APPLY_THEN_UPDATE,
                rule=C.UPD_GD_L2, ns_iters=5, momentum=0.0, last_layer_only=0, w0_per_batch=0, update_chunks=None)
    base.update(kw)
    return C.TttDesc(**base)


def ws_bytes(D):
    n = ctypes.c_size_t(0)
    st = C.lib().ttt_workspace_bytes(ctypes.byref(D), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(d_h=48), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(d_h=4096), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(m_h=0), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(chunk=0), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(N=-1), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(io_dtype=7), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=9), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=C.MASK_TOKEN_CAUSAL), C.TTT_ERR_UNSUPPORTED),
    (dict(mask=C.MASK_FULL, chunk=64), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=C.MASK_STRIDED), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(rule=4), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(ns_iters=-1), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(inner_steps=65), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(inner_steps=-1), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(ascent=2), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(momentum=float("nan")), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(last_layer_only=2), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(parallel_form=2), C.TTT_ERR_INVALID_ARGUMENT),
    # the parallel form needs frozen W1, W3 and plain GD
    (dict(parallel_form=1, rule=C.UPD_GD), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(parallel_form=1, last_layer_only=1), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(parallel_form=1, last_layer_only=1, rule=C.UPD_MUON_L2), C.TTT_ERR_INVALID_ARGUMENT),
    # Variant 2 with Muon has a parallel form, with one gradient step per chunk
    (dict(parallel_form=1, last_layer_only=1, rule=C.UPD_MUON, inner_steps=2), C.TTT_ERR_UNSUPPORTED),
    # per-chunk rates: the momentum comes from chunk_momentum, not from momentum; no parallel form
    (dict(chunk_rates=2), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(chunk_rates=1, momentum=0.9), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(chunk_momentum=P16), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(chunk_rates=1, parallel_form=1, last_layer_only=1, rule=C.UPD_GD), C.TTT_ERR_UNSUPPORTED),
    (dict(parallel_form=1, last_layer_only=1, rule=C.UPD_GD, mask=C.MASK_STRIDED, N=1025 * 64,
          update_chunks=ctypes.cast((ctypes.c_uint8 * 1025)(), ctypes.c_void_p)), C.TTT_ERR_UNSUPPORTED),
])
def test_desc_validation(kw, status):
    st, _ = ws_bytes(desc(**kw))
    assert st == status
    assert C.lib().ttt_last_error()


def test_workspace_sizes():
    st, gd = ws_bytes(desc())
    assert st == C.TTT_OK and gd > 0
    _, muon = ws_bytes(desc(rule=C.UPD_MUON_L2))
    _, mom = ws_bytes(desc(rule=C.UPD_MUON_L2, momentum=0.9))
    assert muon > gd and mom > muon
    _, big = ws_bytes(desc(chunk=256))
    assert big > gd
    st, z = ws_bytes(desc(N=0))
    assert st == C.TTT_OK
    assert C.lib().ttt_last_error() == b""
    # a FULL mask needs one chunk covering the sequence
    assert ws_bytes(desc(mask=C.MASK_FULL, chunk=256))[0] == C.TTT_OK
    # the parallel form holds phi(q), phi(k) ([B H N m] each) and the per-chunk linear-attention
    # states (dS in fp32 and S_c in bf16, 6 bytes per element of the d x m state per chunk)
    st, par = ws_bytes(desc(parallel_form=1, last_layer_only=1, rule=C.UPD_GD))
    assert st == C.TTT_OK
    assert par >= 2 * 2 * 4 * 256 * 128 * 2 + 8 * 4 * 64 * 128 * 6
    st, par0 = ws_bytes(desc(parallel_form=1, last_layer_only=1, rule=C.UPD_GD, N=0))
    assert st == C.TTT_OK and par0 < par
    # with Muon it also holds every (scan, chunk) matrix's Newton-Schulz buffers: at least the fp32
    # result and two bf16 iterate planes of d x m per chunk and scan
    st, pm = ws_bytes(desc(parallel_form=1, last_layer_only=1, rule=C.UPD_MUON, momentum=0.9))
    assert st == C.TTT_OK and pm >= par + 8 * 4 * (64 * 128) * (4 + 2 + 2)


def call_forward(D, q=P16, k=P16, v=P16, eta=P16, W0=P16B, o=P16 + (1 << 30), W_out=None, M=None, ws=None, nws=0):
    return C.lib().ttt_forward(ctypes.byref(D), q, k, v, eta, W0, o, W_out, M, ws, nws, None)


def test_forward_rejects_before_enqueueing():
    D = desc()
    _, need = ws_bytes(D)
    assert call_forward(D, q=None) == C.TTT_ERR_INVALID_ARGUMENT
    assert call_forward(D, W0=None) == C.TTT_ERR_INVALID_ARGUMENT
    assert call_forward(D, q=P16 + 2) == C.TTT_ERR_INVALID_ARGUMENT          # misaligned
    assert call_forward(D, o=P16 + 64) == C.TTT_ERR_INVALID_ARGUMENT         # o overlaps q
    assert call_forward(D, ws=None, nws=0) == C.TTT_ERR_WORKSPACE
    assert call_forward(D, ws=P16 + (1 << 34), nws=need - 1) == C.TTT_ERR_WORKSPACE
    assert call_forward(D, ws=P16 + (1 << 34) + 16, nws=need) == C.TTT_ERR_WORKSPACE  # not 256-aligned
    assert call_forward(D, W_out=P16B + 64) == C.TTT_ERR_INVALID_ARGUMENT    # W_out overlaps W0
    assert b"workspace" in C.lib().ttt_last_error() or b"overlaps" in C.lib().ttt_last_error()
    # no (batch, head): nothing to do, no pointer is touched
    assert call_forward(desc(B=0), q=None, k=None, v=None, eta=None, o=None) == C.TTT_OK


def lin_desc(**kw):
    base = dict(B=1, H=2, N=128, d_k=64, d_v=64, chunk=32, io_dtype=C.TTT_BF16, mask=C.MASK_APPLY_THEN_UPDATE,
                update_chunks=None)
    base.update(kw)
    return C.LinattnDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d_k=48), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(d_k=512), C.TTT_ERR_UNSUPPORTED),        # chunks of 32 leave only the sequential kernel
    (dict(d_k=2080), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(d_v=16), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(chunk=0), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=5), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=C.MASK_FULL), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=C.MASK_STRIDED), C.TTT_ERR_INVALID_ARGUMENT),
])
def test_linattn_validation(kw, status):
    n = ctypes.c_size_t(1)
    assert C.lib().linattn_workspace_bytes(ctypes.byref(lin_desc(**kw)), ctypes.byref(n)) == status


def test_linattn_forward_rejects():
    L = C.lib()
    D = lin_desc()
    assert L.linattn_forward(ctypes.byref(D), None, P16, P16, P16, None, P16B, None, None, 0, None) == \
        C.TTT_ERR_INVALID_ARGUMENT
    assert L.linattn_forward(ctypes.byref(D), P16, P16, P16, P16, None, P16 + 32, None, None, 0, None) == \
        C.TTT_ERR_INVALID_ARGUMENT
    n = ctypes.c_size_t(1)
    assert L.linattn_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK and n.value == 0


def test_linattn_workspace_choice_and_rejects():
    """Large chunks take the chunk-parallel path, which needs 6 bytes per state element per chunk and
    scan in bf16; token-causal mode and small chunks need none.  A short or misaligned workspace is refused
    before anything is enqueued."""
    L = C.lib()
    n = ctypes.c_size_t(1)
    D = lin_desc(B=2, H=3, N=1000, d_k=128, d_v=64, chunk=256)   # 4 chunks, 4*128*64 <= 2*256*192
    assert L.linattn_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK
    per = 2 * 3 * 4 * 128 * 64 * 4                               # fp32 updates; bf16 states take half
    assert n.value == (per + 255) // 256 * 256 + (per // 2 + 255) // 256 * 256
    need = n.value
    for kw in (dict(mask=C.MASK_TOKEN_CAUSAL, N=200), dict(chunk=32)):
        kw = dict(dict(B=2, H=3, N=1000, d_k=128, d_v=64), **kw)
        assert L.linattn_workspace_bytes(ctypes.byref(lin_desc(**kw)), ctypes.byref(n)) == C.TTT_OK and n.value == 0
    # token-causal mode from two 128-token blocks on: the same layout over ceil(N / 128) blocks
    D2 = lin_desc(B=2, H=3, N=1000, d_k=128, d_v=64, mask=C.MASK_TOKEN_CAUSAL)
    assert L.linattn_workspace_bytes(ctypes.byref(D2), ctypes.byref(n)) == C.TTT_OK
    per2 = 2 * 3 * 8 * 128 * 64 * 4
    assert n.value == (per2 + 255) // 256 * 256 + (per2 // 2 + 255) // 256 * 256
    args = (P16, P16 + (1 << 30), P16 + (2 << 30), P16 + (3 << 30), None, P16B, None)
    assert L.linattn_forward(ctypes.byref(D), *args, None, 0, None) == C.TTT_ERR_WORKSPACE
    assert L.linattn_forward(ctypes.byref(D), *args, P16 + (1 << 34), need - 1, None) == C.TTT_ERR_WORKSPACE
    assert L.linattn_forward(ctypes.byref(D), *args, P16 + (1 << 34) + 16, need, None) == C.TTT_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,status", [
    (dict(), C.TTT_OK), (dict(mask=C.MASK_UPDATE_THEN_APPLY, chunk=1), C.TTT_OK), (dict(mask=C.MASK_FULL, chunk=128), C.TTT_OK),
    (dict(mask=C.MASK_TOKEN_CAUSAL), C.TTT_ERR_UNSUPPORTED), (dict(d_k=48), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(d_v=8192), C.TTT_ERR_INVALID_ARGUMENT), (dict(chunk=0), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(mask=C.MASK_STRIDED), C.TTT_ERR_INVALID_ARGUMENT),
])
def test_linattn_backward_validation(kw, status):
    n = ctypes.c_size_t(1)
    assert C.lib().linattn_backward_workspace_bytes(ctypes.byref(lin_desc(**kw)), ctypes.byref(n)) == status


def test_linattn_backward_workspace_and_rejects():
    """Workspace: the chunk update, state and state gradient per chunk (8 bytes per state element in bf16),
    plus dη partials per 128 columns of d_k beyond the first; nothing when N is 0.  Missing,
    misaligned or overlapping buffers and a short workspace are refused before anything is enqueued."""
    L = C.lib()
    n = ctypes.c_size_t(0)
    D = lin_desc(B=2, H=3, N=1000, d_k=320, d_v=64, chunk=256)   # 4 chunks, 3 column tiles of d_k
    assert L.linattn_backward_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK
    al = lambda x: (x + 255) // 256 * 256
    assert n.value == al(2 * 3 * 4 * 320 * 64 * 4) + 2 * al(2 * 3 * 4 * 320 * 64 * 2) + al(3 * 2 * 3 * 1000 * 4)
    need = n.value
    assert L.linattn_backward_workspace_bytes(ctypes.byref(lin_desc(N=0)), ctypes.byref(n)) == C.TTT_OK and n.value == 0
    G = 1 << 30
    ins = [P16, P16 + G, P16 + 2 * G, P16 + 3 * G, None, P16 + 4 * G, None]   # q k v eta S0 dO dS_out
    OB = P16 + (1 << 34)
    outs = [OB, OB + G, OB + 2 * G, OB + 3 * G, None]                           # dq dk dv deta dS0
    ws = P16 + (1 << 36)

    def call(i=None, o=None, w=ws, nw=need):
        a = list(ins if i is None else i)
        b = list(outs if o is None else o)
        return L.linattn_backward(ctypes.byref(D), *a, *b, w, nw, None)

    assert call(i=[None] + ins[1:]) == C.TTT_ERR_INVALID_ARGUMENT                    # q missing
    assert call(o=outs[:3] + [None, None]) == C.TTT_ERR_INVALID_ARGUMENT             # deta missing
    assert call(i=[P16 + 2] + ins[1:]) == C.TTT_ERR_INVALID_ARGUMENT                 # misaligned q
    assert call(o=[P16 + 64] + outs[1:]) == C.TTT_ERR_INVALID_ARGUMENT               # dq overlaps q
    assert b"overlaps" in L.ttt_last_error()
    assert call(o=[OB, OB + 64] + outs[2:]) == C.TTT_ERR_INVALID_ARGUMENT            # dk overlaps dq
    assert call(w=None, nw=0) == C.TTT_ERR_WORKSPACE
    assert call(nw=need - 1) == C.TTT_ERR_WORKSPACE
    assert call(w=ws + 16) == C.TTT_ERR_INVALID_ARGUMENT                             # not 256-aligned
    # no (batch, head): nothing to do, no pointer is touched
    E = lin_desc(B=0)
    assert L.linattn_backward(ctypes.byref(E), *([None] * 13), 0, None) == C.TTT_OK


def test_linattn_wide_keys_need_the_chunk_parallel_path():
    """d_k above 256 is accepted where the chunk-parallel kernels run (they loop over d_k tiles) and
    refused with TTT_ERR_UNSUPPORTED where only the sequential kernel could run; d_k must stay a
    multiple of 32 up to 2048."""
    L = C.lib()
    n = ctypes.c_size_t(0)
    for kw in (dict(chunk=2048), dict(mask=C.MASK_TOKEN_CAUSAL)):
        D = lin_desc(**dict(dict(B=1, H=2, N=4096, d_k=384, d_v=384), **kw))
        assert L.linattn_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK and n.value > 0
    for kw in (dict(mask=C.MASK_TOKEN_CAUSAL, N=200), dict(chunk=64)):
        D = lin_desc(**dict(dict(B=1, H=2, N=4096, d_k=384, d_v=384), **kw))
        assert L.linattn_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_ERR_UNSUPPORTED
        assert b"chunk-parallel" in L.ttt_last_error()
    for dk in (2080, 400):
        D = lin_desc(B=1, H=2, N=4096, d_k=dk, d_v=384, chunk=2048)
        assert L.linattn_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_ERR_INVALID_ARGUMENT


def bwd_desc(**kw):
    return desc(**dict(dict(last_layer_only=1, rule=C.UPD_GD), **kw))


@pytest.mark.parametrize("kw,status", [
    (dict(), C.TTT_OK), (dict(mask=C.MASK_UPDATE_THEN_APPLY, inner_steps=3, ascent=1), C.TTT_OK),
    (dict(parallel_form=1, w0_per_batch=1), C.TTT_OK), (dict(N=0), C.TTT_OK),
    # the layer whose inner loop trains W2 alone by GD (momentum and the L2 norm allowed), and the
    # recurrence (all three weights learning, or W2 alone with Muon) under every rule and momentum,
    # up to 65536 recorded updates
    (dict(last_layer_only=0), C.TTT_OK), (dict(rule=C.UPD_GD_L2), C.TTT_OK),
    (dict(last_layer_only=0, rule=C.UPD_GD_L2, momentum=0.9, inner_steps=2, ascent=1), C.TTT_OK),
    (dict(last_layer_only=0, rule=C.UPD_MUON_L2), C.TTT_OK), (dict(last_layer_only=0, N=1 << 20, chunk=8), C.TTT_ERR_UNSUPPORTED),
    (dict(last_layer_only=0, chunk_rates=1), C.TTT_ERR_UNSUPPORTED),
    (dict(last_layer_only=0, parallel_form=1), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(rule=C.UPD_GD_L2, momentum=0.9, inner_steps=3), C.TTT_OK), (dict(rule=C.UPD_MUON_L2), C.TTT_OK),
    (dict(rule=C.UPD_MUON, momentum=0.9), C.TTT_OK), (dict(momentum=0.9), C.TTT_OK),
    (dict(chunk_rates=1), C.TTT_ERR_UNSUPPORTED), (dict(mask=C.MASK_TOKEN_CAUSAL), C.TTT_ERR_UNSUPPORTED),
    (dict(d_h=48), C.TTT_ERR_INVALID_ARGUMENT), (dict(mask=C.MASK_STRIDED), C.TTT_ERR_INVALID_ARGUMENT),
])
def test_ttt_backward_validation(kw, status):
    n = ctypes.c_size_t(0)
    assert C.lib().ttt_backward_workspace_bytes(ctypes.byref(bwd_desc(**kw)), ctypes.byref(n)) == status


def test_ttt_backward_workspace_and_rejects():
    """Workspace: W1 | W3 and their transposes in bf16, phi(q), phi(k), the factors of phi's backward
    (later dA | dC) of both sides, the scans' dW2 and the dW1 | dW3 partials, then the
    linear-attention backward's workspace over d_k = m, d_v = d.  Missing, misaligned or overlapping buffers and a short
    workspace are refused before anything is enqueued."""
    L = C.lib()
    n = ctypes.c_size_t(0)
    B, H, N, d, m, chunk = 2, 4, 256, 64, 128, 64
    D = bwd_desc()
    assert L.ttt_backward_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK
    al = lambda x: (x + 255) // 256 * 256
    S, dm, nc = B * H, d * m, N // chunk
    # one token part: 4 weight tiles, and two parts of 2 * 2 * 256 / 2 positions would be under 1024
    expect = 2 * al(H * 2 * dm * 2) + 2 * al(S * N * m * 2) + 2 * al(S * N * 2 * m * 2) + al(S * dm * 4) \
        + al(1 * H * 2 * dm * 4) + al(S * nc * dm * 4) + 2 * al(S * nc * dm * 2)
    assert n.value == expect
    need = n.value
    # no tokens: only the scans' dW2
    assert L.ttt_backward_workspace_bytes(ctypes.byref(bwd_desc(N=0)), ctypes.byref(n)) == C.TTT_OK
    assert n.value == al(S * dm * 4)
    G = 1 << 30
    ins = [P16, P16 + G, P16 + 2 * G, P16 + 3 * G, P16 + 4 * G, P16 + 5 * G, None]  # q k v eta W0 dO dW_out
    OB = P16 + (1 << 34)
    outs = [OB, OB + G, OB + 2 * G, OB + 3 * G, OB + 4 * G]                     # dq dk dv deta dW0
    ws = P16 + (1 << 36)

    def call(i=None, o=None, w=ws, nw=need):
        a = list(ins if i is None else i)
        b = list(outs if o is None else o)
        return L.ttt_backward(ctypes.byref(D), *a, *b, w, nw, None)

    assert call(i=[None] + ins[1:]) == C.TTT_ERR_INVALID_ARGUMENT                   # q missing
    assert call(i=ins[:4] + [None] + ins[5:]) == C.TTT_ERR_INVALID_ARGUMENT         # W0 missing
    assert call(o=outs[:3] + [None, outs[4]]) == C.TTT_ERR_INVALID_ARGUMENT         # deta missing
    assert call(i=ins[:5] + [P16 + 5 * G + 8, None]) == C.TTT_ERR_INVALID_ARGUMENT  # misaligned dO
    assert call(o=outs[:4] + [OB + 4 * G + 4]) == C.TTT_ERR_INVALID_ARGUMENT        # misaligned dW0
    assert call(o=[P16 + 64] + outs[1:]) == C.TTT_ERR_INVALID_ARGUMENT              # dq overlaps q
    assert b"overlaps" in L.ttt_last_error()
    assert call(o=outs[:4] + [P16 + 4 * G + 16]) == C.TTT_ERR_INVALID_ARGUMENT      # dW0 overlaps W0
    assert call(o=[OB, OB + 64] + outs[2:]) == C.TTT_ERR_INVALID_ARGUMENT           # dk overlaps dq
    assert call(w=None, nw=0) == C.TTT_ERR_WORKSPACE
    assert call(nw=need - 1) == C.TTT_ERR_WORKSPACE
    assert call(w=ws + 16) == C.TTT_ERR_INVALID_ARGUMENT                            # not 256-aligned
    # no (batch, head): nothing to do, no pointer is touched
    assert L.ttt_backward(ctypes.byref(bwd_desc(B=0)), *([None] * 13), 0, None) == C.TTT_OK


def test_full_backward_workspace():
    """All three weights learning: the forward's workspace (no Muon), the weights before every update
    and after the last (fp32), the row norms of every update (GD + L2), the running weight gradient,
    Gamma, the six [m][d] operand blocks, the key chunk's planes (4m + 2m + m), the deta partials,
    the query range's planes (2m + m) and the weight-gradient parts; momentum adds its gradient,
    several inner steps the fp32 dk, dv accumulators, fp32 operands a scratch of 3 x 128 x 128
    floats per key tile."""
    L = C.lib()
    n = ctypes.c_size_t(0)
    al = lambda x: (x + 255) // 256 * 256
    B, H, N, d, m, chunk = 2, 4, 256, 64, 128, 64
    S, dm = B * H, d * m
    for rule, mom, steps, mask, flags in ((C.UPD_GD, 0.0, 1, C.MASK_APPLY_THEN_UPDATE, None),
                                          (C.UPD_GD_L2, 0.9, 2, C.MASK_STRIDED, [0, 0, 1, 1])):
        arr = None if flags is None else (ctypes.c_uint8 * 4)(*flags)
        keep = None if arr is None else ctypes.cast(arr, ctypes.c_void_p)
        D = desc(rule=rule, momentum=mom, inner_steps=steps, mask=mask, update_chunks=keep)
        st, fwd = ws_bytes(desc(rule=rule, momentum=mom, inner_steps=steps, mask=mask, update_chunks=keep))
        assert st == C.TTT_OK
        assert L.ttt_backward_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK
        T = steps * (4 if flags is None else sum(flags))
        qcap = chunk if flags is None else 3 * chunk  # strided: chunks 0-2 read the first weights
        expect = al(fwd) + al((T + 1) * S * 3 * dm * 4) + (al(T * S * (2 * m + d) * 4) if rule == C.UPD_GD_L2 else 0)
        expect += al(S * 3 * dm * 4) + (al(S * 3 * dm * 4) if mom else 0) + al(S * 3 * dm * 4) + al(S * 6 * dm * 2)
        expect += al(S * chunk * 4 * m * 2) + al(S * chunk * 2 * m * 2)  # (bf16: no first-pass scratch)
        expect += al(S * chunk * m * 2)
        if steps > 1:
            expect += 2 * al(S * chunk * d * 4)
        expect += al(1 * S * chunk * 4) + al(S * qcap * 2 * m * 2) + al(S * qcap * m * 2)
        expect += al(1 * S * 3 * dm * 4)  # one part: 16 tiles, and parts under 1024 positions are not taken
        assert n.value == expect, (rule, mom, steps)


def test_training_record_sizes_and_rejects():
    """The record: the weights before every update and after the last (fp32), the row norms of every
    update (L2 rules), every update's Newton-Schulz input (Muon); ttt_forward_record's workspace is
    the forward's (no parallel form); the backward from a record needs the backward's workspace
    without the record and the forward's.  Descriptors outside the recurrence's backward, NULL,
    short or misaligned records and overlaps are refused before anything is enqueued."""
    L = C.lib()
    al = lambda x: (x + 255) // 256 * 256
    B, H, N, d, m, chunk = 2, 4, 256, 64, 128, 64
    S, dm, T = B * H, d * m, 4
    r, w, n, full = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    for rule, extra in ((C.UPD_GD, 0), (C.UPD_GD_L2, al(T * S * (2 * m + d) * 4)),
                        (C.UPD_MUON_L2, al(T * S * (2 * m + d) * 4) + al(T * S * 3 * dm * 4))):
        D = desc(rule=rule, momentum=0.9)
        assert L.ttt_record_bytes(ctypes.byref(D), ctypes.byref(r), ctypes.byref(w)) == C.TTT_OK
        assert r.value == al((T + 1) * S * 3 * dm * 4) + extra
        assert w.value == ws_bytes(D)[1]
        assert L.ttt_backward_record_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK
        assert L.ttt_backward_workspace_bytes(ctypes.byref(D), ctypes.byref(full)) == C.TTT_OK
        assert n.value == full.value - al(w.value) - al(r.value)
    # W2 alone by GD walks the recurrence back too (the pair's route); per-chunk rates have no backward
    assert L.ttt_record_bytes(ctypes.byref(desc(last_layer_only=1, rule=C.UPD_GD)), ctypes.byref(r),
                              ctypes.byref(w)) == C.TTT_OK
    assert L.ttt_record_bytes(ctypes.byref(desc(chunk_rates=1)), ctypes.byref(r), ctypes.byref(w)) == \
        C.TTT_ERR_UNSUPPORTED
    assert L.ttt_record_bytes(ctypes.byref(desc()), None, ctypes.byref(w)) == C.TTT_ERR_INVALID_ARGUMENT
    D = desc()
    assert L.ttt_record_bytes(ctypes.byref(D), ctypes.byref(r), ctypes.byref(w)) == C.TTT_OK
    G = 1 << 30
    q, k, v, eta, W0, o, Wo = (P16 + i * G for i in range(7))
    rec, ws = P16 + (1 << 36), P16 + (1 << 37)

    def fwd(rp=rec, rn=r.value, oo=o):
        return L.ttt_forward_record(ctypes.byref(D), q, k, v, eta, W0, oo, Wo, rp, rn, ws, w.value, None)

    assert fwd(rp=None) == C.TTT_ERR_INVALID_ARGUMENT
    assert fwd(rp=rec + 16) == C.TTT_ERR_INVALID_ARGUMENT                 # not 256-aligned
    assert fwd(rn=r.value - 1) == C.TTT_ERR_WORKSPACE
    assert fwd(rp=o) == C.TTT_ERR_INVALID_ARGUMENT                        # the record over o
    assert b"overlaps" in L.ttt_last_error()
    assert fwd(oo=q + 64) == C.TTT_ERR_INVALID_ARGUMENT                   # o over q
    assert L.ttt_backward_record_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == C.TTT_OK
    OB = P16 + (1 << 38)
    dq, dk, dv, deta, dW0 = (OB + i * G for i in range(5))
    dO = P16 + 8 * G

    def bwd(rp=rec, rn=r.value, dqq=dq):
        return L.ttt_backward_record(ctypes.byref(D), q, k, v, eta, rp, rn, dO, None, dqq, dk, dv, deta, dW0, ws,
                                     n.value, None)

    assert bwd(rp=None) == C.TTT_ERR_INVALID_ARGUMENT
    assert bwd(rn=r.value - 1) == C.TTT_ERR_WORKSPACE
    assert bwd(rp=rec + 16) == C.TTT_ERR_INVALID_ARGUMENT
    assert bwd(dqq=rec + 64) == C.TTT_ERR_INVALID_ARGUMENT                # dq over the record
    assert L.ttt_forward_record(ctypes.byref(desc(B=0)), *([None] * 8), 0, None, 0, None) == C.TTT_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(C, "_lib", None)
    monkeypatch.setattr(C, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        C.lib()


def _gpu_count():
    try:
        import torch
        return torch.cuda.device_count()   # counts devices without initialising HIP
    except Exception:
        return 0


@pytest.mark.skipif(_gpu_count() > 0, reason="checks the answer of a machine without a GPU")
def test_valid_calls_without_a_device_report_device_error():
    """On a machine with no usable HIP device, calls whose arguments pass validation stop at the
    device-buffer check with TTT_ERR_DEVICE and a message; nothing is launched."""
    L = C.lib()
    D = desc()
    _, need = ws_bytes(D)
    assert call_forward(D, ws=P16 + (1 << 34), nws=need) == C.TTT_ERR_DEVICE
    assert b"no usable HIP device" in L.ttt_last_error()
    Dl = lin_desc()
    assert L.linattn_forward(ctypes.byref(Dl), P16, P16 + (1 << 30), P16 + (2 << 30), P16 + (3 << 30), None, P16B,
                             None, None, 0, None) == C.TTT_ERR_DEVICE
    n = ctypes.c_size_t(0)
    L.linattn_backward_workspace_bytes(ctypes.byref(Dl), ctypes.byref(n))
    G = 1 << 30
    OB = P16 + (1 << 34)
    assert L.linattn_backward(ctypes.byref(Dl), P16, P16 + G, P16 + 2 * G, P16 + 3 * G, None, P16 + 4 * G, None,
                              OB, OB + G, OB + 2 * G, OB + 3 * G, None, P16 + (1 << 36), n.value,
                              None) == C.TTT_ERR_DEVICE
    Db = bwd_desc()
    L.ttt_backward_workspace_bytes(ctypes.byref(Db), ctypes.byref(n))
    assert L.ttt_backward(ctypes.byref(Db), P16, P16 + G, P16 + 2 * G, P16 + 3 * G, P16 + 4 * G, P16 + 5 * G, None,
                          OB, OB + G, OB + 2 * G, OB + 3 * G, OB + 4 * G, P16 + (1 << 36), n.value,
                          None) == C.TTT_ERR_DEVICE
    # the status table answers for any non-negative value
    assert L.ttt_status_string(C.TTT_ERR_DEVICE) == b"HIP device or launch error"
    assert L.ttt_status_string(0x7FFFFFFF) == b"unknown status"



def swa_desc(**kw):
    base = dict(B=2, H=4, N=1000, d=384, window=256, io_dtype=C.TTT_BF16)
    base.update(kw)
    return C.SwaDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d=48), C.TTT_ERR_INVALID_ARGUMENT), (dict(d=416), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(window=0), C.TTT_ERR_INVALID_ARGUMENT), (dict(N=-1), C.TTT_ERR_INVALID_ARGUMENT),
    (dict(io_dtype=3), C.TTT_ERR_INVALID_ARGUMENT), (dict(), C.TTT_OK), (dict(d=32, window=1), C.TTT_OK),
])
def test_swa_validation_and_workspace(kw, status):
    L = C.lib()
    n = ctypes.c_size_t(0)
    D = swa_desc(**kw)
    assert L.swa_workspace_bytes(ctypes.byref(D), ctypes.byref(n)) == status
    if status == C.TTT_OK:
        # bf16 heads with d a multiple of 64 (not 320): the v blocks of 32 keys that the query-resident
        # walk reads; otherwise the transformed queries in the io dtype
        es = 2 if D.io_dtype == C.TTT_BF16 else 4
        if D.io_dtype == C.TTT_BF16 and D.d % 64 == 0 and D.d != 320:
            assert n.value == D.B * D.H * -(-D.N // 32) * 32 * D.d * 2
        else:
            assert n.value == D.B * D.H * D.N * D.d * es


def test_swa_forward_rejects_before_enqueueing():
    L = C.lib()
    D = swa_desc()
    n = ctypes.c_size_t(0)
    L.swa_workspace_bytes(ctypes.byref(D), ctypes.byref(n))
    args = (P16, P16 + (1 << 30), P16 + (2 << 30))
    assert L.swa_forward(ctypes.byref(D), None, *args[1:], None, None, None, None, P16B, P16 + (1 << 34), n.value,
                         None) == C.TTT_ERR_INVALID_ARGUMENT
    assert L.swa_forward(ctypes.byref(D), *args, None, None, None, None, P16B, None, 0, None) == C.TTT_ERR_WORKSPACE
    assert L.swa_forward(ctypes.byref(D), *args, None, None, None, None, P16B, P16 + (1 << 34), n.value - 1,
                         None) == C.TTT_ERR_WORKSPACE
    assert L.swa_forward(ctypes.byref(D), *args, None, None, None, None, P16 + 64, P16 + (1 << 34), n.value,
                         None) == C.TTT_ERR_INVALID_ARGUMENT   # o overlaps q
    assert L.swa_forward(ctypes.byref(D), *args, P16 + 4, None, None, None, P16B, P16 + (1 << 34), n.value,
                         None) == C.TTT_ERR_INVALID_ARGUMENT   # misaligned scale vector
    # nothing to do: no pointer is touched
    assert L.swa_forward(ctypes.byref(swa_desc(N=0)), None, None, None, None, None, None, None, None, None, 0,
                         None) == C.TTT_OK
