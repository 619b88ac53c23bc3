"""ctypes declarations of the C ABI in include/ttt.h (libttt.so, built in-tree for gfx950).

There is no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_size_t, c_void_p, POINTER

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttt.so")

# enums of include/ttt.h
TTT_OK, TTT_ERR_INVALID_ARGUMENT, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_ERR_DEVICE = range(5)
TTT_F32, TTT_BF16 = 0, 1
MASK_FULL, MASK_UPDATE_THEN_APPLY, MASK_APPLY_THEN_UPDATE, MASK_STRIDED, MASK_TOKEN_CAUSAL = range(5)
UPD_GD, UPD_GD_L2, UPD_MUON_L2, UPD_MUON = range(4)

# every function include/ttt.h declares
EXPORTS = (
    "ttt_abi_version", "ttt_status_string", "ttt_last_error",
    "ttt_workspace_bytes", "ttt_forward", "ttt_forward_noalloc", "ttt_backward_workspace_bytes", "ttt_backward",
    "ttt_record_bytes", "ttt_forward_record", "ttt_backward_record_workspace_bytes", "ttt_backward_record",
    "linattn_workspace_bytes", "linattn_forward", "linattn_backward_workspace_bytes", "linattn_backward",
    "swa_workspace_bytes", "swa_forward",
    "ttt_profile_enable", "ttt_profile_select", "ttt_profile_read", "ttt_profile_kernel_name",
    "ttt_probe_mfma_bf16",
)
PROF_KERNELS = 32
NOALLOC_SCRATCH_BYTES = 64 << 20   # TTT_NOALLOC_SCRATCH_BYTES of include/ttt.h


class TttDesc(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("H", c_int32), ("N", c_int32),
        ("d_h", c_int32), ("m_h", c_int32), ("chunk", c_int32),
        ("io_dtype", c_int32), ("mask", c_int32), ("rule", c_int32),
        ("ns_iters", c_int32), ("momentum", c_float), ("last_layer_only", c_int32),
        ("w0_per_batch", c_int32), ("update_chunks", c_void_p),
        ("inner_steps", c_int32), ("ascent", c_int32), ("parallel_form", c_int32),
        ("chunk_rates", c_int32), ("chunk_momentum", c_void_p),
    ]


class LinattnDesc(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("H", c_int32), ("N", c_int32),
        ("d_k", c_int32), ("d_v", c_int32), ("chunk", c_int32),
        ("io_dtype", c_int32), ("mask", c_int32), ("update_chunks", c_void_p),
    ]


class SwaDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("H", c_int32), ("N", c_int32), ("d", c_int32), ("window", c_int32),
                ("io_dtype", c_int32)]


class TttError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libttt.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m linear_attention_chunk_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    L.ttt_abi_version.restype = c_int32
    L.ttt_abi_version.argtypes = []
    L.ttt_status_string.restype = ctypes.c_char_p
    L.ttt_status_string.argtypes = [c_int32]
    L.ttt_last_error.restype = ctypes.c_char_p
    L.ttt_last_error.argtypes = []
    L.ttt_workspace_bytes.restype = c_int32
    L.ttt_workspace_bytes.argtypes = [POINTER(TttDesc), POINTER(c_size_t)]
    L.ttt_forward.restype = c_int32
    L.ttt_forward.argtypes = [POINTER(TttDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    L.ttt_forward_noalloc.restype = c_int32
    L.ttt_forward_noalloc.argtypes = [POINTER(TttDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p]
    L.ttt_backward_workspace_bytes.restype = c_int32
    L.ttt_backward_workspace_bytes.argtypes = [POINTER(TttDesc), POINTER(c_size_t)]
    L.ttt_backward.restype = c_int32
    L.ttt_backward.argtypes = [POINTER(TttDesc)] + [c_void_p] * 13 + [c_size_t, c_void_p]
    L.ttt_record_bytes.restype = c_int32
    L.ttt_record_bytes.argtypes = [POINTER(TttDesc), POINTER(c_size_t), POINTER(c_size_t)]
    L.ttt_forward_record.restype = c_int32
    L.ttt_forward_record.argtypes = [POINTER(TttDesc)] + [c_void_p] * 8 + [c_size_t, c_void_p, c_size_t, c_void_p]
    L.ttt_backward_record_workspace_bytes.restype = c_int32
    L.ttt_backward_record_workspace_bytes.argtypes = [POINTER(TttDesc), POINTER(c_size_t)]
    L.ttt_backward_record.restype = c_int32
    L.ttt_backward_record.argtypes = [POINTER(TttDesc)] + [c_void_p] * 5 + [c_size_t] + [c_void_p] * 8 + \
        [c_size_t, c_void_p]
    L.linattn_workspace_bytes.restype = c_int32
    L.linattn_workspace_bytes.argtypes = [POINTER(LinattnDesc), POINTER(c_size_t)]
    L.linattn_forward.restype = c_int32
    L.linattn_forward.argtypes = [POINTER(LinattnDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    L.linattn_backward_workspace_bytes.restype = c_int32
    L.linattn_backward_workspace_bytes.argtypes = [POINTER(LinattnDesc), POINTER(c_size_t)]
    L.linattn_backward.restype = c_int32
    L.linattn_backward.argtypes = [POINTER(LinattnDesc)] + [c_void_p] * 13 + [c_size_t, c_void_p]
    L.swa_workspace_bytes.restype = c_int32
    L.swa_workspace_bytes.argtypes = [POINTER(SwaDesc), POINTER(c_size_t)]
    L.swa_forward.restype = c_int32
    L.swa_forward.argtypes = [POINTER(SwaDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_size_t, c_void_p]
    L.ttt_profile_enable.restype = c_int32
    L.ttt_profile_enable.argtypes = [c_int32]
    L.ttt_profile_select.restype = c_int32
    L.ttt_profile_select.argtypes = [ctypes.c_uint32]
    L.ttt_profile_read.restype = c_int32
    L.ttt_profile_read.argtypes = [POINTER(c_float), POINTER(c_int32), c_int32]
    L.ttt_profile_kernel_name.restype = ctypes.c_char_p
    L.ttt_profile_kernel_name.argtypes = [c_int32]
    L.ttt_probe_mfma_bf16.restype = c_int32
    L.ttt_probe_mfma_bf16.argtypes = [c_int32, c_int32, ctypes.c_void_p, ctypes.c_void_p]
    _lib = L
    return L


def profile_enable(on: bool) -> None:
    check(lib().ttt_profile_enable(1 if on else 0))


def profile_select(names=None) -> None:
    """Bracket only the named kernel classes (None: every class)."""
    if names is None:
        mask = 0xFFFFFFFF
    else:
        index = {lib().ttt_profile_kernel_name(i).decode(): i for i in range(PROF_KERNELS)}
        mask = 0
        for n in names:
            mask |= 1 << index[n]
    check(lib().ttt_profile_select(mask))


def profile_read() -> dict:
    """{kernel name: (total ms, launches)} since the previous read (waits for the events)."""
    ms = (c_float * PROF_KERNELS)()
    cnt = (c_int32 * PROF_KERNELS)()
    check(lib().ttt_profile_read(ms, cnt, PROF_KERNELS))
    return {lib().ttt_profile_kernel_name(i).decode(): (float(ms[i]), int(cnt[i])) for i in range(PROF_KERNELS)}


def check(status: int) -> None:
    if status != TTT_OK:
        L = lib()
        msg = L.ttt_last_error().decode() or L.ttt_status_string(status).decode()
        raise TttError(status, msg)
