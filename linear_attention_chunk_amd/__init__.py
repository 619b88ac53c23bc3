"""MI355X (gfx950) large-chunk TTT-KVB layer and chunked linear attention.

The computation lives in libttt.so (hand-written HIP kernels behind the C ABI of include/ttt.h);
this package only marshals PyTorch tensors into that ABI.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, LinattnDesc, SwaDesc, TttDesc, TttError, lib,
    MASK_FULL, MASK_UPDATE_THEN_APPLY, MASK_APPLY_THEN_UPDATE, MASK_STRIDED, MASK_TOKEN_CAUSAL,
    UPD_GD, UPD_GD_L2, UPD_MUON_L2, UPD_MUON, TTT_F32, TTT_BF16,
)


def __getattr__(name):
    # the torch-based binding is imported on first use, so the ctypes layer loads without torch
    if name in ("ttt_forward", "ttt_forward_noalloc", "linattn_forward", "pack_weights", "unpack_weights", "ttt_desc", "linattn_desc",
                "ttt_workspace_bytes", "linattn_workspace_bytes", "swa_forward", "swa_workspace_bytes",
                "linattn_backward", "linattn_backward_workspace_bytes", "ttt_backward",
                "ttt_backward_workspace_bytes", "ttt_forward_record", "ttt_record_bytes"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
