"""fp64 CPU oracle for the TTT-KVB layer, chunked linear attention and LaCT's sliding-window attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU-baseline
leg, never by the product path.  It imports nothing from the HIP library.
"""
from .ttt_ref import *  # noqa: F401,F403
from .swa_ref import swa_scan_ref, swa_forward_ref  # noqa: F401
from .ttt_ref import (  # noqa: F401
    MASK_FULL, MASK_UPDATE_THEN_APPLY, MASK_APPLY_THEN_UPDATE, MASK_STRIDED, MASK_TOKEN_CAUSAL,
    UPD_GD, UPD_GD_L2, UPD_MUON_L2, UPD_MUON,
    swiglu_apply, chunk_gradients, l2_normalize_rows, newton_schulz, chunk_bounds,
    ttt_scan_ref, ttt_forward_ref, linattn_scan_ref, linattn_forward_ref, gemm_intensity,
    linattn_backward_scan_ref, linattn_backward_ref,
    ttt_lastlayer_backward_scan_ref, ttt_lastlayer_backward_ref,
    swiglu_apply_backward, chunk_gradients_backward, ttt_backward_scan_ref, ttt_backward_ref,
    newton_schulz_backward,
)
