"""MI355X-native causal sliding-window attention with a fused RoPE + RMS QK-norm prologue.

The computation lives in libswa.so (HIP kernels for gfx950 behind the C ABI of
include/swa.h); ``binding`` marshals torch GPU tensors into it, one wrapper per entry point.
``inputs`` draws the seeded synthetic workloads.
"""

from . import binding
from .binding import (SwaError, rope_table, rope_qknorm_fwd, rope_qknorm_bwd, ve_gate_v,
                      ve_gate_dv, ve_gate_v_bwd, swa_fwd, swa_bwd, swa_bwd_workspace_size,
                      SWA_WINDOW_FULL)

__all__ = ["binding", "SwaError", "rope_table", "rope_qknorm_fwd", "rope_qknorm_bwd", "ve_gate_v",
           "ve_gate_dv", "ve_gate_v_bwd", "swa_fwd", "swa_bwd", "swa_bwd_workspace_size",
           "SWA_WINDOW_FULL"]
