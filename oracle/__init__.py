"""CPU oracle for causal sliding-window attention with a RoPE + RMS QK-norm prologue.

TEST INFRASTRUCTURE. This package is a plain, slow, float64 numpy statement of
what the attention path computes. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code,
constants or helpers with the HIP library and never imports it; the library
never imports this package.

Every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against facts that do not come from this code
(library routines, closed forms, finite differences, invariants).
"""

from .prologue import (rope_angles, rope, rope_transpose, rms_norm, rms_norm_bwd,
                       rope_qknorm, rope_qknorm_bwd, round_bf16)
from .gate import ve_gate, ve_gate_bwd, apply_gate, ve_lookup, ve_table_grad
from .attention import (window_mask, segment_ids, visible_mask, attention_fwd,
                        attention_fwd_online, attention_bwd, attention_probs, pair_count)
from .layer import layer_fwd, layer_bwd
from . import fp8

__all__ = [
    "rope_angles", "rope", "rope_transpose", "rms_norm", "rms_norm_bwd", "rope_qknorm",
    "rope_qknorm_bwd", "round_bf16", "ve_gate", "ve_gate_bwd", "apply_gate", "ve_lookup",
    "ve_table_grad", "window_mask",
    "segment_ids", "visible_mask",
    "attention_fwd", "attention_fwd_online", "attention_bwd", "attention_probs", "pair_count",
    "layer_fwd", "layer_bwd", "fp8",
]
