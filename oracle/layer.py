"""Oracle for one whole attention-core call: prologue, optional gate, attention; and its backward.

TEST INFRASTRUCTURE (see the package docstring).

Order of the steps ("从4万美元到73美元：GPT-2复现的成本革命" §2.2 and the lanjinlin.com.cn
repost, "1." and "3."): q_hat = RMSNorm(RoPE(q)), k_hat = RMSNorm(RoPE(k)),
v_eff = v + 2 sigmoid(x[:, :, :32] Wg) * ve (gate workloads only), then
attention with scale 1/sqrt(D) and the per-layer window.

``round_boundary=True`` rounds q_hat and k_hat to bfloat16, which is where
the library stores them between its prologue and its attention calls; the
rest stays float64.
"""

from __future__ import annotations

import numpy as np

from .prologue import rope_qknorm, rope_qknorm_bwd, round_bf16
from .gate import ve_gate, apply_gate, ve_gate_bwd
from .attention import attention_fwd, attention_bwd


def layer_fwd(q, k, v, window, *, base=10000.0, eps=1e-6, scale=None, x32=None, Wg=None, ve=None,
              round_boundary=False, doc_id=None):
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    qh, rq = rope_qknorm(q, base, eps)
    kh, rk = rope_qknorm(k, base, eps)
    if round_boundary:
        qh, kh = round_bf16(qh), round_bf16(kh)
    out = {"qh": qh, "kh": kh, "rq": rq, "rk": rk}
    if Wg is not None:
        g = ve_gate(x32, Wg)
        v_eff = apply_gate(v, g, ve)
        out["g"] = g
    else:
        v_eff = v
    out["v_eff"] = v_eff
    O, lse = attention_fwd(qh, kh, v_eff, window, scale, doc_id=doc_id)
    out["O"], out["lse"] = O, lse
    return out


def layer_bwd(q, k, v, dO, window, fwd, *, base=10000.0, eps=1e-6, scale=None, x32=None, Wg=None,
              ve=None, doc_id=None):
    """Gradients w.r.t. the pre-RoPE q, k, the raw v (and ve, Wg, x32 with the gate)."""
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    dqh, dkh, dv_eff = attention_bwd(fwd["qh"], fwd["kh"], fwd["v_eff"], dO, window, scale,
                                     lse=fwd["lse"], doc_id=doc_id)
    out = {"dqh": dqh, "dkh": dkh, "dv_eff": dv_eff}
    out["dq"] = rope_qknorm_bwd(q, dqh, base, eps)
    out["dk"] = rope_qknorm_bwd(k, dkh, base, eps)
    if Wg is not None:
        dv, dve, dg, dWg, dx32 = ve_gate_bwd(x32, Wg, fwd["g"], dv_eff, ve)
        out.update(dv=dv, dve=dve, dg=dg, dWg=dWg, dx32=dx32)
    else:
        out["dv"] = dv_eff
    return out
