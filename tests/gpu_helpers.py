"""Shared helpers for the GPU parity tests: device transfer, error metrics, bars, runners."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw

# Parity bars: fp32 path max abs error; bf16 path relative L2 error on O, dQ, dK, dV and max
# abs error on the logsumexp.
F32_MAX_ABS = 1e-5
BF16_REL_L2 = 1e-2
BF16_LSE_ABS = 2e-3


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdtype(dtype)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def check(name: str, got: np.ndarray, want: np.ndarray, dtype: str, lse: bool = False,
          sum_scaled: bool = False):
    """Assert the parity bar of `dtype` for one output.

    sum_scaled: the output is a long fp32 sum whose magnitude grows with its length (dgate is a
    sum over D); its fp32 bar is 1e-5 relative to max(1, max |want|).
    """
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if dtype == "f32":
        err = max_abs(got, want)
        if sum_scaled:
            err /= max(1.0, float(np.max(np.abs(want))))
        assert err <= F32_MAX_ABS, f"{name}: max abs {err:.3g} > {F32_MAX_ABS}"
    elif lse:
        err = max_abs(got, want)
        assert err <= BF16_LSE_ABS, f"{name}: lse max abs {err:.3g} > {BF16_LSE_ABS}"
    else:
        err = rel_l2(got, want)
        assert err <= BF16_REL_L2, f"{name}: rel L2 {err:.3g} > {BF16_REL_L2}"
    return err


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def gpu_layer(x: dict, wl, window: int, fused_gate: bool = True, bwd: str = "recompute",
              qnorm: bool = False):
    """Whole layer on the GPU: prologue, optional gate, swa_fwd, swa_bwd, prologue backward.
    fused_gate=False takes the materialised route: ve_gate_v writes v_eff, the attention runs
    without the gate, ve_gate_dv turns dv_eff into dve and dgate. bwd="ds" runs the backward
    with the score gradient stored (swa_bwd_ds) instead of swa_bwd. qnorm=True (with bwd="ds")
    runs the query half of the prologue inside the attention kernels (swa_fwd_qnorm,
    swa_bwd_dq_ds_qnorm) and the prologue calls on k only."""
    dt = wl.dtype
    q, k, v, dO = (dev(x[n], dt) for n in ("q", "k", "v", "dO"))
    cs = sw.rope_table(wl.T, wl.D, wl.base)
    if qnorm:
        assert bwd == "ds"
        qn, kn = None, sw.rope_qknorm_fwd(None, k, cs, wl.eps)[1]
    else:
        qn, kn = sw.rope_qknorm_fwd(q, k, cs, wl.eps)
    out = {"qn": qn, "kn": kn}
    ve = gate = ve_ids = None
    if wl.gate:
        xg = dev(x["x"], dt)
        Wg = torch.from_numpy(x["Wg"]).cuda()
        if "table" in x:   # table mode: the kernels gather the rows by token id
            ve = dev(x["table"], dt)
            ve_ids = torch.from_numpy(x["ids"].astype(np.int32)).cuda()
        else:
            ve = dev(x["ve"], dt)
        if fused_gate:
            gate = sw.ve_gate_v(xg, Wg)
        else:
            gate, v = sw.ve_gate_v(xg, Wg, v, ve, materialize=True, ve_ids=ve_ids)
            ve_kernel = (ve, ve_ids)
            ve = ve_ids = None
        out["gate"] = gate
    bounds = None
    if "doc_id" in x:
        bounds = sw.swa_doc_bounds(torch.from_numpy(x["doc_id"].astype(np.int32)).cuda())
        out["doc_bounds"] = bounds
    fgate = gate if ve is not None else None
    if qnorm:
        qn, o, lse = sw.swa_fwd_qnorm(q, cs, kn, v, window, wl.scale, eps=wl.eps, ve=ve,
                                      gate=fgate, doc_bounds=bounds, ve_ids=ve_ids)
        out["qn"] = qn
    else:
        o, lse = sw.swa_fwd(qn, kn, v, window, wl.scale, ve=ve, gate=fgate, doc_bounds=bounds,
                            ve_ids=ve_ids)
    bwd_fn = sw.swa_bwd_ds if bwd == "ds" else sw.swa_bwd
    ws = None
    if qnorm:
        ws = torch.empty(sw.swa_bwd_ds_workspace_size(wl.B, wl.T, wl.H, wl.D, window,
                                                      q.dtype), dtype=torch.uint8, device="cuda")
    kw = dict(stages=True, workspace=ws) if qnorm else {}
    grads = bwd_fn(qn, kn, v, o, lse, dO, window, wl.scale, ve=ve, gate=fgate,
                   doc_bounds=bounds, ve_ids=ve_ids, **kw)
    if wl.gate and not fused_gate:
        grads = tuple(grads) + sw.ve_gate_dv(grads[2], ve_kernel[0], gate, ve_ids=ve_kernel[1])
    dqn, dkn, dv = grads[:3]
    if qnorm:
        dq = sw.swa_bwd_dq_ds_qnorm(kn, q, cs, ws, window, wl.scale, eps=wl.eps,
                                    doc_bounds=bounds)
        dk = sw.rope_qknorm_bwd(None, k, cs, None, dkn, wl.eps)[1]
    else:
        dq, dk = sw.rope_qknorm_bwd(q, k, cs, dqn, dkn, wl.eps)
    out.update(O=o, lse=lse, dqh=dqn, dkh=dkn, dv=dv, dq=dq, dk=dk)
    if wl.gate:
        out["dve"], out["dgate"] = grads[3], grads[4]
        dWg, dx32 = sw.ve_gate_v_bwd(xg, Wg, gate, grads[4])
        out["dWg"], out["dx32"] = dWg, dx32
    torch.cuda.synchronize()
    return out


def oracle_layer(x: dict, wl, window: int, sel=None):
    """Oracle for the same layer; sel = (b, h) restricts to one sequence and head."""
    f = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "dO")}
    kw = dict(base=wl.base, eps=wl.eps, scale=wl.scale)
    gk = {}
    if wl.gate:
        if "table" in x:
            ve = oracle.ve_lookup(x["table"].astype(np.float64), x["ids"])
        else:
            ve = x["ve"].astype(np.float64)
        gk = dict(x32=x["x"][..., :32].astype(np.float64), Wg=x["Wg"].astype(np.float64), ve=ve)
    doc = x.get("doc_id")
    if sel is not None:
        b, h = sel
        f = {n: a[b:b + 1, :, h:h + 1] for n, a in f.items()}
        doc = doc[b:b + 1] if doc is not None else None
        if wl.gate:
            D = wl.D
            gk = dict(x32=gk["x32"][b:b + 1], Wg=gk["Wg"][:, h:h + 1],
                      ve=gk["ve"][b:b + 1, :, h * D:(h + 1) * D])
    fwd = oracle.layer_fwd(f["q"], f["k"], f["v"], window, round_boundary=(wl.dtype == "bf16"),
                           doc_id=doc, **kw, **gk)
    bwd = oracle.layer_bwd(f["q"], f["k"], f["v"], f["dO"], window, fwd, doc_id=doc, **kw, **gk)
    if wl.gate and "table" in x and sel is None:
        bwd["dtable"] = oracle.ve_table_grad(bwd["dve"], x["ids"], x["table"].shape[0])
    return fwd, bwd


def compare_layer(g: dict, fwd: dict, bwd: dict, dtype: str, sel=None, gate=False):
    """Compare GPU outputs (optionally the (b, h) slice) with the oracle; returns errors."""
    def pick(name, t, layout="bthd"):
        a = host(t)
        if sel is None:
            return a
        b, h = sel
        if layout == "bthd":
            return a[b:b + 1, :, h:h + 1]
        if layout == "bht":
            return a[b:b + 1, h:h + 1]
        if layout == "bth":
            return a[b:b + 1, :, h:h + 1]
        raise ValueError(layout)

    errs = {}
    errs["O"] = check("O", pick("O", g["O"]), fwd["O"], dtype)
    errs["lse"] = check("lse", pick("lse", g["lse"], "bht"), fwd["lse"], dtype, lse=True)
    for n in ("dqh", "dkh", "dq", "dk", "dv"):
        errs[n] = check(n, pick(n, g[n]), bwd[n], dtype)
    if gate:
        errs["gate"] = check("gate", pick("gate", g["gate"], "bth"), fwd["g"], "f32")
        if sel is None:
            B, T, H, D = g["O"].shape
            if "dtable" in bwd:   # a float sum over the tokens of each id
                errs["dtable"] = check("dtable", host(g["dve"]), bwd["dtable"], dtype,
                                       sum_scaled=True)
            else:
                errs["dve"] = check("dve", host(g["dve"]), bwd["dve"], dtype)
            errs["dgate"] = check("dgate", host(g["dgate"]), bwd["dg"], dtype, sum_scaled=True)
    return errs
