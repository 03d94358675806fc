"""GPU checks of the backward's row terms and workspace, through the C ABI.

* The row terms delta_i = dO_i . O_i and lse_i (stored negated, lse in log2 units) that
  swa_bwd_preprocess and swa_bwd_dq_rowterms write are compared with the oracle's
  delta = sum_d dO * O and lse ("GPT-2 124M 复现" §19: the backward recomputes P from the
  scores and the saved row statistics).
* A workspace that holds NaN bit patterns before the call (an allocation that is reused,
  never cleared) must not leak into the gradients: the last 128-query tile of the last head
  reads rows past the sequence end, whose queries are masked.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
from gpu_helpers import BF16_LSE_ABS, announce, check, dev, host, rel_l2

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


def _stage(wl):
    """q_hat, k_hat from the oracle prologue rounded to the storage type; v, dO as drawn."""
    x = make_inputs(wl)
    qh, _ = oracle.rope_qknorm(x["q"].astype(np.float64), wl.base, wl.eps)
    kh, _ = oracle.rope_qknorm(x["k"].astype(np.float64), wl.base, wl.eps)
    if wl.dtype == "bf16":
        qh, kh = oracle.round_bf16(qh), oracle.round_bf16(kh)
    else:
        qh = qh.astype(np.float32).astype(np.float64)
        kh = kh.astype(np.float32).astype(np.float64)
    return qh, kh, x["v"].astype(np.float64), x["dO"].astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("writer", ["preprocess", "dq_rowterms"])
def test_row_terms_against_oracle(writer, D, dtype):
    B, T, H, W = 2, 300, 3, 100
    announce("row terms", writer, D, dtype)
    wl = small_workload(B, T, H, D, W, dtype, seed=41 + D)
    qh, kh, v, dO = _stage(wl)
    tq, tk, tv, tdo = (dev(a, dtype) for a in (qh, kh, v, dO))
    o, lse = sw.swa_fwd(tq, tk, tv, W)
    ws = torch.empty(sw.swa_bwd_workspace_size(B, T, H, D, tq.dtype), dtype=torch.uint8,
                     device="cuda")
    if writer == "preprocess":
        sw.swa_bwd_preprocess(o, tdo, lse, ws)
    else:
        sw.swa_bwd_stages(tq, tk, tv, o, lse, tdo, W, workspace=ws)
    torch.cuda.synchronize()
    nd, nl = (host(t) for t in sw.rowterm_views(ws, B, T, H))
    O_ref, lse_ref = oracle.attention_fwd(qh, kh, v, W, wl.scale)
    delta_ref = np.sum(dO * O_ref, axis=-1).transpose(0, 2, 1)          # (B, H, T)
    # against the oracle: the bars of O (relative L2) and of lse (max abs)
    assert rel_l2(-nd, delta_ref) <= (1e-5 if dtype == "f32" else 1e-2)
    check("lse from the row term", -nl / LOG2E, lse_ref, dtype, lse=(dtype == "bf16"))
    # against the float64 dot product of the GPU's own O and dO (the kernel's float32 sum)
    delta_own = np.sum(dO * host(o), axis=-1).transpose(0, 2, 1)
    scale = np.sqrt(np.sum(dO ** 2, axis=-1) * np.sum(host(o) ** 2, axis=-1)).transpose(0, 2, 1)
    assert np.max(np.abs(-nd - delta_own) / np.maximum(scale, 1.0)) <= 1e-5
    np.testing.assert_allclose(-nl, host(lse) * LOG2E, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("T", [100, 300])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("preprocess", [False, True])
def test_nan_filled_workspace(T, D, preprocess):
    """The workspace is filled with NaN before the backward; every gradient must still be
    finite and match the oracle (the row terms past the end of the last head are masked
    queries, written as zeros by the kernels that write the row terms)."""
    B, H, W = 2, 3, 64
    announce("nan workspace", T, D, preprocess)
    wl = small_workload(B, T, H, D, W, "bf16", seed=900 + T + D)
    qh, kh, v, dO = _stage(wl)
    tq, tk, tv, tdo = (dev(a, "bf16") for a in (qh, kh, v, dO))
    o, lse = sw.swa_fwd(tq, tk, tv, W)
    ws = torch.empty(sw.swa_bwd_workspace_size(B, T, H, D, tq.dtype), dtype=torch.uint8,
                     device="cuda")
    ws.view(torch.float32).fill_(float("nan"))
    dq, dk, dv = sw.swa_bwd_stages(tq, tk, tv, o, lse, tdo, W, workspace=ws,
                                   preprocess=preprocess)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attention_fwd(qh, kh, v, W, wl.scale)
    refs = oracle.attention_bwd(qh, kh, v, dO, W, wl.scale, lse=lse_ref)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = host(got)
        assert np.all(np.isfinite(g)), f"{name}: non-finite values"
        check(name, g, want, "bf16")
