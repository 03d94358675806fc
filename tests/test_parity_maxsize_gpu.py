"""GPU parity at the largest size the entry points accept: B*T*H*D just under 2^30 elements.

The benchmarked bf16 route (query prologue inside the attention kernels, backward with the
stored score gradient, key prologue in its own passes) and the float32 path run on tensors of
about 2^30 elements (2 GB in bf16, 4 GB in float32), so the rows of the last (b, h) head sit at
the top of the range the kernels' 32-bit buffer offsets and index arithmetic have to cover.

Inputs: N(0, 1) drawn on the device from a seeded torch generator (the host generator of the
inputs module would need tens of GB of host memory at this size); the oracle sees the same
values, copied back head by head. For each sampled head the prologue oracle runs over the whole
sequence (true positions) and the attention oracle on slices, as in the long-sequence test: a
query's output and gradient depend only on the keys of its window, a key's gradients only on
the queries that see it. The prologue backward is row-wise, so it is applied to the sampled rows
alone (zeros elsewhere).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from gpu_helpers import announce, check

pytestmark = pytest.mark.gpu

BASE, EPS = 10000.0, 1e-6
N = 64   # rows / keys per sampled block


def _head(t: torch.Tensor, b: int, h: int) -> np.ndarray:
    """Head (b, h) of a (B, T, H, D) device tensor as a (1, T, 1, D) float64 host array."""
    return t[b, :, h, :].float().cpu().numpy().astype(np.float64)[None, :, None, :]


def _check_head(dt, tensors, b, h, T, W, scale):
    """O, lse, dq (w.r.t. the raw q) on sampled query rows and dk (w.r.t. the raw k), dv on
    sampled keys of head (b, h), against the oracle; also the stored q_hat, k_hat rows."""
    q, k, v, dO = (_head(tensors[n], b, h) for n in ("q", "k", "v", "dO"))
    qh, _ = oracle.rope_qknorm(q, BASE, EPS)
    kh, _ = oracle.rope_qknorm(k, BASE, EPS)
    if dt == "bf16":   # the kernels read the q_hat, k_hat they stored in bf16
        qh, kh = oracle.round_bf16(qh), oracle.round_bf16(kh)
    o, dq, dk, dv = (_head(tensors[n], b, h) for n in ("o", "dq", "dk", "dv"))
    lse = tensors["lse"][b, h].float().cpu().numpy().astype(np.float64)[None, None, :]
    for name in ("qn", "kn"):
        got = _head(tensors[name], b, h)
        want = qh if name == "qn" else kh
        for r0 in (0, T - N):
            check(f"{name}[{b},{h}]", got[:, r0:r0 + N], want[:, r0:r0 + N], dt)
    for r0 in (0, T // 2 + 3, T - N):                  # query rows, incl. the sequence end
        a = max(0, r0 - W + 1)
        sl, rows = slice(a, r0 + N), slice(r0 - a, r0 - a + N)
        O_ref, lse_ref = oracle.attention_fwd(qh[:, sl], kh[:, sl], v[:, sl], W, scale)
        dqh_ref, _, _ = oracle.attention_bwd(qh[:, sl], kh[:, sl], v[:, sl], dO[:, sl], W, scale,
                                             lse=lse_ref)
        dqh = np.zeros_like(q)
        dqh[:, r0:r0 + N] = dqh_ref[:, rows]
        dq_ref = oracle.rope_qknorm_bwd(q, dqh, BASE, EPS)[:, r0:r0 + N]
        check(f"O[{b},{h}]", o[:, r0:r0 + N], O_ref[:, rows], dt)
        check(f"lse[{b},{h}]", lse[:, :, r0:r0 + N], lse_ref[:, :, rows], dt, lse=True)
        check(f"dq[{b},{h}]", dq[:, r0:r0 + N], dq_ref, dt)
    for j0 in (0, T - W - N, T - N):                   # keys, incl. those at the end
        a, e = max(0, j0 - W + 1), min(T, j0 + N + W - 1)
        sl, keys = slice(a, e), slice(j0 - a, j0 - a + N)
        _, lse_ref = oracle.attention_fwd(qh[:, sl], kh[:, sl], v[:, sl], W, scale)
        _, dkh_ref, dv_ref = oracle.attention_bwd(qh[:, sl], kh[:, sl], v[:, sl], dO[:, sl], W,
                                                  scale, lse=lse_ref)
        dkh = np.zeros_like(k)
        dkh[:, j0:j0 + N] = dkh_ref[:, keys]
        dk_ref = oracle.rope_qknorm_bwd(k, dkh, BASE, EPS)[:, j0:j0 + N]
        check(f"dk[{b},{h}]", dk[:, j0:j0 + N], dk_ref, dt)
        check(f"dv[{b},{h}]", dv[:, j0:j0 + N], dv_ref[:, keys], dt)


def _inputs(shape, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return {n: torch.randn(shape, generator=g, device="cuda", dtype=dtype)
            for n in ("q", "k", "v", "dO")}


def test_max_size_bf16_benchmarked_route():
    B, T, H, D, W = 8, 32768, 31, 128, 1024
    assert B * T * H * D < 1 << 30 and B * T * H * D > 0.96 * (1 << 30)
    announce("max size bf16", B, T, H, D, W)
    scale = 1.0 / math.sqrt(D)
    t = _inputs((B, T, H, D), torch.bfloat16, seed=30)
    cs = sw.rope_table(T, D, BASE)
    t["kn"] = sw.rope_qknorm_fwd(None, t["k"], cs, EPS)[1]
    t["qn"], t["o"], t["lse"] = sw.swa_fwd_qnorm(t["q"], cs, t["kn"], t["v"], W, scale, eps=EPS)
    ws = torch.empty(sw.swa_bwd_ds_workspace_size(B, T, H, D, W, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    _, dkn, t["dv"] = sw.swa_bwd_ds(t["qn"], t["kn"], t["v"], t["o"], t["lse"], t["dO"], W, scale,
                                    workspace=ws, stages=True)
    t["dq"] = sw.swa_bwd_dq_ds_qnorm(t["kn"], t["q"], cs, ws, W, scale, eps=EPS)
    del ws
    t["dk"] = sw.rope_qknorm_bwd(None, t["k"], cs, None, dkn, EPS)[1]
    del dkn
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B // 2, 17), (B - 1, H - 1)):
        _check_head("bf16", t, b, h, T, W, scale)
    del t
    torch.cuda.empty_cache()


def test_max_size_f32():
    B, T, H, D, W = 4, 32768, 63, 128, 8
    assert B * T * H * D < 1 << 30 and B * T * H * D > 0.98 * (1 << 30)
    announce("max size f32", B, T, H, D, W)
    scale = 1.0 / math.sqrt(D)
    t = _inputs((B, T, H, D), torch.float32, seed=31)
    cs = sw.rope_table(T, D, BASE)
    t["qn"], t["kn"] = sw.rope_qknorm_fwd(t["q"], t["k"], cs, EPS)
    t["o"], t["lse"] = sw.swa_fwd(t["qn"], t["kn"], t["v"], W, scale)
    dqn, dkn, t["dv"] = sw.swa_bwd(t["qn"], t["kn"], t["v"], t["o"], t["lse"], t["dO"], W, scale)
    t["dq"], t["dk"] = sw.rope_qknorm_bwd(t["q"], t["k"], cs, dqn, dkn, EPS)
    del dqn, dkn
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B // 2, 40), (B - 1, H - 1)):
        _check_head("f32", t, b, h, T, W, scale)
    del t
    torch.cuda.empty_cache()
