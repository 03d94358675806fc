"""GPU parity on long sequences (T = 32768), where offsets reach into the hundreds of megabytes.

The oracle is the dense definition, too large at this length, so it runs on slices: a query's
output and dq depend only on the keys of its window, and a key's dk, dv only on the queries
that see it (whose windows start at most W - 1 before the key). For a block of rows r0..r0+n
the slice [r0 - W + 1, r0 + n) of (q_hat, k_hat, v, dO) reproduces their O, lse and dq; for a
block of keys j0..j0+n the slice [j0 - W + 1, j0 + n + W - 1) reproduces their dk and dv. q_hat
and k_hat come from the oracle prologue over the whole sequence (true positions), so the
slices need only the attention oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
from gpu_helpers import announce, check, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("W", [1024, 4096])
def test_long_sequence_sampled_rows_and_keys(W):
    B, T, H, D = 1, 32768, 2, 128
    announce("long sequence", T, W)
    wl = small_workload(B, T, H, D, W, "bf16", seed=W)
    x = make_inputs(wl)
    qh = oracle.round_bf16(oracle.rope_qknorm(x["q"].astype(np.float64), wl.base, wl.eps)[0])
    kh = oracle.round_bf16(oracle.rope_qknorm(x["k"].astype(np.float64), wl.base, wl.eps)[0])
    v, dO = x["v"].astype(np.float64), x["dO"].astype(np.float64)
    tq, tk, tv, tdo = (dev(a, "bf16") for a in (qh, kh, v, dO))
    o, lse = sw.swa_fwd(tq, tk, tv, W, wl.scale)
    dq, dk, dv = sw.swa_bwd(tq, tk, tv, o, lse, tdo, W, wl.scale)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (host(t) for t in (o, lse, dq, dk, dv))
    n = 64
    for r0 in (0, 5000, T // 2 + 3, T - n):          # query rows, incl. the sequence end
        a = max(0, r0 - W + 1)
        sl = slice(a, r0 + n)
        O_ref, lse_ref = oracle.attention_fwd(qh[:, sl], kh[:, sl], v[:, sl], W, wl.scale)
        dq_ref, _, _ = oracle.attention_bwd(qh[:, sl], kh[:, sl], v[:, sl], dO[:, sl], W,
                                            wl.scale, lse=lse_ref)
        rows = slice(r0 - a, r0 - a + n)
        check("O", o[:, r0:r0 + n], O_ref[:, rows], "bf16")
        check("lse", lse[:, :, r0:r0 + n], lse_ref[:, :, rows], "bf16", lse=True)
        check("dq", dq[:, r0:r0 + n], dq_ref[:, rows], "bf16")
    for j0 in (0, 7777, T - W - n, T - n):            # keys, incl. those near the end
        a, b = max(0, j0 - W + 1), min(T, j0 + n + W - 1)
        sl = slice(a, b)
        _, lse_ref = oracle.attention_fwd(qh[:, sl], kh[:, sl], v[:, sl], W, wl.scale)
        _, dk_ref, dv_ref = oracle.attention_bwd(qh[:, sl], kh[:, sl], v[:, sl], dO[:, sl], W,
                                                 wl.scale, lse=lse_ref)
        keys = slice(j0 - a, j0 - a + n)
        check("dk", dk[:, j0:j0 + n], dk_ref[:, keys], "bf16")
        check("dv", dv[:, j0:j0 + n], dv_ref[:, keys], "bf16")
