"""GPU parity of the longest-first block order (small full-causal grids) against the fp64 oracle.

With window >= T, no document masking, a head count B * H divisible by 8 and the re-read
per-head tiles of one XCD's heads within its L2, the forward, dK/dV and stored-dS dQ kernels
map workgroup ids to (head, block) longest first across the heads of each XCD instead of head
by head. These cases take that order (several heads per XCD, a ragged last block, window
beyond T, both head dims) and check O, the logsumexp and every gradient of both backward
routes, so that a block the order dropped or visited twice shows up as a mismatch.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import small_workload, make_inputs
from gpu_helpers import announce, check, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


@pytest.mark.parametrize("B,T,H,D,W", [(2, 300, 4, 64, 300), (2, 1024, 8, 64, 1024),
                                       (1, 640, 8, 128, 700), (4, 129, 4, 128, 129),
                                       (8, 256, 12, 64, 4096)])
def test_longest_first_order(B, T, H, D, W):
    announce("longest-first order", B, T, H, D, W)
    wl = small_workload(B, T, H, D, W, "bf16", seed=9100 + T + H + D)
    x = make_inputs(wl)
    qh, _ = oracle.rope_qknorm(x["q"].astype(np.float64), wl.base, wl.eps)
    kh, _ = oracle.rope_qknorm(x["k"].astype(np.float64), wl.base, wl.eps)
    qh, kh = oracle.round_bf16(qh), oracle.round_bf16(kh)
    v, dO = x["v"].astype(np.float64), x["dO"].astype(np.float64)
    tq, tk, tv, tdo = (dev(a, "bf16") for a in (qh, kh, v, dO))
    o, lse = sw.swa_fwd(tq, tk, tv, W)
    rc = sw.swa_bwd(tq, tk, tv, o, lse, tdo, W)
    ds = sw.swa_bwd_ds(tq, tk, tv, o, lse, tdo, W)
    torch.cuda.synchronize()
    Wc = min(W, T)
    o_ref, lse_ref = oracle.attention_fwd(qh, kh, v, Wc, wl.scale)
    check("O", host(o), o_ref, "bf16")
    check("lse", host(lse), lse_ref, "bf16", lse=True)
    refs = oracle.attention_bwd(qh, kh, v, dO, Wc, wl.scale, lse=lse_ref)
    for route, got in (("recompute", rc), ("stored dS", ds)):
        for name, g, r in zip(("dq", "dk", "dv"), got, refs):
            check(f"{route} {name}", host(g), r, "bf16")
