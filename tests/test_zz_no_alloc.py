"""swa_bwd_noalloc (the backward on the library's static scratch, for callers that cannot
allocate) against swa_bwd through the C ABI: bitwise equal outputs on consecutive calls, the
second with a smaller input, and the oracle's bars on each."""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
from gpu_helpers import announce, check, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


def _case(B, T, H, D, W, dtype, seed):
    wl = small_workload(B, T, H, D, W, dtype, seed=seed)
    x = make_inputs(wl)
    qh, _ = oracle.rope_qknorm(x["q"].astype(np.float64), wl.base, wl.eps)
    kh, _ = oracle.rope_qknorm(x["k"].astype(np.float64), wl.base, wl.eps)
    if dtype == "bf16":
        qh, kh = oracle.round_bf16(qh), oracle.round_bf16(kh)
    else:
        qh = qh.astype(np.float32).astype(np.float64)
        kh = kh.astype(np.float32).astype(np.float64)
    v, dO = x["v"].astype(np.float64), x["dO"].astype(np.float64)
    return wl, qh, kh, v, dO


def test_noalloc_matches_swa_bwd_on_consecutive_calls():
    cases = [(2, 1000, 4, 128, 300, "bf16", 61),    # first call
             (1, 200, 2, 64, 100, "bf16", 62),      # second call, smaller
             (1, 70, 2, 64, 70, "f32", 63)]         # third, the float32 kernels
    for B, T, H, D, W, dtype, seed in cases:
        announce("noalloc", B, T, H, D, W, dtype)
        wl, qh, kh, v, dO = _case(B, T, H, D, W, dtype, seed)
        tq, tk, tv, tdo = (dev(a, dtype) for a in (qh, kh, v, dO))
        o, lse = sw.swa_fwd(tq, tk, tv, W)
        want = sw.swa_bwd(tq, tk, tv, o, lse, tdo, W)
        got = sw.swa_bwd_noalloc(tq, tk, tv, o, lse, tdo, W)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(g, w), f"{name} differs from swa_bwd"
        _, lse_ref = oracle.attention_fwd(qh, kh, v, W, wl.scale)
        refs = oracle.attention_bwd(qh, kh, v, dO, W, wl.scale, lse=lse_ref)
        for name, g, r in zip(("dq", "dk", "dv"), got, refs):
            check(name, host(g), r, dtype)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    q = torch.zeros(1, 4096, 1024, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1024, 4096, dtype=torch.float32, device="cuda")
    with pytest.raises(sw.SwaError) as e:
        sw.swa_bwd_noalloc(q, q, q, q, lse, q, 128)
    assert e.value.status == 4 and "SWA_NOALLOC_SCRATCH_BYTES" in str(e.value)
