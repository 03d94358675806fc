"""GPU parity of document-masked attention (a token attends only inside its own document)
against the oracle, through the C ABI: the document-bounds kernel, whole layers on small
shapes (ragged tails, single-token documents, documents longer than the window), the full
d24 short layer on BOS-aligned packed rows, the staged backward and repeatability."""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import (WORKLOADS, doc_layout, make_inputs,
                                                   small_workload)
from gpu_helpers import announce, check, compare_layer, dev, gpu_layer, host, oracle_layer

pytestmark = pytest.mark.gpu


def _expected_bounds(ids: np.ndarray) -> np.ndarray:
    """[start, end) of each token's run from the oracle's segment numbering."""
    seg = oracle.segment_ids(ids)
    B, T = ids.shape
    out = np.zeros((B, T, 2), dtype=np.int64)
    for b in range(B):
        vals, first, counts = np.unique(seg[b], return_index=True, return_counts=True)
        out[b, :, 0] = first[seg[b]]
        out[b, :, 1] = first[seg[b]] + counts[seg[b]]
    return out


@pytest.mark.parametrize("B,T,mean", [(1, 1, 1), (3, 7, 2), (2, 1023, 40), (2, 1024, 1),
                                      (1, 1025, 300), (3, 3000, 100)])
def test_doc_bounds_kernel(B, T, mean):
    announce("doc bounds", B, T, mean)
    ids = doc_layout(np.random.default_rng(B * 1000 + T), B, T, mean)
    got = sw.swa_doc_bounds(torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), _expected_bounds(ids))


def test_doc_bounds_runs_of_repeated_ids():
    """Ids that come back later start a new document (runs, not equal values)."""
    ids = np.array([[5, 5, 7, 7, 7, 5, 9, 9]], dtype=np.int32)
    got = sw.swa_doc_bounds(torch.from_numpy(ids).cuda()).cpu().numpy()
    np.testing.assert_array_equal(got[0, :, 0], [0, 0, 2, 2, 2, 5, 6, 6])
    np.testing.assert_array_equal(got[0, :, 1], [2, 2, 5, 5, 5, 6, 8, 8])


DOC_CASES = [(100, 100, 64, "bf16", 10), (129, 64, 128, "bf16", 40), (300, 77, 128, "bf16", 2),
             (700, 300, 64, "bf16", 200), (1100, 1100, 128, "bf16", 600), (257, 257, 128, "f32", 30),
             (64, 16, 64, "f32", 8), (2048, 1024, 128, "bf16", 512)]


@pytest.mark.parametrize("T,W,D,dtype,mean", DOC_CASES)
def test_layer_with_documents(T, W, D, dtype, mean):
    announce("doc e2e", T, W, D, dtype, mean)
    wl = small_workload(2, T, 2, D, W, dtype, seed=900 + T + W + mean, doc_mean=mean)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, W)
    fwd, bwd = oracle_layer(x, wl, W)
    errs = compare_layer(g, fwd, bwd, dtype)
    print("doc", T, W, D, dtype, mean, {k: f"{v:.2e}" for k, v in errs.items()})


def test_layer_with_documents_and_gate():
    wl = small_workload(2, 300, 3, 128, 100, "bf16", seed=77, gate=True, C=64, doc_mean=50)
    announce("doc e2e gate")
    x = make_inputs(wl)
    g = gpu_layer(x, wl, 100)
    fwd, bwd = oracle_layer(x, wl, 100)
    compare_layer(g, fwd, bwd, "bf16", gate=True)


@pytest.mark.parametrize("route", ["recompute", "benchmarked"])
def test_full_size_documents_sampled_heads(route):
    """The d24 short layer (B=16, T=2048, H=12, D=128, W=1024) on packed rows with ~512-token
    documents, whole (b, h) heads checked: on the recomputing backward with the separate
    prologue, and on the route the benchmark times (query prologue inside the forward and dQ
    kernels, backward with the stored score gradient)."""
    wl = WORKLOADS["d24_short_doc"]
    announce("full size docs", route)
    x = make_inputs(wl)
    if route == "benchmarked":
        g = gpu_layer(x, wl, wl.window, bwd="ds", qnorm=True)
    else:
        g = gpu_layer(x, wl, wl.window)
    for sel in ((0, 0), (15, 11), (7, 4)):
        fwd, bwd = oracle_layer(x, wl, wl.window, sel=sel)
        errs = compare_layer(g, fwd, bwd, wl.dtype, sel=sel)
        print("docs", sel, {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_token_documents(dtype):
    """Every token its own document: P = 1 on the diagonal, so O = V exactly; dv = dO (exactly
    in fp32; the bf16 backward recomputes S with K rounded after its scale * log2(e)
    pre-scaling, so there P = 1 only to ~2^-9 relative and dv meets the bf16 bar); dq = dk = 0
    up to rounding."""
    B, T, H, D = 2, 200, 2, 64
    announce("single-token docs", dtype)
    rng = np.random.default_rng(3)
    q, k, v, dO = (dev(rng.standard_normal((B, T, H, D)), dtype) for _ in range(4))
    ids = torch.arange(T, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    bounds = sw.swa_doc_bounds(ids)
    o, lse = sw.swa_fwd(q, k, v, 100, doc_bounds=bounds)
    dq, dk, dv = sw.swa_bwd(q, k, v, o, lse, dO, 100, doc_bounds=bounds)
    torch.cuda.synchronize()
    assert torch.equal(o, v)
    if dtype == "f32":
        assert torch.equal(dv, dO)
    else:
        check("dv", host(dv), host(dO), dtype)
    assert float(dq.float().abs().max()) < 1e-2 and float(dk.float().abs().max()) < 1e-2


def test_documents_staged_backward_and_repeatability():
    wl = small_workload(2, 1000, 4, 128, 300, "bf16", seed=19, doc_mean=150)
    announce("doc stages/repeat")
    x = make_inputs(wl)
    q, k, v, dO = (dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
    bounds = sw.swa_doc_bounds(torch.from_numpy(x["doc_id"]).cuda())
    o1, l1 = sw.swa_fwd(q, k, v, 300, doc_bounds=bounds)
    o2, l2 = sw.swa_fwd(q, k, v, 300, doc_bounds=bounds)
    g1 = sw.swa_bwd(q, k, v, o1, l1, dO, 300, doc_bounds=bounds)
    g2 = sw.swa_bwd_stages(q, k, v, o1, l1, dO, 300, doc_bounds=bounds)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # without the bounds the same inputs give different results (the mask is in effect)
    o3, _ = sw.swa_fwd(q, k, v, 300)
    torch.cuda.synchronize()
    assert not torch.equal(o1, o3)
