"""GPU parity of the backward with the score gradient stored (swa_bwd_ds and its stages)
against the fp64 oracle, through the C ABI.

The dK/dV kernel stores the bf16 dS^T it forms for dK in 32 x 32 chunks; the dQ kernel reads
them back (dq = scale dS k) instead of recomputing S, P and dP. Cases: edge shapes (sequence
ends inside a chunk, windows around the 32- and 128-row block sizes, W = 1), many tiles, both
head dims, the gate, document masking, the value-embedding table, a NaN-filled workspace
(chunks the dK/dV kernel does not compute must never be read), bitwise repeatability, the
stages against the one call, and the full d24 layers in the launch configuration the
benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import WORKLOADS, make_inputs, small_workload
from gpu_helpers import (announce, check, compare_layer, dev, gpu_layer, host, oracle_layer,
                         rel_l2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


def _stage(wl):
    x = make_inputs(wl)
    qh, _ = oracle.rope_qknorm(x["q"].astype(np.float64), wl.base, wl.eps)
    kh, _ = oracle.rope_qknorm(x["k"].astype(np.float64), wl.base, wl.eps)
    qh, kh = oracle.round_bf16(qh), oracle.round_bf16(kh)
    return qh, kh, x["v"].astype(np.float64), x["dO"].astype(np.float64)


def _run(B, T, H, D, W, seed, stages=False, nan_ws=False):
    wl = small_workload(B, T, H, D, W, "bf16", seed=seed)
    qh, kh, v, dO = _stage(wl)
    tq, tk, tv, tdo = (dev(a, "bf16") for a in (qh, kh, v, dO))
    o, lse = sw.swa_fwd(tq, tk, tv, W)
    ws = None
    if nan_ws:
        ws = torch.empty(sw.swa_bwd_ds_workspace_size(B, T, H, D, W, torch.bfloat16),
                         dtype=torch.uint8, device="cuda")
        ws.view(torch.float32).fill_(float("nan"))
    got = sw.swa_bwd_ds(tq, tk, tv, o, lse, tdo, W, workspace=ws, stages=stages)
    torch.cuda.synchronize()
    Wc = min(W, T)
    _, lse_ref = oracle.attention_fwd(qh, kh, v, Wc, wl.scale)
    refs = oracle.attention_bwd(qh, kh, v, dO, Wc, wl.scale, lse=lse_ref)
    for name, g, r in zip(("dq", "dk", "dv"), got, refs):
        check(name, host(g), r, "bf16")
    return (tq, tk, tv, o, lse, tdo), got


EDGE = []
for T in (1, 17, 100, 129, 300):
    for W in sorted({1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, T - 1, T, T + 5}):
        if W >= 1:
            EDGE.append((T, W))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,W", EDGE)
def test_ds_edge_shapes(T, W, D):
    announce("ds edge", T, W, D)
    _run(2, T, 2, D, W, seed=3000 + 7 * T + W + D)


@pytest.mark.parametrize("T,W,D", [(512, 128, 128), (700, 300, 64), (1024, 1024, 64),
                                   (2048, 1024, 128), (2048, 2048, 128), (333, 1, 128),
                                   (1000, 513, 128)])
def test_ds_many_tiles(T, W, D):
    announce("ds many tiles", T, W, D)
    _run(1, T, 2, D, W, seed=T + W + D + 17)


@pytest.mark.parametrize("T,D", [(100, 64), (300, 128), (129, 128)])
def test_ds_nan_filled_workspace(T, D):
    announce("ds nan workspace", T, D)
    _run(2, T, 3, D, 64, seed=4100 + T + D, nan_ws=True)


def test_ds_stages_equal_one_call_and_repeatable():
    announce("ds stages / repeatability")
    args, g1 = _run(2, 1000, 4, 128, 300, seed=9)
    tq, tk, tv, o, lse, tdo = args
    g2 = sw.swa_bwd_ds(tq, tk, tv, o, lse, tdo, 300)
    g3 = sw.swa_bwd_ds(tq, tk, tv, o, lse, tdo, 300, stages=True)
    # the recomputing stages in the same order (preprocess, dK/dV, dQ)
    ref = sw.swa_bwd_stages(tq, tk, tv, o, lse, tdo, 300, preprocess=True)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a, b) and torch.equal(a, c)
    # dk and dv come from the same dK/dV kernel on the same row terms
    assert torch.equal(g1[1], ref[1]) and torch.equal(g1[2], ref[2])
    assert rel_l2(host(g1[0]), host(ref[0])) <= 1e-2


@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("T,W,D", [(100, 37, 64), (300, 64, 128), (129, 129, 128)])
def test_ds_layer_end_to_end(T, W, D, gate):
    announce("ds e2e", T, W, D, gate)
    wl = small_workload(2, T, 3, D, W, "bf16", seed=700 + T + W, gate=gate, C=96)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, W, bwd="ds")
    fwd, bwd = oracle_layer(x, wl, W)
    compare_layer(g, fwd, bwd, "bf16", gate=gate)


@pytest.mark.parametrize("T,W,D,mean", [(300, 100, 128, 40), (700, 256, 64, 90), (256, 256, 128, 1)])
def test_ds_document_masking(T, W, D, mean):
    announce("ds doc", T, W, D, mean)
    wl = small_workload(2, T, 2, D, W, "bf16", seed=800 + T + mean, doc_mean=mean)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, W, bwd="ds")
    fwd, bwd = oracle_layer(x, wl, W)
    compare_layer(g, fwd, bwd, "bf16")


def test_ds_ve_table():
    announce("ds ve table")
    wl = small_workload(2, 300, 2, 128, 100, "bf16", seed=811, gate=True, C=64, ve_table=True,
                        vocab=37)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, 100, bwd="ds")
    fwd, bwd = oracle_layer(x, wl, 100)
    compare_layer(g, fwd, bwd, "bf16", gate=True)


@pytest.mark.parametrize("name,heads", [("d24_short", [(0, 0), (15, 11), (8, 6)]),
                                        ("d24_full", [(0, 0), (15, 11)]),
                                        ("gpt2_124m", [(0, 0), (7, 11)])])
def test_ds_full_size_sampled_heads(name, heads):
    """Full layer on the route the benchmark times (query prologue inside the forward and dQ
    kernels, the stored-dS backward); the oracle checks whole (b, h) heads."""
    wl = WORKLOADS[name]
    announce("ds full size", name)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, wl.window, bwd="ds", qnorm=True)
    for sel in heads:
        fwd, bwd = oracle_layer(x, wl, wl.window, sel=sel)
        compare_layer(g, fwd, bwd, "bf16", sel=sel)
    assert all(np.all(np.isfinite(host(g[n]))) for n in ("dq", "dk", "dv"))
