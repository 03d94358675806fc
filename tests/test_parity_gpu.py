"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded inputs.

Bars: fp32 path max abs error <= 1e-5; bf16 path relative L2 error <= 1e-2 on O, dq, dk, dv
(and the other gradients) and max abs error <= 2e-3 on the logsumexp. In the bf16 path the
oracle rounds q_hat and k_hat to bf16, which is where the library stores them; everything else
in the oracle is float64.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import (WORKLOADS, make_inputs, small_workload,
                                                   sssl_layer_workload)
from gpu_helpers import (announce, check, compare_layer, dev, gpu_layer, host, oracle_layer,
                         rel_l2, max_abs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


# ------------------------------------------------------------------------------ prologue

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_qknorm_fwd_bwd(dtype, D):
    wl = small_workload(2, 37, 3, D, 37, dtype, seed=11)
    announce("rope_qknorm", dtype, D)
    x = make_inputs(wl)
    q, k, g1, g2 = (dev(x[n], dtype) for n in ("q", "k", "v", "dO"))
    cs = sw.rope_table(wl.T, D, wl.base)
    ang = oracle.rope_angles(wl.T, D, wl.base)
    np.testing.assert_allclose(host(cs)[..., 0], np.cos(ang), atol=1e-7)
    np.testing.assert_allclose(host(cs)[..., 1], np.sin(ang), atol=1e-7)
    qn, kn = sw.rope_qknorm_fwd(q, k, cs, wl.eps)
    dq, dk = sw.rope_qknorm_bwd(q, k, cs, g1, g2, wl.eps)
    for src, gn, outn, outd in (("q", "v", qn, dq), ("k", "dO", kn, dk)):
        xs = x[src].astype(np.float64)
        want, _ = oracle.rope_qknorm(xs, wl.base, wl.eps)
        check(f"{src}_hat", host(outn), want, dtype)
        wantd = oracle.rope_qknorm_bwd(xs, x[gn].astype(np.float64), wl.base, wl.eps)
        check(f"d{src}", host(outd), wantd, dtype)


# ------------------------------------------------------------------------------ attention stage

def _stage_inputs(wl):
    """q_hat, k_hat from the oracle prologue, rounded to the storage type; v, dO as drawn."""
    x = make_inputs(wl)
    qh, _ = oracle.rope_qknorm(x["q"].astype(np.float64), wl.base, wl.eps)
    kh, _ = oracle.rope_qknorm(x["k"].astype(np.float64), wl.base, wl.eps)
    if wl.dtype == "bf16":
        qh, kh = oracle.round_bf16(qh), oracle.round_bf16(kh)
    else:
        qh, kh = qh.astype(np.float32).astype(np.float64), kh.astype(np.float32).astype(np.float64)
    return qh, kh, x["v"].astype(np.float64), x["dO"].astype(np.float64)


def _run_stage(wl, window):
    qh, kh, v, dO = _stage_inputs(wl)
    dt = wl.dtype
    tq, tk, tv, tdo = dev(qh, dt), dev(kh, dt), dev(v, dt), dev(dO, dt)
    o, lse = sw.swa_fwd(tq, tk, tv, window, wl.scale)
    dq, dk, dv = sw.swa_bwd(tq, tk, tv, o, lse, tdo, window, wl.scale)
    torch.cuda.synchronize()
    W = wl.T if window == sw.SWA_WINDOW_FULL else window
    O_ref, lse_ref = oracle.attention_fwd(qh, kh, v, W, wl.scale)
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd(qh, kh, v, dO, W, wl.scale, lse=lse_ref)
    check("O", host(o), O_ref, dt)
    check("lse", host(lse), lse_ref, dt, lse=True)
    check("dq", host(dq), dq_ref, dt)
    check("dk", host(dk), dk_ref, dt)
    check("dv", host(dv), dv_ref, dt)


EDGE = []
for T in (1, 17, 100, 129):
    for W in sorted({1, 2, 63, 64, 65, T - 1, T, T + 5}):
        if W >= 1:
            EDGE.append((T, W))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,W", EDGE)
def test_attention_stage_edge_shapes(T, W, D, dtype):
    announce("stage", T, W, D, dtype)
    wl = small_workload(2, T, 2, D, W, dtype, seed=1000 + T * 7 + W)
    _run_stage(wl, W)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_full_window_sentinel(dtype):
    announce("stage full sentinel", dtype)
    wl = small_workload(1, 200, 3, 64, 200, dtype, seed=77)
    _run_stage(wl, sw.SWA_WINDOW_FULL)


@pytest.mark.parametrize("T,W,D", [(512, 128, 128), (700, 300, 64), (1024, 1024, 64),
                                   (2048, 1024, 128), (2048, 2048, 128), (333, 1, 128)])
def test_attention_stage_many_tiles(T, W, D):
    announce("stage many tiles", T, W, D)
    wl = small_workload(1, T, 2, D, W, "bf16", seed=T + W + D)
    _run_stage(wl, W)


# ------------------------------------------------------------------------------ end to end

def test_tiny_f32_layer_end_to_end():
    """The tiny fp32 causal workload (B=1, T=64, H=2, D=64, seed 0): whole layer, fp32 bar."""
    wl = WORKLOADS["tiny_f32"]
    announce("tiny_f32 e2e")
    x = make_inputs(wl)
    g = gpu_layer(x, wl, wl.window)
    fwd, bwd = oracle_layer(x, wl, wl.window)
    errs = compare_layer(g, fwd, bwd, "f32")
    print("tiny_f32 errors", {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("T,W,D", [(100, 37, 64), (129, 129, 128), (300, 64, 128)])
def test_layer_end_to_end_small(T, W, D, gate, dtype):
    announce("e2e small", T, W, D, gate, dtype)
    wl = small_workload(2, T, 3, D, W, dtype, seed=500 + T + W, gate=gate, C=96)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, W)
    fwd, bwd = oracle_layer(x, wl, W)
    compare_layer(g, fwd, bwd, dtype, gate=gate)
    if gate:
        bar = 1e-4 if dtype == "f32" else 1e-2
        assert rel_l2(host(g["dWg"]), bwd["dWg"]) <= bar
        check("dx32", host(g["dx32"]), bwd["dx32"], dtype)


# ------------------------------------------------------------------------------ full sizes

FULL = [("gpt2_124m", [(0, 0), (7, 11), (3, 5)]),
        ("d24_short", [(0, 0), (15, 11), (8, 6)]),
        ("d24_full", [(0, 0), (15, 11)]),
        ("d24_short_ve", [(0, 0), (15, 11)])]


@pytest.mark.parametrize("name,heads", FULL)
def test_full_size_sampled_heads(name, heads):
    """Full workload on the GPU, at the benchmark's shapes, on the recomputing backward with the
    separate prologue (the benchmarked route has its own full-size test with the stored-dS
    backward); the oracle checks whole (b, h) heads (every query row and every gradient of those
    heads)."""
    wl = WORKLOADS[name]
    announce("full size", name)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, wl.window)
    for sel in heads:
        fwd, bwd = oracle_layer(x, wl, wl.window, sel=sel)
        errs = compare_layer(g, fwd, bwd, wl.dtype, sel=sel, gate=wl.gate)
        print(name, sel, {k: f"{v:.2e}" for k, v in errs.items()})
    # properties over all heads: finite outputs, lse within its bounds
    lse = host(g["lse"])
    T, W = wl.T, wl.window
    assert np.all(np.isfinite(lse))
    cnt = np.minimum(np.arange(T) + 1, W).astype(np.float64)
    sD = math.sqrt(wl.D)  # |s| <= sqrt(D) after QK-norm
    assert np.all(lse <= np.log(cnt) + sD + 1e-2) and np.all(lse >= np.log(cnt) - sD - 1e-2)


def test_sssl_sweep_layers_sampled():
    """Two layers of the 24-layer 3-short:1-long sweep (a short and a full one), one head each."""
    for layer in (2, 3):
        wl = sssl_layer_workload(layer)
        announce("sssl layer", layer, wl.window)
        x = make_inputs(wl)
        g = gpu_layer(x, wl, wl.window)
        fwd, bwd = oracle_layer(x, wl, wl.window, sel=(layer, layer))
        compare_layer(g, fwd, bwd, "bf16", sel=(layer, layer))


# ------------------------------------------------------------------------------ repeatability

def test_forward_and_backward_bitwise_repeatable():
    wl = small_workload(2, 1000, 4, 128, 300, "bf16", seed=9)
    announce("repeatability")
    qh, kh, v, dO = _stage_inputs(wl)
    tq, tk, tv, tdo = (dev(a, "bf16") for a in (qh, kh, v, dO))
    o1, l1 = sw.swa_fwd(tq, tk, tv, 300)
    o2, l2 = sw.swa_fwd(tq, tk, tv, 300)
    g1 = sw.swa_bwd(tq, tk, tv, o1, l1, tdo, 300)
    g2 = sw.swa_bwd(tq, tk, tv, o1, l1, tdo, 300)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # no atomics anywhere: every output is written by exactly one wave, in a fixed order
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # the C-ABI stages in the one-call order (dQ with the row terms, then dK/dV) give exactly
    # what the one-call backward gives
    g3 = sw.swa_bwd_stages(tq, tk, tv, o1, l1, tdo, 300)
    torch.cuda.synchronize()
    for a, b in zip(g1, g3):
        assert torch.equal(a, b)
    # the other order (preprocess, dK/dV, dQ) differs only by the rounding of delta's sum
    g4 = sw.swa_bwd_stages(tq, tk, tv, o1, l1, tdo, 300, preprocess=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g4):
        assert rel_l2(host(a), host(b)) <= 1e-3


def test_gate_kernels_against_oracle():
    wl = small_workload(3, 77, 5, 64, 77, "bf16", seed=31, gate=True, C=80)
    announce("gate kernels")
    x = make_inputs(wl)
    xg = dev(x["x"], "bf16")
    Wg = torch.from_numpy(x["Wg"]).cuda()
    v, ve = dev(x["v"], "bf16"), dev(x["ve"], "bf16")
    gate, v_eff = sw.ve_gate_v(xg, Wg, v, ve, materialize=True)
    g_ref = oracle.ve_gate(x["x"][..., :32].astype(np.float64), x["Wg"].astype(np.float64))
    check("gate", host(gate), g_ref, "f32")
    ve_ref = oracle.apply_gate(x["v"].astype(np.float64), g_ref, x["ve"].astype(np.float64))
    check("v_eff", host(v_eff), ve_ref, "bf16")
    # oracle gate backward for a random upstream dv_eff; its dgate (rounded to fp32) drives the GPU
    dv_eff = np.random.default_rng(5).standard_normal(x["v"].shape)
    x32 = x["x"][..., :32].astype(np.float64)
    _, _, dg_ref, dWg_ref, dx_ref = oracle.ve_gate_bwd(x32, x["Wg"].astype(np.float64), g_ref,
                                                       dv_eff, x["ve"].astype(np.float64))
    dgate = torch.from_numpy(dg_ref.astype(np.float32)).cuda()
    dWg, dx32 = sw.ve_gate_v_bwd(xg, Wg, gate, dgate)
    assert rel_l2(host(dWg), dWg_ref) <= 1e-4
    check("dx32", host(dx32), dx_ref, "bf16")
    # bitwise repeatable reduction
    dWg2, _ = sw.ve_gate_v_bwd(xg, Wg, gate, dgate)
    assert torch.equal(dWg, dWg2)


def test_abi_errors_on_gpu_tensors():
    q = torch.zeros(1, 16, 1, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sw.SwaError) as e:
        sw.swa_fwd(q, q, q, 4)
    assert e.value.status == 2
