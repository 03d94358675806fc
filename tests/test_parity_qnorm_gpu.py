"""GPU tests of the query half of the prologue run inside the attention kernels.

swa_fwd_qnorm normalises each workgroup's raw query rows (RoPE, then RMS norm) before its key
loop; swa_bwd_dq_ds_qnorm applies the prologue's backward to its dq_hat rows before storing dq;
rope_qknorm_fwd / rope_qknorm_bwd then run on k only. Both fused kernels use the prologue
kernels' row arithmetic in the same lane layout, so every output must equal the separate calls
bit for bit: q_hat, O, lse, dq (and the k-only prologue's k_hat, dk). Cases: ragged and
single-row sequences, both head dims, windows below and above T, the fused gate, document
masking and the full-size layers the benchmark times; one end-to-end layer against the oracle.
"""

import numpy as np
import pytest
import torch

from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import WORKLOADS, make_inputs, small_workload
from gpu_helpers import announce, compare_layer, dev, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


def _equal(name, a, b):
    assert a.shape == b.shape and a.dtype == b.dtype, name
    diff = int((a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32) !=
                b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)).sum())
    assert diff == 0, f"{name}: {diff} elements differ"


def _both_routes(wl, window, gate=False):
    x = make_inputs(wl)
    q, k, v, dO = (dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
    cs = sw.rope_table(wl.T, wl.D, wl.base)
    ve = fgate = ids = bounds = None
    if gate:
        ve = dev(x["ve"], "bf16")
        fgate = sw.ve_gate_v(dev(x["x"], "bf16"), torch.from_numpy(x["Wg"]).cuda())
    if "doc_id" in x:
        bounds = sw.swa_doc_bounds(torch.from_numpy(x["doc_id"].astype(np.int32)).cuda())
    # separate prologue calls
    qn, kn = sw.rope_qknorm_fwd(q, k, cs, wl.eps)
    o, lse = sw.swa_fwd(qn, kn, v, window, wl.scale, ve=ve, gate=fgate, doc_bounds=bounds)
    ws = torch.empty(sw.swa_bwd_ds_workspace_size(wl.B, wl.T, wl.H, wl.D, window, q.dtype),
                     dtype=torch.uint8, device="cuda")
    grads = sw.swa_bwd_ds(qn, kn, v, o, lse, dO, window, wl.scale, ve=ve, gate=fgate,
                          doc_bounds=bounds, workspace=ws, stages=True)
    dq, dk = sw.rope_qknorm_bwd(q, k, cs, grads[0], grads[1], wl.eps)
    # fused: the query half inside the attention kernels, the prologue calls on k only
    kn2 = sw.rope_qknorm_fwd(None, k, cs, wl.eps)[1]
    qn2, o2, lse2 = sw.swa_fwd_qnorm(q, cs, kn2, v, window, wl.scale, eps=wl.eps, ve=ve,
                                     gate=fgate, doc_bounds=bounds)
    dq2 = sw.swa_bwd_dq_ds_qnorm(kn2, q, cs, ws, window, wl.scale, eps=wl.eps, doc_bounds=bounds)
    dk2 = sw.rope_qknorm_bwd(None, k, cs, None, grads[1], wl.eps)[1]
    torch.cuda.synchronize()
    for name, a, b in (("k_hat", kn2, kn), ("q_hat", qn2, qn), ("O", o2, o), ("lse", lse2, lse),
                       ("dq", dq2, dq), ("dk", dk2, dk)):
        _equal(name, a, b)


CASES = [(1, 1, 64), (17, 5, 128), (129, 64, 64), (129, 129, 128), (300, 100, 128),
         (300, 400, 64), (700, 256, 128)]


@pytest.mark.parametrize("T,W,D", CASES)
def test_qnorm_equals_separate_prologue(T, W, D):
    announce("qnorm bitwise", T, W, D)
    _both_routes(small_workload(2, T, 3, D, W, "bf16", seed=1300 + T + W + D), W)


@pytest.mark.parametrize("T,W,D", [(130, 64, 128), (257, 257, 64)])
def test_qnorm_with_fused_gate(T, W, D):
    announce("qnorm gate", T, W, D)
    _both_routes(small_workload(2, T, 2, D, W, "bf16", seed=1400 + T, gate=True, C=64), W,
                 gate=True)


@pytest.mark.parametrize("T,W,D,mean", [(300, 100, 128, 40), (700, 256, 64, 90)])
def test_qnorm_document_masking(T, W, D, mean):
    announce("qnorm doc", T, W, D, mean)
    _both_routes(small_workload(2, T, 2, D, W, "bf16", seed=1500 + T, doc_mean=mean), W)


@pytest.mark.parametrize("name", ["d24_short", "d24_full", "gpt2_124m"])
def test_qnorm_full_size(name):
    """The full layers in the launch configuration the benchmark times, whole tensors."""
    wl = WORKLOADS[name]
    announce("qnorm full size", name)
    _both_routes(wl, wl.window)


@pytest.mark.parametrize("gate", [False, True])
def test_qnorm_layer_against_oracle(gate):
    announce("qnorm e2e", gate)
    wl = small_workload(2, 200, 3, 128, 77, "bf16", seed=1600, gate=gate, C=96)
    x = make_inputs(wl)
    g = gpu_layer(x, wl, 77, fused_gate=False, bwd="ds", qnorm=True)
    fwd, bwd = oracle_layer(x, wl, 77)
    compare_layer(g, fwd, bwd, "bf16", gate=gate)
