"""Full-size parity of the gated value-embedding layer on the route the benchmark times.

The d24 short layer with the value-embedding gate (B=16, T=2048, H=12, D=128, window 1024,
x of width 1536, ve rows from a 50304 x 1536 table; "3. Value Embeddings" on the
lanjinlin.com.cn repost: v = v + gate * ve with gate = 2 sigmoid(ve_gate(x[:, :, :32]))) runs
the materialised route: ve_gate_v writes v_eff, the attention runs on v_eff, ve_gate_dv turns
dv_eff into dve and dgate, ve_gate_v_bwd reduces dWg over all B*T = 32768 rows (256 chunks of
128 rows) and writes dx32. Every output is compared with the oracle over all 192 heads.
A second case reads the value embedding from the full 50304-row table by token id.
"""

import numpy as np
import pytest
import torch

from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import WORKLOADS, Workload, make_inputs
from gpu_helpers import announce, check, compare_layer, gpu_layer, host, oracle_layer, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.load()


def _run(wl):
    x = make_inputs(wl)
    g = gpu_layer(x, wl, wl.window, fused_gate=False)
    fwd, bwd = oracle_layer(x, wl, wl.window)
    errs = compare_layer(g, fwd, bwd, "bf16", gate=True)
    errs["dWg"] = rel_l2(host(g["dWg"]), bwd["dWg"])
    assert errs["dWg"] <= 1e-2, errs["dWg"]
    errs["dx32"] = check("dx32", host(g["dx32"]), bwd["dx32"], "bf16")
    print(wl.name, {k: f"{v:.2e}" for k, v in errs.items()})
    return errs


def test_d24_short_ve_materialised_all_heads():
    wl = WORKLOADS["d24_short_ve"]
    announce("full size gated, materialised route, all heads", wl.name)
    _run(wl)


def test_ve_table_full_vocabulary():
    """Table mode with the full 50304-row table (B = 4 sequences of the d24 shape: 8192 rows,
    64 chunks of the dWg reduction)."""
    base = WORKLOADS["d24_short_vetable"]
    wl = Workload("d24_vetable_b4", B=4, T=base.T, H=base.H, D=base.D, window=base.window,
                  dtype="bf16", seed=base.seed, gate=True, C=base.C, ve_table=True)
    assert wl.vocab == 50304
    announce("full vocabulary table mode", wl.name)
    _run(wl)
