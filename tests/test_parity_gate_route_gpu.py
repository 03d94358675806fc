"""GPU parity of the materialised value-embedding route against the oracle, through the C ABI:
ve_gate_v writes v_eff = v + gate * ve (per-token rows or table rows by token id), the attention
kernels run on v_eff without the gate, and ve_gate_dv turns dv_eff into dve (or the table's
gradient) and dgate. Also checks that this route and the fused one agree."""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
from gpu_helpers import announce, check, compare_layer, dev, gpu_layer, host, oracle_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("table", [False, True])
def test_gate_dv_against_oracle(dtype, D, table):
    B, T, H, vocab = 2, 97, 3, 13
    announce("ve_gate_dv", dtype, D, table)
    wl = small_workload(B, T, H, D, T, dtype, seed=D + 7 * table, gate=True, ve_table=table,
                        vocab=vocab)
    x = make_inputs(wl)
    rng = np.random.default_rng(3)
    dv_eff = rng.standard_normal((B, T, H, D))
    if dtype == "bf16":
        dv_eff = oracle.round_bf16(dv_eff)
    gate = torch.from_numpy((0.5 + rng.random((B, T, H))).astype(np.float32)).cuda()
    g = host(gate)
    if table:
        x["ids"][0, 3], x["ids"][1, 50] = -2, vocab   # outside the table: zero row, no gradient
        ve_host = oracle.ve_lookup(x["table"].astype(np.float64), x["ids"])
        ve_t = dev(x["table"], dtype)
        ids = torch.from_numpy(x["ids"]).cuda()
    else:
        ve_host = x["ve"].astype(np.float64)
        ve_t, ids = dev(x["ve"], dtype), None
    dve, dgate = sw.ve_gate_dv(dev(dv_eff, dtype), ve_t, gate, ve_ids=ids)
    torch.cuda.synchronize()
    x32 = np.zeros((B, T, 32))
    _, dve_ref, dg_ref, _, _ = oracle.ve_gate_bwd(x32, np.zeros((32, H)), g, dv_eff, ve_host)
    check("dgate", host(dgate), dg_ref, dtype, sum_scaled=True)
    if table:
        check("dtable", host(dve), oracle.ve_table_grad(dve_ref, x["ids"], vocab), dtype,
              sum_scaled=True)
    else:
        check("dve", host(dve), dve_ref, dtype)


def test_materialise_table_rows():
    """ve_gate_v in the table mode writes v + gate * table[id] (zero row for a bad id)."""
    B, T, H, D, vocab = 2, 64, 2, 128, 7
    announce("ve_gate_v table rows")
    wl = small_workload(B, T, H, D, T, "bf16", seed=12, gate=True, C=40, ve_table=True,
                        vocab=vocab)
    x = make_inputs(wl)
    x["ids"][1, 9] = 1 << 20
    gate, v_eff = sw.ve_gate_v(dev(x["x"], "bf16"), torch.from_numpy(x["Wg"]).cuda(),
                               dev(x["v"], "bf16"), dev(x["table"], "bf16"), materialize=True,
                               ve_ids=torch.from_numpy(x["ids"]).cuda())
    torch.cuda.synchronize()
    ve = oracle.ve_lookup(x["table"].astype(np.float64), x["ids"])
    want = oracle.apply_gate(x["v"].astype(np.float64), host(gate), ve)
    check("v_eff", host(v_eff), want, "bf16")
    np.testing.assert_array_equal(host(v_eff)[1, 9], x["v"][1, 9])   # zero row: v_eff = v


LAYERS = [  # B, T, H, D, W, dtype, table, vocab
    (2, 300, 2, 128, 100, "bf16", False, 0),
    (2, 300, 2, 128, 100, "bf16", True, 29),
    (2, 200, 3, 64, 64, "bf16", True, 6),
    (1, 160, 2, 64, 160, "f32", False, 0),
    (2, 130, 2, 128, 50, "f32", True, 9),
]


@pytest.mark.parametrize("B,T,H,D,W,dtype,table,vocab", LAYERS)
def test_materialised_route_layer(B, T, H, D, W, dtype, table, vocab):
    announce("materialised gate layer", B, T, H, D, W, dtype, table)
    kw = dict(ve_table=True, vocab=vocab) if table else {}
    wl = small_workload(B, T, H, D, W, dtype, seed=T + vocab, gate=True, **kw)
    x = make_inputs(wl)
    if table:
        x["ids"][0, 1] = -1
    g = gpu_layer(x, wl, W, fused_gate=False)
    fwd, bwd = oracle_layer(x, wl, W)
    compare_layer(g, fwd, bwd, dtype, gate=True)


def test_routes_agree():
    """Both routes round v_eff to bf16 the same way, so the attention outputs and dq, dk, dv are
    bit-identical; dve and dgate differ only by where dv_eff is rounded."""
    B, T, H, D, W = 2, 256, 2, 128, 96
    announce("gate routes agree")
    wl = small_workload(B, T, H, D, W, "bf16", seed=4, gate=True)
    x = make_inputs(wl)
    a = gpu_layer(x, wl, W, fused_gate=True)
    b = gpu_layer(x, wl, W, fused_gate=False)
    for n in ("O", "lse", "dqh", "dkh", "dv", "dq", "dk", "gate"):
        assert torch.equal(a[n], b[n]), n
    for n in ("dve", "dgate"):
        assert check(n, host(b[n]), host(a[n]), "bf16") <= 1e-2
