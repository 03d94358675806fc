"""GPU parity of the value-embedding table mode against the oracle, through the C ABI: the
kernels gather each token's row of a (rows, H*D) table by token id inside their V loads, and the
backward adds gate * dv_eff of every token into the float table gradient row of its id. Cases
cover heavily repeated ids (a small vocabulary, so many tokens share a row), ids outside the
table (a zero row, no gradient), both head dims and both dtypes, the staged backward, and the
agreement with the per-token mode on the same rows."""

import numpy as np
import pytest
import torch

from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
from gpu_helpers import announce, compare_layer, dev, gpu_layer, host, oracle_layer

pytestmark = pytest.mark.gpu


def _inputs(B, T, H, D, W, dtype, seed, vocab, bad=()):
    wl = small_workload(B, T, H, D, W, dtype, seed, gate=True, ve_table=True, vocab=vocab)
    x = make_inputs(wl)
    for (b, t), val in bad:          # ids outside [0, vocab): zero value embedding
        x["ids"][b, t] = val
    return wl, x


CASES = [  # B, T, H, D, W, dtype, vocab
    (2, 300, 2, 128, 100, "bf16", 37),
    (2, 260, 3, 64, 64, "bf16", 5),       # five rows shared by 520 tokens
    (1, 200, 2, 128, 200, "bf16", 1000),
    (2, 150, 2, 64, 40, "f32", 11),
    (1, 130, 2, 128, 130, "f32", 3),
]


@pytest.mark.parametrize("B,T,H,D,W,dtype,vocab", CASES)
def test_vetable_layer(B, T, H, D, W, dtype, vocab):
    announce("ve table layer", B, T, H, D, W, dtype, vocab)
    bad = (((0, 5), -1), ((B - 1, T - 1), vocab), ((0, T // 2), 1 << 30))
    wl, x = _inputs(B, T, H, D, W, dtype, seed=B * 1000 + T + vocab, vocab=vocab, bad=bad)
    g = gpu_layer(x, wl, W)
    fwd, bwd = oracle_layer(x, wl, W)
    compare_layer(g, fwd, bwd, dtype, gate=True)
    dt = host(g["dve"])
    assert dt.shape == (vocab, H * D)
    unused = np.setdiff1d(np.arange(vocab), x["ids"])
    assert np.all(dt[unused] == 0.0)          # rows no token uses get no gradient


def test_vetable_matches_per_token_mode():
    """Table mode and per-token mode on the gathered rows give the same O, lse and dq, dk, dv,
    dgate bit for bit; the table gradient equals the per-token dve summed by id."""
    B, T, H, D, W, vocab = 2, 320, 2, 128, 128, 23
    announce("ve table vs per-token", B, T, H, D, W)
    wl, x = _inputs(B, T, H, D, W, "bf16", seed=77, vocab=vocab)
    q, k, v, dO = (dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
    table = dev(x["table"], "bf16")
    ids = torch.from_numpy(x["ids"]).cuda()
    ve = table[ids.long()].contiguous()
    gate = sw.ve_gate_v(dev(x["x"], "bf16"), torch.from_numpy(x["Wg"]).cuda())
    o1, l1 = sw.swa_fwd(q, k, v, W, ve=ve, gate=gate)
    o2, l2 = sw.swa_fwd(q, k, v, W, ve=table, gate=gate, ve_ids=ids)
    g1 = sw.swa_bwd(q, k, v, o1, l1, dO, W, ve=ve, gate=gate)
    g2 = sw.swa_bwd_stages(q, k, v, o2, l2, dO, W, ve=table, gate=gate, ve_ids=ids)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1[:3] + (g1[4],), g2[:3] + (g2[4],)):
        assert torch.equal(a, b)
    want = torch.zeros((vocab, H * D), dtype=torch.float32, device="cuda")
    want.index_add_(0, ids.reshape(-1).long(), g1[3].float().reshape(B * T, H * D))
    # per-token dve is rounded to bf16, the table gradient adds the float values
    err = (g2[3] - want).norm() / want.norm()
    assert err.item() <= 1e-2, err.item()


def test_vetable_gradient_accumulates():
    """A second backward adds into the same table gradient: the result is twice the first, up
    to the order of the float atomics."""
    B, T, H, D, W, vocab = 1, 256, 2, 64, 100, 9
    announce("ve table accumulation")
    wl, x = _inputs(B, T, H, D, W, "bf16", seed=5, vocab=vocab)
    q, k, v, dO = (dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
    table = dev(x["table"], "bf16")
    ids = torch.from_numpy(x["ids"]).cuda()
    gate = sw.ve_gate_v(dev(x["x"], "bf16"), torch.from_numpy(x["Wg"]).cuda())
    o, lse = sw.swa_fwd(q, k, v, W, ve=table, gate=gate, ve_ids=ids)
    g1 = sw.swa_bwd(q, k, v, o, lse, dO, W, ve=table, gate=gate, ve_ids=ids)
    first = g1[3].clone()
    sw.swa_bwd(q, k, v, o, lse, dO, W, ve=table, gate=gate, ve_ids=ids, grads=g1)
    torch.cuda.synchronize()
    torch.testing.assert_close(g1[3], 2 * first, rtol=1e-5, atol=1e-5)
