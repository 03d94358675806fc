"""HIP-graph capture of the path: the entry points allocate nothing, clear nothing and never
synchronise, so a whole training layer (prologue, attention forward, backward, prologue
backward) and a decoding step (prologue into the ring cache, attention over the window) can be
captured once and replayed. Every replay is compared bitwise with the same work run eagerly
(the kernels are deterministic), with eager work of the program between the replays, and the
replayed layer is also held to the oracle's bars.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_sliding_window_rope_amd import binding as sw
from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
from gpu_helpers import announce, check, host

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm fn up on a side stream (default priority), then capture it; returns (graph, outs)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    return g, outs


def test_layer_graph_replay_matches_eager_and_oracle():
    wl = small_workload(2, 300, 3, 128, 100, "bf16", seed=17)
    announce("graph replay: layer", wl.name)
    x = make_inputs(wl)
    t = {n: torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v", "dO")}
    cs = sw.rope_table(wl.T, wl.D, wl.base)

    def layer():
        qn, kn = sw.rope_qknorm_fwd(t["q"], t["k"], cs, wl.eps)
        o, lse = sw.swa_fwd(qn, kn, t["v"], wl.window, wl.scale)
        dqn, dkn, dv = sw.swa_bwd(qn, kn, t["v"], o, lse, t["dO"], wl.window, wl.scale)
        dq, dk = sw.rope_qknorm_bwd(t["q"], t["k"], cs, dqn, dkn, wl.eps)
        return o, lse, dq, dk, dv

    eager = [a.clone() for a in layer()]
    torch.cuda.synchronize()
    g, outs = _capture(layer)
    for rep in range(3):
        for a in outs:
            a.fill_(float("nan"))   # a replay must rewrite every output
        (t["q"].float() * 2).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "lse", "dq", "dk", "dv"), outs, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"

    f = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "dO")}
    fwd = oracle.layer_fwd(f["q"], f["k"], f["v"], wl.window, base=wl.base, eps=wl.eps,
                           round_boundary=True)
    bwd = oracle.layer_bwd(f["q"], f["k"], f["v"], f["dO"], wl.window, fwd, base=wl.base,
                           eps=wl.eps)
    o, lse, dq, dk, dv = (host(a) for a in outs)
    check("O", o, fwd["O"], "bf16")
    check("lse", lse, fwd["lse"], "bf16", lse=True)
    check("dq", dq, bwd["dq"], "bf16")
    check("dk", dk, bwd["dk"], "bf16")
    check("dv", dv, bwd["dv"], "bf16")


def test_stored_ds_layer_graph_replay_matches_eager():
    """The benchmarked route: the prologue on k alone, the forward with the query prologue
    inside, the stored-dS backward (row terms, dK/dV storing dS, dQ with the query prologue's
    backward) on one workspace, the prologue backward on k alone. The workspace is filled with
    NaN bit patterns before each replay: chunks that are never written must never be read."""
    wl = small_workload(2, 300, 3, 128, 100, "bf16", seed=19)
    announce("graph replay: stored-dS layer", wl.name)
    x = make_inputs(wl)
    t = {n: torch.from_numpy(x[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v", "dO")}
    cs = sw.rope_table(wl.T, wl.D, wl.base)
    ws = torch.empty(sw.swa_bwd_ds_workspace_size(wl.B, wl.T, wl.H, wl.D, wl.window,
                                                  torch.bfloat16), dtype=torch.uint8,
                     device="cuda")

    def layer():
        kn = sw.rope_qknorm_fwd(None, t["k"], cs, wl.eps)[1]
        qn, o, lse = sw.swa_fwd_qnorm(t["q"], cs, kn, t["v"], wl.window, wl.scale, eps=wl.eps)
        _, dkn, dv = sw.swa_bwd_ds(qn, kn, t["v"], o, lse, t["dO"], wl.window, wl.scale,
                                   workspace=ws, stages=True)
        dq = sw.swa_bwd_dq_ds_qnorm(kn, t["q"], cs, ws, wl.window, wl.scale, eps=wl.eps)
        dk = sw.rope_qknorm_bwd(None, t["k"], cs, None, dkn, wl.eps)[1]
        return o, lse, dq, dk, dv

    eager = [a.clone() for a in layer()]
    torch.cuda.synchronize()
    g, outs = _capture(layer)
    for rep in range(3):
        for a in outs:
            a.fill_(float("nan"))
        ws.view(torch.float32).fill_(float("nan"))
        (t["q"].float() * 2).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "lse", "dq", "dk", "dv"), outs, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"

    f = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "dO")}
    fwd = oracle.layer_fwd(f["q"], f["k"], f["v"], wl.window, base=wl.base, eps=wl.eps,
                           round_boundary=True)
    bwd = oracle.layer_bwd(f["q"], f["k"], f["v"], f["dO"], wl.window, fwd, base=wl.base,
                           eps=wl.eps)
    o, lse, dq, dk, dv = (host(a) for a in outs)
    check("O", o, fwd["O"], "bf16")
    check("lse", lse, fwd["lse"], "bf16", lse=True)
    check("dq", dq, bwd["dq"], "bf16")
    check("dk", dk, bwd["dk"], "bf16")
    check("dv", dv, bwd["dv"], "bf16")


def test_decode_step_graph_replay_matches_eager():
    """A decoding step captured once; between replays the program writes the next token's
    q, k, v into the captured input buffers and advances the positions on the device. The
    positions cross the end of the ring (slot p mod C)."""
    B, H, D, cap, W, steps = 4, 12, 128, 256, 128, 5
    announce("graph replay: decode step")
    g0 = torch.Generator(device="cuda")
    g0.manual_seed(23)
    rnd = lambda *s: torch.randn(s, generator=g0, device="cuda").to(torch.bfloat16)
    Q, K, V = rnd(steps, B, H, D), rnd(steps, B, H, D), rnd(steps, B, H, D)
    start = torch.tensor([130, 200, 5, 253], dtype=torch.int32, device="cuda")
    cs = sw.rope_table(2 * cap, D, 10000.0)
    # both caches start from the same history
    kc_e = rnd(B, cap, H, D)
    vc_e = rnd(B, cap, H, D)
    kc_g, vc_g = kc_e.clone(), vc_e.clone()

    pos_e = start.clone()
    eager = []
    for i in range(steps):
        qn = sw.swa_decode_prologue(Q[i], K[i], V[i], cs, pos_e, kc_e, vc_e)
        o, lse = sw.swa_decode(qn, kc_e, vc_e, pos_e, W)
        eager.append((o.clone(), lse.clone()))
        pos_e.add_(1)
    torch.cuda.synchronize()

    xq, xk, xv = Q[0].clone(), K[0].clone(), V[0].clone()
    pos_g = start.clone()

    def step():
        qn = sw.swa_decode_prologue(xq, xk, xv, cs, pos_g, kc_g, vc_g)
        return sw.swa_decode(qn, kc_g, vc_g, pos_g, W)

    g, (o_g, lse_g) = _capture(step)   # the warm-up wrote step 0's k, v: replay 0 rewrites them
    for i in range(steps):
        xq.copy_(Q[i])
        xk.copy_(K[i])
        xv.copy_(V[i])
        o_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, eager[i][0]), f"step {i}: o differs from the eager run"
        assert torch.equal(lse_g, eager[i][1]), f"step {i}: lse differs from the eager run"
        pos_g.add_(1)
    torch.cuda.synchronize()
    assert torch.equal(kc_g, kc_e) and torch.equal(vc_g, vc_e)
