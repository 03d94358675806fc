#!/usr/bin/env python3
"""Throughput of the attention core (forward + backward) on one MI355X.

One step = the attention of every layer of the nanochat d24 model, forward then backward,
as in a training step: for layers 0..23 rope_qknorm_fwd + swa_fwd, then for layers 23..0
swa_bwd (dQ with the row terms, then dK/dV) + rope_qknorm_bwd. Windows follow the 3-short:1-long
tiling (layers 3, 7, ... full 2048, the rest 1024); B=16 sequences of T=2048, H=12, D=128,
bf16 storage, fp32 accumulation. Inputs are synthetic N(0, 1) tensors drawn on the device
from a seeded generator, one set per layer (kernel time does not depend on the values).

The metric counts algorithmic MFMA FLOPs only over visible (query, key) pairs: 4*D per pair
forward, 10*D per pair backward (the five contractions of the recomputing backward).

Prints one JSON line. --gpus above 1 is refused: the benchmark measures one GPU (sharded
over the batch, attention needs no exchange between GPUs).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (unmasked FLOPs) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA: twice the bf16 rate
FP8_METRIC = "attention forward TFLOP/s on fp8 operands (unmasked FLOPs) and % of MI355X fp8 MFMA peak"


def pairs(T: int, W: int) -> int:
    W = min(W, T)
    return W * (W + 1) // 2 + (T - W) * W


def layer_list(name: str):
    from causal_sliding_window_rope_amd.inputs import WORKLOADS, sssl_windows
    if name == "sssl24":
        return dict(B=16, T=2048, H=12, D=128, gate=False,
                    windows=sssl_windows(24, 1024, 2048),
                    desc="d24 attention sweep: 24 layers, 3-short:1-long windows "
                         "(18 x 1024, 6 x 2048), B=16, T=2048, H=12, D=128")
    wl = WORKLOADS[name]
    return dict(B=wl.B, T=wl.T, H=wl.H, D=wl.D, gate=wl.gate, windows=[wl.window],
                doc_mean=wl.doc_mean, seed=wl.seed, ve_table=wl.ve_table,
                desc=f"{name}: B={wl.B}, T={wl.T}, H={wl.H}, D={wl.D}, window {wl.window}"
                     + (", value-embedding gate" if wl.gate else "")
                     + (" reading the (50304, H*D) table by token id" if wl.ve_table else "")
                     + (f", packed rows of documents averaging {wl.doc_mean} tokens"
                        if wl.doc_mean else ""))


def doc_starts(cfg):
    """(B, T) start of each token's document for document-masked workloads, else None."""
    import numpy as np
    from causal_sliding_window_rope_amd.inputs import doc_layout
    if not cfg.get("doc_mean"):
        return None, None
    ids = doc_layout(np.random.default_rng(cfg["seed"]), cfg["B"], cfg["T"], cfg["doc_mean"])
    starts = np.zeros_like(ids)
    for b in range(ids.shape[0]):
        change = np.ones(ids.shape[1], dtype=bool)
        change[1:] = ids[b, 1:] != ids[b, :-1]
        pos = np.where(change, np.arange(ids.shape[1]), 0)
        starts[b] = np.maximum.accumulate(pos)
    return ids, starts


def visible_pairs(cfg, W, starts):
    """Visible (query, key) pairs per head summed over the batch."""
    import numpy as np
    B, T = cfg["B"], cfg["T"]
    if starts is None:
        return pairs(T, W) * B
    i = np.arange(T)[None, :]
    return int(np.minimum(i - starts + 1, W).sum())


def make_layers(cfg, torch, seed0=1000):
    """Per-layer device tensors (inputs + forward outputs kept for the backward)."""
    B, T, H, D = cfg["B"], cfg["T"], cfg["H"], cfg["D"]
    layers = []
    for l, W in enumerate(cfg["windows"]):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed0 + l)
        t = {n: torch.randn((B, T, H, D), generator=g, device="cuda", dtype=torch.float32)
             .to(torch.bfloat16) for n in ("q", "k", "v", "dO")}
        t["qn"], t["kn"] = torch.empty_like(t["q"]), torch.empty_like(t["k"])
        t["o"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        if cfg["gate"]:
            t["x"] = torch.randn((B, T, 1536), generator=g, device="cuda").to(torch.bfloat16)
            t["Wg"] = torch.randn((32, H), generator=g, device="cuda") * 0.02
            table = torch.randn((50304, H * D), generator=g, device="cuda").to(torch.bfloat16)
            ids = torch.randint(0, 50304, (B, T), generator=g, device="cuda")
            if cfg.get("ve_table"):
                t["ve"], t["ids"] = table, ids.to(torch.int32)
            else:
                t["ve"] = table[ids].contiguous()
            del table
            t["gate"] = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
            t["veff"] = torch.empty_like(t["v"])   # materialised v + gate * ve, kept for the bwd
        t["W"] = W
        layers.append(t)
    return layers


def run_bench(args):
    import torch
    from causal_sliding_window_rope_amd import binding as sw

    sw.load()  # raises if the HIP library is missing: there is no other path
    cfg = layer_list(args.workload)
    B, T, H, D = cfg["B"], cfg["T"], cfg["H"], cfg["D"]
    scale = D ** -0.5
    layers = make_layers(cfg, torch)
    doc_ids, starts = doc_starts(cfg)
    if doc_ids is not None:
        # one document layout per batch, shared by every layer (as in a training step)
        bounds_t = sw.swa_doc_bounds(torch.from_numpy(doc_ids).cuda())
        for t in layers:
            t["bounds"] = bounds_t
    cs = sw.rope_table(T, D, 10000.0)
    # gradient buffers shared by all layers
    g = {n: torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
         for n in ("dqn", "dkn", "dv", "dq", "dk")}
    if cfg.get("ve_table"):
        # the table gradient is accumulated into (zeroed once; steps keep adding to it)
        g["dve"] = torch.zeros((50304, H * D), dtype=torch.float32, device="cuda")
        g["dgate"] = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
        g["dWg"] = torch.empty((32, H), dtype=torch.float32, device="cuda")
    elif cfg["gate"]:
        g["dve"] = torch.empty((B, T, H * D), dtype=torch.bfloat16, device="cuda")
        g["dgate"] = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
        g["dWg"] = torch.empty((32, H), dtype=torch.float32, device="cuda")
    stored_ds = args.bwd == "ds"
    # one workspace serves every layer (sized for the widest window)
    ws_bytes = (sw.swa_bwd_ds_workspace_size(B, T, H, D, max(cfg["windows"]), torch.bfloat16)
                if stored_ds else sw.swa_bwd_workspace_size(B, T, H, D, torch.bfloat16))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    if cfg["gate"]:
        g["gws"] = torch.empty(sw.load().ve_gate_v_bwd_workspace_size(B, T, H), dtype=torch.uint8,
                               device="cuda")
    lib = sw.load()
    P = sw._ptr
    nws = ws.numel()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def call(name, *a):
        st = getattr(lib, name)(*a)
        if st != 0:
            raise sw.SwaError(name, st, lib.swa_last_error().decode())

    fused_gate = args.fused_gate
    # the query half of the prologue inside swa_fwd_qnorm and / or its backward inside
    # swa_bwd_dq_ds_qnorm (stored-dS backward only); the prologue calls then run on k alone for
    # that half. By default both (measured fastest or level on the d24 sweep and the GPT-2
    # layer).
    mode = "off" if args.no_qnorm else args.qnorm
    if mode == "auto":
        mode = "on"
    qn_fwd = stored_ds and mode in ("on", "fwd")   # the forward half inside swa_fwd_qnorm
    qn_bwd = stored_ds and mode in ("on", "bwd")   # its backward inside swa_bwd_dq_ds_qnorm

    def step(rec):
        stream = sw._stream()   # the current stream: the capture stream when recording a graph
        # forward, layers in order
        for li, t in enumerate(layers):
            bounds, ids = t.get("bounds"), t.get("ids")
            rows = 0 if ids is None else t["ve"].shape[0]
            call("rope_qknorm_fwd", None if qn_fwd else P(t["q"]), P(t["k"]), P(cs),
                 None if qn_fwd else P(t["qn"]), P(t["kn"]), B, T, H, D, 1e-6, sw.SWA_BF16, stream)
            ve = gate = fids = None
            frows, v = 0, t["v"]
            if cfg["gate"] and fused_gate:
                call("ve_gate_v", P(t["x"]), 1536, P(t["Wg"]), P(t["gate"]), None, None, None, 0,
                     None, B, T, H, D, sw.SWA_BF16, stream)
                ve, gate, fids, frows = t["ve"], t["gate"], ids, rows
            elif cfg["gate"]:
                call("ve_gate_v", P(t["x"]), 1536, P(t["Wg"]), P(t["gate"]), P(t["v"]), P(t["ve"]),
                     P(ids), rows, P(t["veff"]), B, T, H, D, sw.SWA_BF16, stream)
                v = t["veff"]
            if rec: rec["fwd"][li][0].record()
            if qn_fwd:
                call("swa_fwd_qnorm", P(t["q"]), P(cs), 1e-6, P(t["kn"]), P(v), P(ve), P(gate),
                     P(fids), frows, P(bounds), P(t["qn"]), P(t["o"]), P(t["lse"]),
                     B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
            else:
                call("swa_fwd", P(t["qn"]), P(t["kn"]), P(v), P(ve), P(gate), P(fids), frows,
                     P(bounds), P(t["o"]), P(t["lse"]),
                     B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
            if rec: rec["fwd"][li][1].record()
        # backward, layers in reverse
        for li in reversed(range(len(layers))):
            t = layers[li]
            bounds, ids = t.get("bounds"), t.get("ids")
            rows = 0 if ids is None else t["ve"].shape[0]
            ve = gate = dve = dgate = fids = None
            frows, v = 0, t["v"]
            if cfg["gate"] and fused_gate:
                ve, gate, dve, dgate = t["ve"], t["gate"], g["dve"], g["dgate"]
                fids, frows = ids, rows
            elif cfg["gate"]:
                v = t["veff"]
            if stored_ds:
                # row terms (delta, lse), then dK/dV storing the bf16 dS it forms, then dQ from
                # the stored dS
                if rec: rec["bwd"][li][0].record()
                call("swa_bwd_preprocess", P(t["o"]), P(t["dO"]), P(t["lse"]), P(ws), nws,
                     B, T, H, D, sw.SWA_BF16, stream)
                if rec: rec["bwd"][li][1].record()
                call("swa_bwd_dkdv_ds", P(t["qn"]), P(t["kn"]), P(v), P(ve), P(gate), P(fids),
                     frows, P(bounds), P(t["lse"]), P(t["dO"]), P(g["dkn"]), P(g["dv"]), P(dve),
                     P(dgate), P(ws), nws, B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
                if rec: rec["bwd"][li][2].record()
                if qn_bwd:   # dq w.r.t. the raw q straight from the dQ kernel
                    call("swa_bwd_dq_ds_qnorm", P(t["kn"]), P(bounds), P(t["q"]), P(cs), 1e-6,
                         P(g["dq"]), P(ws), nws, B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
                else:
                    call("swa_bwd_dq_ds", P(t["kn"]), P(bounds), P(g["dqn"]), P(ws), nws,
                         B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
                if rec: rec["bwd"][li][3].record()
            else:
                # dQ first: its kernel also writes the row terms (delta, lse) that dK/dV reads
                if rec: rec["bwd"][li][0].record()
                if rec: rec["bwd"][li][1].record()
                call("swa_bwd_dq_rowterms", P(t["qn"]), P(t["kn"]), P(v), P(ve), P(gate), P(fids),
                     frows, P(bounds), P(t["o"]), P(t["lse"]), P(t["dO"]), P(g["dqn"]), P(ws),
                     nws, B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
                if rec: rec["bwd"][li][2].record()
                call("swa_bwd_dkdv", P(t["qn"]), P(t["kn"]), P(v), P(ve), P(gate), P(fids), frows,
                     P(bounds), P(t["lse"]),
                     P(t["dO"]), P(g["dkn"]), P(g["dv"]), P(dve), P(dgate), P(ws), nws,
                     B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
                if rec: rec["bwd"][li][3].record()
            call("rope_qknorm_bwd", None if qn_bwd else P(t["q"]), P(t["k"]), P(cs),
                 None if qn_bwd else P(g["dqn"]), P(g["dkn"]), None if qn_bwd else P(g["dq"]),
                 P(g["dk"]), B, T, H, D, 1e-6, sw.SWA_BF16, stream)
            if cfg["gate"]:
                if not fused_gate:   # dve, dgate from dv_eff (= dv)
                    call("ve_gate_dv", P(g["dv"]), P(t["ve"]), P(ids), rows, P(t["gate"]),
                         P(g["dve"]), P(g["dgate"]), B, T, H, D, sw.SWA_BF16, stream)
                call("ve_gate_v_bwd", P(t["x"]), 1536, P(t["Wg"]), P(t["gate"]), P(g["dgate"]),
                     P(g["dWg"]), None, P(g["gws"]), g["gws"].numel(), B, T, H, sw.SWA_BF16,
                     stream)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    nl = len(layers)
    recs = [{"fwd": [[ev(), ev()] for _ in range(nl)], "bwd": [[ev() for _ in range(4)] for _ in range(nl)]}
            for _ in range(args.steps)]
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()          # one GPU: no process group, so no barrier is needed
    t0 = time.perf_counter()
    e0.record()
    for k in range(args.steps):
        step(recs[k])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    eager_ms = step_ms
    if args.graph:
        # the whole step as one HIP graph, captured after the eager pass above (which supplies
        # the per-kernel times); value and ms_per_step are then the replay times
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(None)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        step_ms = e0.elapsed_time(e1) / args.steps

    fwd_ms = sum(r["fwd"][l][0].elapsed_time(r["fwd"][l][1]) for r in recs for l in range(nl))
    seg = lambda a, b: sum(r["bwd"][l][a].elapsed_time(r["bwd"][l][b]) for r in recs
                           for l in range(nl))
    if stored_ds:   # events: | preprocess | dK/dV (+ dS store) | dQ from dS |
        pre_ms, kv_ms, dq_ms = seg(0, 1), seg(1, 2), seg(2, 3)
    else:           # events: | | dQ with the row terms | dK/dV |
        pre_ms, dq_ms, kv_ms = seg(0, 1), seg(1, 2), seg(2, 3)
    launches = args.steps * nl

    npairs = sum(visible_pairs(cfg, W, starts) for W in cfg["windows"]) * H
    fwd_flop = 4 * D * npairs
    bwd_flop = 10 * D * npairs
    flop = fwd_flop + bwd_flop
    value = flop / (step_ms * 1e-3) / 1e12
    core_ms = (fwd_ms + pre_ms + kv_ms + dq_ms) / args.steps
    fwd_tf = fwd_flop / (fwd_ms / args.steps * 1e-3) / 1e12
    bwd_tf = bwd_flop / ((pre_ms + kv_ms + dq_ms) / args.steps * 1e-3) / 1e12
    # algorithmic FLOPs of each backward kernel: the dK/dV kernel recomputes S and dP and forms
    # dV, dK (8*D per pair); the dQ kernel forms dQ from the stored dS (2*D per pair), or, on the
    # recomputing path, recomputes S and dP once more (6*D per pair). The metric credits 10*D
    # per pair to the backward as a whole.
    kv_flop = 8 * D * npairs
    dq_flop = (2 if stored_ds else 6) * D * npairs

    # dominant kernel: the one with the largest share of the step
    kv_name = "dkdv_bf16_kernel (swa_bwd_dkdv_ds)" if stored_ds else "dkdv_bf16_kernel (swa_bwd_dkdv)"
    dq_name = "dq_ds_kernel (swa_bwd_dq_ds)" if stored_ds else "dq_bf16_kernel (swa_bwd_dq_rowterms)"
    cands = [(kv_name, kv_ms, kv_flop), ("fwd_bf16_kernel (swa_fwd)", fwd_ms, fwd_flop),
             (dq_name, dq_ms, dq_flop)]
    dom, dom_total_ms, dom_total_flop = max(cands, key=lambda x: x[1])
    dom_ms, dom_flop = dom_total_ms / launches, dom_total_flop / nl
    achieved = dom_flop / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "avg_launch_us": round(dom_ms * 1e3, 2),
                "traffic": traffic_from_profile(dom, args.workload)}
    if cfg["gate"]:
        cfg["desc"] += ("; gate fused into the attention kernels" if args.fused_gate
                        else "; v_eff materialised once per layer")
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["desc"], "global_batch": B, "seq_len": T, "heads": H,
                   "head_dim": D, "windows": sorted(set(cfg["windows"])),
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "breakdown": {
            "algorithmic_tflop_per_step": round(flop / 1e12, 4),
            "attention_core_ms_per_step": round(core_ms, 4),
            "attention_core_tflops": round(flop / (core_ms * 1e-3) / 1e12, 2),
            "attention_core_pct_of_peak": round(100 * flop / (core_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "prologue_and_gate_ms_per_step": round(eager_ms - core_ms, 4),
            "swa_fwd_tflops": round(fwd_tf, 2),
            "swa_bwd_tflops_credited": round(bwd_tf, 2),
            "backward": ("row terms, dK/dV storing dS, dQ from the stored dS" if stored_ds
                         else "dQ with the row terms, then dK/dV (S and dP recomputed twice)"),
            "query_prologue": {("on", "on"): "inside the forward and dQ kernels (their times "
                                              "include it)",
                               ("on", "off"): "forward inside the forward kernel, backward in "
                                              "the prologue call",
                               ("off", "on"): "forward in the prologue call, backward inside "
                                              "the dQ kernel",
                               ("off", "off"): "in the prologue calls"}[
                                   ("on" if qn_fwd else "off", "on" if qn_bwd else "off")],
            "swa_bwd_dkdv_tflops_executed": round(kv_flop / (kv_ms / args.steps * 1e-3) / 1e12, 2),
            "swa_bwd_dq_tflops_executed": round(dq_flop / (dq_ms / args.steps * 1e-3) / 1e12, 2),
            "swa_fwd_ms_per_step": round(fwd_ms / args.steps, 4),
            "swa_bwd_preprocess_ms_per_step": round(pre_ms / args.steps, 4),
            "swa_bwd_dkdv_ms_per_step": round(kv_ms / args.steps, 4),
            "swa_bwd_dq_ms_per_step": round(dq_ms / args.steps, 4),
            "wall_s_timed_region": round(wall, 3),
            "launch": "hip graph replay" if args.graph else "eager stream",
            "eager_ms_per_step": round(eager_ms, 4),
        },
        "roofline": roofline,
    }
    return result


# source files each timed kernel is compiled from (a change to any of them invalidates the
# committed counter figures for that kernel)
KERNEL_SOURCES = {
    "fwd_bf16_kernel": ("fwd.hip", "common.h", "rope_row.h"),
    "dkdv_bf16_kernel": ("bwd.hip", "common.h", "dsbuf.h"),
    "dq_bf16_kernel": ("dq.hip", "common.h"),
    "dq_ds_kernel": ("dqds.hip", "common.h", "dsbuf.h", "rope_row.h"),
}


def kernel_sources_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "causal_sliding_window_rope_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


DECODE_METRIC = "decode tokens/s (one new token per sequence through 24 sliding-window layers)"


def run_decode_bench(args):
    """Sliding-window decoding from a K/V cache: B = 32 sequences at position 2047 (full
    context) through the 24 d24 layers (windows 3-short:1-long), ring caches of 2048 slots per
    layer filled with synthetic N(0, 1) keys / values. One step = every layer's positional
    prologue (RoPE + QK-norm of the new q, k; k, v stored in the cache) and its windowed
    attention over the cache; tokens per step = B. The attention reads W cached K and V rows per
    (sequence, head), so it is priced against HBM bandwidth."""
    import torch
    from causal_sliding_window_rope_amd import binding as sw
    from causal_sliding_window_rope_amd.inputs import sssl_windows
    lib = sw.load()
    B, H, D, cap, p_pos = 32, 12, 128, 2048, 2047
    windows = sssl_windows(24, 1024, 2048)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    rnd = lambda *shape: torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    layers = []
    for W in windows:
        layers.append(dict(W=W, q=rnd(B, H, D), k=rnd(B, H, D), v=rnd(B, H, D),
                           kc=rnd(B, cap, H, D), vc=rnd(B, cap, H, D),
                           qn=torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda"),
                           o=torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda"),
                           lse=torch.empty((B, H), dtype=torch.float32, device="cuda")))
    cs = sw.rope_table(cap, D, 10000.0)
    pos = torch.full((B,), p_pos, dtype=torch.int32, device="cuda")
    nws = max(sw.swa_decode_workspace_size(B, H, D, cap, max(windows)), 256)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    P = sw._ptr
    scale = D ** -0.5
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def call(name, *a):
        st = getattr(lib, name)(*a)
        if st != 0:
            raise sw.SwaError(name, st, lib.swa_last_error().decode())

    def step(rec):
        st = sw._stream()   # the current stream: the capture stream when recording a graph
        for li, t in enumerate(layers):
            call("swa_decode_prologue", P(t["q"]), P(t["k"]), P(t["v"]), P(cs), cap, P(pos),
                 P(t["qn"]), P(t["kc"]), P(t["vc"]), B, H, D, cap, 1e-6, sw.SWA_BF16, st)
            if rec: rec[li][0].record()
            call("swa_decode", P(t["qn"]), P(t["kc"]), P(t["vc"]), P(pos), P(t["o"]), P(t["lse"]),
                 P(ws), nws, B, H, D, cap, t["W"], scale, sw.SWA_BF16, st)
            if rec: rec[li][1].record()

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = [[[ev(), ev()] for _ in layers] for _ in range(args.steps)]
    e0, e1 = ev(), ev()
    e0.record()
    for k in range(args.steps):
        step(recs[k])
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / args.steps
    dec_ms = sum(r[l][0].elapsed_time(r[l][1]) for r in recs for l in range(len(layers)))
    eager_ms = step_ms
    if args.graph:
        # the whole 24-layer step as one HIP graph (captured after the eager pass above, which
        # supplies the per-kernel times); value and ms_per_step are then the replay times
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(None)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / args.steps
    launches = args.steps * len(layers)
    # algorithmic HBM bytes of the attention: W cached K and V rows per (sequence, head), the
    # query read and the output written (bf16), lse (fp32)
    def attn_bytes(W):
        return B * H * (2 * W * D * 2 + 2 * D * 2 + 4)
    total_bytes = sum(attn_bytes(l["W"]) for l in layers)
    achieved = total_bytes / (dec_ms / args.steps * 1e-3) / 1e9
    return {
        "metric": DECODE_METRIC, "value": round(B / (step_ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "d24 decoding: 24 layers (18 x window 1024, 6 x 2048), 32 "
                               "sequences at position 2047, ring caches of 2048 slots, H=12, D=128",
                   "batch": B, "context": p_pos + 1, "parallelism": "single GPU"},
        "breakdown": {"swa_decode_ms_per_step": round(dec_ms / args.steps, 4),
                      "prologue_ms_per_step": round(eager_ms - dec_ms / args.steps, 4),
                      "attention_bytes_per_step": total_bytes,
                      "launch": "hip graph replay" if args.graph else "eager stream",
                      "eager_ms_per_step": round(eager_ms, 4)},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel + combine_kernel (swa_decode)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "avg_launch_us": round(dec_ms / launches * 1e3, 2), "traffic": None},
    }


def run_fp8_bench(args):
    """The d24 sweep's forward on fp8 operands: for each of the 24 layers (18 with W = 1024,
    6 with W = 2048; B=16, T=2048, H=12, D=128) rope_qknorm_fwd_fp8 (q_hat, k_hat written as
    e4m3 at scale 1), swa_fp8_pack of v (scale 1/64) and swa_fwd_fp8. value = 4*D FLOP per
    visible pair over the 24 layers / step time. The bf16 prologue + swa_fwd on the same inputs
    are timed alongside (outside the step) for comparison."""
    import torch
    from causal_sliding_window_rope_amd import binding as sw
    lib = sw.load()
    cfg = layer_list("sssl24")
    B, T, H, D = cfg["B"], cfg["T"], cfg["H"], cfg["D"]
    scale = D ** -0.5
    layers = make_layers(cfg, torch)
    nv = lib.swa_fp8_v_bytes(B, T, H, D)
    for t in layers:
        del t["dO"]
        t["q8"] = torch.empty((B, T, H, D), dtype=torch.uint8, device="cuda")
        t["k8"] = torch.empty_like(t["q8"])
        t["v8t"] = torch.empty(nv, dtype=torch.uint8, device="cuda")
    cs = sw.rope_table(T, D, 10000.0)
    P, stream = sw._ptr, sw._stream()
    sv = 1.0 / 64
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def call(name, *a):
        st = getattr(lib, name)(*a)
        if st != 0:
            raise sw.SwaError(name, st, lib.swa_last_error().decode())

    def step(rec):
        for li, t in enumerate(layers):
            call("rope_qknorm_fwd_fp8", P(t["q"]), P(t["k"]), P(cs), P(t["q8"]), P(t["k8"]), B, T,
                 H, D, 1e-6, sw.SWA_BF16, stream)
            if rec: rec[li][0].record()
            call("swa_fp8_pack", None, None, P(t["v"]), 1.0, 1.0, sv, None, None, P(t["v8t"]),
                 B, T, H, D, sw.SWA_BF16, stream)
            if rec: rec[li][1].record()
            call("swa_fwd_fp8", P(t["q8"]), P(t["k8"]), P(t["v8t"]), 1.0, 1.0, sv, None, P(t["o"]),
                 P(t["lse"]), B, T, H, D, t["W"], scale, stream)
            if rec: rec[li][2].record()

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = [[[ev(), ev(), ev()] for _ in layers] for _ in range(args.steps)]
    e0, e1 = ev(), ev()
    e0.record()
    for k in range(args.steps):
        step(recs[k])
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / args.steps
    nl = len(layers)
    pack_ms = sum(r[l][0].elapsed_time(r[l][1]) for r in recs for l in range(nl)) / args.steps
    f8_ms = sum(r[l][1].elapsed_time(r[l][2]) for r in recs for l in range(nl)) / args.steps
    # the bf16 kernel on the same inputs, for comparison
    for t in layers:
        call("rope_qknorm_fwd", P(t["q"]), P(t["k"]), P(cs), P(t["qn"]), P(t["kn"]), B, T, H, D,
             1e-6, sw.SWA_BF16, stream)
    b16 = [[ev(), ev()] for _ in range(nl * args.steps)]
    for k in range(args.steps):
        for li, t in enumerate(layers):
            b16[k * nl + li][0].record()
            call("swa_fwd", P(t["qn"]), P(t["kn"]), P(t["v"]), None, None, None, 0, None, P(t["o"]),
                 P(t["lse"]), B, T, H, D, t["W"], scale, sw.SWA_BF16, stream)
            b16[k * nl + li][1].record()
    torch.cuda.synchronize()
    bf_ms = sum(a.elapsed_time(b) for a, b in b16) / args.steps
    flop = sum(4 * D * pairs(T, t["W"]) * B * H for t in layers)
    value = flop / (step_ms * 1e-3) / 1e12
    f8_tf = flop / (f8_ms * 1e-3) / 1e12
    return {
        "metric": FP8_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "d24 sweep forward on fp8 (e4m3) operands: 24 layers "
                               "(18 x window 1024, 6 x 2048), B=16, T=2048, H=12, D=128",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": D,
                   "windows": sorted(set(cfg["windows"])), "parallelism": "single GPU"},
        "breakdown": {
            "algorithmic_tflop_per_step": round(flop / 1e12, 4),
            "swa_fwd_fp8_ms_per_step": round(f8_ms, 4),
            "swa_fwd_fp8_tflops": round(f8_tf, 2),
            "swa_fp8_pack_v_ms_per_step": round(pack_ms, 4),
            "prologue_ms_per_step": round(step_ms - f8_ms - pack_ms, 4),
            "bf16_swa_fwd_ms_same_inputs": round(bf_ms, 4),
            "bf16_swa_fwd_tflops": round(flop / (bf_ms * 1e-3) / 1e12, 2),
        },
        "roofline": {"bound": "mfma", "kernel": "fwd_fp8_kernel", "achieved": round(f8_tf, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(f8_tf / PEAK_FP8_TFLOPS, 4),
                     "avg_launch_us": round(f8_ms / nl * 1e3, 2),
                     "traffic": traffic_from_profile("fwd_fp8_kernel", "d24_fwd_fp8")},
    }


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by its copy-kernel calibration factor), if the
    counters were taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    name = kernel.split()[0]
    if name not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            ent = json.load(f)[workload]["kernels"][name]
    except (OSError, ValueError, KeyError):
        return None
    if ent.get("sources_sha256") != kernel_sources_sha256(name):
        return None
    return ent["hbm_bytes_per_launch"]


def cpu_baseline(args):
    """The fp64 numpy oracle, as it stands, on a bounded sample of the same workload: whole
    (b, h) heads of a short (1024) and a full (2048) d24 layer, prologue + attention forward and
    backward + prologue backward, until about args.cpu_seconds of CPU work."""
    import numpy as np
    import oracle
    from causal_sliding_window_rope_amd.inputs import make_inputs, small_workload
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cfg = layer_list(args.workload)
    T, D = cfg["T"], cfg["D"]
    wins = sorted(set(cfg["windows"]))
    done_flop, secs, heads = 0, 0.0, {}
    hcount = 0
    while secs < args.cpu_seconds and hcount < 512:
        W = wins[hcount % len(wins)]
        wl = small_workload(1, T, 1, D, W, "bf16", seed=9000 + hcount,
                            doc_mean=cfg.get("doc_mean") or 0)
        x = make_inputs(wl)
        f = {n: x[n].astype(np.float64) for n in ("q", "k", "v", "dO")}
        doc = x.get("doc_id")
        t0 = time.perf_counter()
        fwd = oracle.layer_fwd(f["q"], f["k"], f["v"], W, round_boundary=True, doc_id=doc)
        oracle.layer_bwd(f["q"], f["k"], f["v"], f["dO"], W, fwd, doc_id=doc)
        secs += time.perf_counter() - t0
        if doc is None:
            done_flop += 14 * D * pairs(T, W)
        else:
            done_flop += 14 * D * int(oracle.visible_mask(T, W, oracle.segment_ids(doc)[0]).sum())
        heads[W] = heads.get(W, 0) + 1
        hcount += 1
    sample = ", ".join(f"{n} head(s) of T={T}, D={D}, window {w}" for w, n in sorted(heads.items()))
    return {"value": round(done_flop / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, prologue + fwd + bwd of {sample}; "
                      f"{secs:.1f} s; {len(os.sched_getaffinity(0))} cores visible, "
                      f"{platform.processor() or platform.machine()}"}


def cpu_baseline_decode(args):
    """The decoding oracle (float64 numpy) on whole sequences of the decode workload: the
    positional prologue and the windowed attention of one new token, sequences until about
    args.cpu_seconds; tokens/s scaled to one token through all 24 layers."""
    import numpy as np
    from oracle.decode import decode_fwd, rope_qknorm_at
    from causal_sliding_window_rope_amd.inputs import sssl_windows
    H, D, cap, p_pos = 12, 128, 2048, 2047
    windows = sssl_windows(24, 1024, 2048)
    rng = np.random.default_rng(4242)
    kc = rng.standard_normal((1, cap, H, D))
    vc = rng.standard_normal((1, cap, H, D))
    secs, layers_done = 0.0, 0
    while secs < args.cpu_seconds and layers_done < 2400:
        W = windows[layers_done % len(windows)]
        q = rng.standard_normal((1, H, D))
        t0 = time.perf_counter()
        qn = rope_qknorm_at(q, np.array([p_pos]), 10000.0, 1e-6)
        decode_fwd(qn, kc, vc, np.array([p_pos]), W, D ** -0.5)
        secs += time.perf_counter() - t0
        layers_done += 1
    tokens = layers_done / len(windows)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    return {"value": round(tokens / secs, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 numpy decoding oracle, {layers_done} layer steps of one sequence "
                      f"({tokens:.1f} tokens through 24 layers) in {secs:.1f} s"}


def cpu_baseline_fp8(args):
    """The fp8 oracle (e4m3 quantisation of q_hat, k_hat, v and the float64 attention of the
    decoded values) on whole (b, h) heads of a short and a full d24 layer, forward only, until
    about args.cpu_seconds; TFLOP/s with the same 4*D-per-visible-pair count."""
    import numpy as np
    from oracle import fp8
    T, D = 2048, 128
    rng = np.random.default_rng(77)
    secs, flop, heads = 0.0, 0, {}
    while secs < args.cpu_seconds and sum(heads.values()) < 512:
        W = (1024, 2048)[sum(heads.values()) % 2]
        q, k, v = (rng.standard_normal((1, T, 1, D)) for _ in range(3))
        t0 = time.perf_counter()
        fp8.attention_fwd_fp8(fp8.quantize(q, 1.0), fp8.quantize(k, 1.0), fp8.quantize(v, 1 / 64),
                              1.0, 1.0, 1 / 64, W, D ** -0.5)
        secs += time.perf_counter() - t0
        flop += 4 * D * pairs(T, W)
        heads[W] = heads.get(W, 0) + 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    sample = ", ".join(f"{n} head(s) of window {w}" for w, n in sorted(heads.items()))
    return {"value": round(flop / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 numpy fp8 oracle (quantise + forward) on {sample}, T={T}, D={D}; "
                      f"{secs:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sssl24",
                    choices=["sssl24", "d24_short", "d24_full", "gpt2_124m", "d24_short_ve",
                             "d24_short_doc", "d24_short_vetable", "d24_decode", "d24_fwd_fp8"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--fused-gate", action="store_true",
                    help="gated workloads: form v_eff inside the attention kernels instead of "
                         "materialising it once per layer (the default, faster route)")
    ap.add_argument("--graph", action="store_true",
                    help="time the whole step (24-layer sweep, single layer or decoding step) as "
                         "one captured HIP graph (replays) instead of eager launches; the "
                         "per-kernel figures still come from an eager pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd", choices=("ds", "recompute"), default="ds",
                    help="backward: dS stored by the dK/dV kernel and read by the dQ kernel "
                         "(default), or S and dP recomputed in both")
    ap.add_argument("--qnorm", choices=("auto", "on", "off", "fwd", "bwd"), default="auto",
                    help="with --bwd ds: run the query half of the RoPE/QK-norm prologue and of "
                         "its backward inside the forward and dQ kernels (swa_fwd_qnorm, "
                         "swa_bwd_dq_ds_qnorm: on), only the forward half (fwd) or only the "
                         "backward half (bwd) there, or both in the separate prologue calls "
                         "(off); auto: on")
    ap.add_argument("--no-qnorm", action="store_true", help="the same as --qnorm off")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain device-to-device copy of this many MiB 5 times (used to "
                         "scale HBM byte counters under rocprofv3), then exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the benchmark measures one GPU "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.workload == "d24_fwd_fp8":
        res = run_fp8_bench(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_fp8(args)
        print(json.dumps(res), flush=True)
        return
    if args.workload == "d24_decode":
        res = run_decode_bench(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_decode(args)
        print(json.dumps(res), flush=True)
        return
    res = run_bench(args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
