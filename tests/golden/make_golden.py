"""Writes tests/golden/tiny_f32_oracle.json: oracle outputs on the tiny fp32 causal workload.

Calls only oracle/ and the seeded input generator. The stored numbers are a
regression anchor for the oracle itself (they pin nothing about the pages);
the pins live in tests/test_oracle_*.py.
Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from causal_sliding_window_rope_amd.inputs import WORKLOADS, make_inputs  # noqa: E402


def summarise(a):
    a = np.asarray(a, dtype=np.float64)
    flat = a.reshape(-1)
    idx = np.linspace(0, flat.size - 1, 7).astype(int)
    return {"sum": float(flat.sum()), "sumsq": float((flat * flat).sum()),
            "samples": [[int(i), float(flat[i])] for i in idx]}


def main():
    wl = WORKLOADS["tiny_f32"]
    x = {k: v.astype(np.float64) for k, v in make_inputs(wl).items()}
    fwd = oracle.layer_fwd(x["q"], x["k"], x["v"], wl.window, base=wl.base, eps=wl.eps)
    bwd = oracle.layer_bwd(x["q"], x["k"], x["v"], x["dO"], wl.window, fwd, base=wl.base, eps=wl.eps)
    out = {"workload": "tiny_f32 (B=1, T=64, H=2, D=64, window 64, base 1e4, eps 1e-6, seed 0)",
           "O": summarise(fwd["O"]), "lse": summarise(fwd["lse"]), "qh": summarise(fwd["qh"]),
           "dq": summarise(bwd["dq"]), "dk": summarise(bwd["dk"]), "dv": summarise(bwd["dv"])}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
