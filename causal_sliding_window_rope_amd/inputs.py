"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and casts them to the storage precision.
It holds none of the attention, RoPE, norm or gate arithmetic, so the HIP path
and the CPU oracle can both be fed from it without sharing any of the method.

Recipe (the same on every machine):

* generator: ``numpy.random.default_rng(seed)``; every draw is
  ``standard_normal(shape)`` in float64, C order;
* draw order: q, k, v, dO (each (B, T, H, D)); for gated-value-embedding
  workloads the stream continues with x (B, T, C), Wg (32, H) scaled by 0.02
  (standard deviation 0.02), the embedding table (vocab, H*D), then token ids
  ``integers(0, vocab, (B, T))``; ve = table[ids]; table-mode workloads keep the
  table and the ids (int32) instead of handing over the gathered rows;
* document-masked workloads continue with the document layout: per row,
  documents of length max(1, round(lognormal(log(mean) - 1/2, 1))) tokens
  back to back, the last one cut at the row end (a BOS-aligned packed row);
  doc_id (B, T) int32 numbers the documents of a row 0, 1, ...;
* cast float64 -> float32 (numpy, round to nearest even), then for bf16
  workloads float32 -> bfloat16 with round-to-nearest-even on the bit pattern.
  bf16 values are returned as float32 arrays whose values are exactly
  representable in bfloat16, so they convert to torch.bfloat16 without change.
"""

from __future__ import annotations

import dataclasses

import numpy as np

VOCAB = 50304  # GPT-2 vocabulary padded to a multiple of 64
GATE_CH = 32   # the gate reads the first 32 channels of the block input


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Workload:
    """Shape and options of one attention layer call."""
    name: str
    B: int
    T: int
    H: int
    D: int
    window: int          # keys per query including itself; >= T means full causal
    dtype: str           # "f32" or "bf16"
    seed: int
    base: float = 10000.0
    eps: float = 1e-6
    gate: bool = False   # gated value embedding on V
    C: int = 0           # width of the block input x (gate workloads only)
    vocab: int = VOCAB
    doc_mean: int = 0    # mean document length of a packed row (0: one document per row)
    ve_table: bool = False   # hand the value-embedding table and token ids to the kernels

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


# The five workloads: a tiny fp32 causal case, the GPT-2 124M layer, the
# nanochat d24 short (window 1024) layer, its full (2048) layer as used in the
# 3-short:1-long sweep, and the d24 short layer with the value-embedding gate.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, T=64, H=2, D=64, window=64, dtype="f32", seed=0),
    "gpt2_124m": Workload("gpt2_124m", B=8, T=1024, H=12, D=64, window=1024, dtype="bf16", seed=2),
    "d24_short": Workload("d24_short", B=16, T=2048, H=12, D=128, window=1024, dtype="bf16", seed=3),
    "d24_full": Workload("d24_full", B=16, T=2048, H=12, D=128, window=2048, dtype="bf16", seed=1003),
    "d24_short_ve": Workload("d24_short_ve", B=16, T=2048, H=12, D=128, window=1024, dtype="bf16",
                             seed=5, gate=True, C=1536),
    # the d24 short layer on BOS-aligned rows packing documents of ~512 tokens on average
    "d24_short_doc": Workload("d24_short_doc", B=16, T=2048, H=12, D=128, window=1024,
                              dtype="bf16", seed=7, doc_mean=512),
    # the gated layer reading its value embedding from the (vocab, H*D) table by token id
    "d24_short_vetable": Workload("d24_short_vetable", B=16, T=2048, H=12, D=128, window=1024,
                                  dtype="bf16", seed=5, gate=True, C=1536, ve_table=True),
}


def sssl_windows(n_layers: int = 24, short: int = 1024, long: int = 2048) -> list[int]:
    """Per-layer windows of the 3-short:1-long tiling: every fourth layer (3, 7, ...) is full."""
    return [long if (l % 4) == 3 else short for l in range(n_layers)]


def sssl_layer_workload(layer: int, B: int = 16, T: int = 2048, H: int = 12, D: int = 128) -> Workload:
    w = sssl_windows()[layer]
    return Workload(f"d24_layer{layer}", B=B, T=T, H=H, D=D, window=w, dtype="bf16", seed=1000 + layer)


def make_inputs(wl: Workload, heads: tuple[int, int] | None = None) -> dict[str, np.ndarray]:
    """Draw the inputs of one workload.

    Returns float32 arrays q, k, v, dO of shape (B, T, H, D) (bf16-representable
    when wl.dtype == "bf16"); with the gate also x (B, T, C), Wg (32, H) kept in
    float32, ve (B, T, H*D) and ids (B, T) int64.
    ``heads=(b_count, h_count)`` keeps only the first b_count sequences and
    h_count heads after drawing the full tensors (used for bounded CPU samples).
    """
    rng = np.random.default_rng(wl.seed)
    shp = (wl.B, wl.T, wl.H, wl.D)
    out: dict[str, np.ndarray] = {}
    for name in ("q", "k", "v", "dO"):
        out[name] = rng.standard_normal(shp).astype(np.float32)
    if wl.gate:
        out["x"] = rng.standard_normal((wl.B, wl.T, wl.C)).astype(np.float32)
        out["Wg"] = (rng.standard_normal((GATE_CH, wl.H)) * 0.02).astype(np.float32)
        table = rng.standard_normal((wl.vocab, wl.H * wl.D)).astype(np.float32)
        ids = rng.integers(0, wl.vocab, (wl.B, wl.T))
        if wl.dtype == "bf16":
            table = round_to_bf16(table)
        out["ve"] = table[ids]
        out["ids"] = ids
        if wl.ve_table:
            out["table"] = table
            out["ids"] = ids.astype(np.int32)
        del table
    if wl.doc_mean > 0:
        out["doc_id"] = doc_layout(rng, wl.B, wl.T, wl.doc_mean)
    if wl.dtype == "bf16":
        for name in ("q", "k", "v", "dO", "x"):
            if name in out:
                out[name] = round_to_bf16(out[name])
    if heads is not None:
        nb, nh = heads
        for name in ("q", "k", "v", "dO"):
            out[name] = np.ascontiguousarray(out[name][:nb, :, :nh])
        if wl.gate:
            out["x"] = np.ascontiguousarray(out["x"][:nb])
            out["Wg"] = np.ascontiguousarray(out["Wg"][:, :nh])
            out["ve"] = np.ascontiguousarray(out["ve"][:nb].reshape(nb, wl.T, wl.H, wl.D)[:, :, :nh]
                                             .reshape(nb, wl.T, nh * wl.D))
            out["ids"] = out["ids"][:nb]
        if wl.doc_mean > 0:
            out["doc_id"] = np.ascontiguousarray(out["doc_id"][:nb])
    return out


def doc_layout(rng, B: int, T: int, mean_len: float) -> np.ndarray:
    """(B, T) int32 document numbers of BOS-aligned packed rows (see the module recipe)."""
    ids = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        t, d = 0, 0
        while t < T:
            n = max(1, int(round(rng.lognormal(np.log(mean_len) - 0.5, 1.0))))
            ids[b, t:t + n] = d
            t += n
            d += 1
    return ids


def small_workload(B: int, T: int, H: int, D: int, window: int, dtype: str, seed: int,
                   gate: bool = False, C: int = 64, doc_mean: int = 0, ve_table: bool = False,
                   vocab: int = VOCAB) -> Workload:
    """A parity-test case with arbitrary (small) sizes and the same recipe."""
    return Workload(f"case_B{B}_T{T}_H{H}_D{D}_W{window}_{dtype}", B=B, T=T, H=H, D=D,
                    window=window, dtype=dtype, seed=seed, gate=gate, C=C if gate else 0,
                    doc_mean=doc_mean, ve_table=ve_table, vocab=vocab)
