"""Oracle for sliding-window decoding from a K/V cache (one new token per sequence).

TEST INFRASTRUCTURE (see the package docstring).

Passages followed:

* "GPT-2 124M 复现" (notes.cassieliang.com) §7: the course's generation loop
  recomputes every prefix position each step (no K/V cache); production
  generation keeps the past keys and values instead. Reading: one decoding
  step for a sequence whose new token sits at position p computes exactly the
  row p of the training forward (same RoPE angle p * theta_i, same QK-norm,
  same window), reading the keys and values of positions max(0, p-W+1)..p from
  a cache.
* Cache layout (a reading; the pages fix none): per sequence a ring of C slots,
  position j stored at slot j mod C, in the native (B, C, H, D) layout. A window
  of W keys needs W <= C. C >= the longest context means no wrap at all.

Arrays are float64: qn, o (B, H, D); caches (B, C, H, D); pos (B,); lse (B, H).
"""

from __future__ import annotations

import numpy as np

from .prologue import rms_norm


def rope_qknorm_at(x: np.ndarray, pos: np.ndarray, base: float, eps: float) -> np.ndarray:
    """RoPE at position pos[b] of each row x[b, h] (B, H, D), then the RMS QK-norm."""
    B, H, D = x.shape
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None, None] * theta[None, None, :]   # (B, 1, D/2)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    u = np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)
    return rms_norm(u, eps)[0]


def window_positions(p: int, window: int) -> np.ndarray:
    """Key positions a query at position p sees: max(0, p-W+1) .. p."""
    return np.arange(max(0, p - window + 1), p + 1)


def decode_fwd(qn: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos, window: int,
               scale: float):
    """Attention of each sequence's new query over its cached window: o (B, H, D), lse (B, H)."""
    B, C, H, D = k_cache.shape
    assert window <= C, "the ring must hold the whole window"
    o = np.zeros((B, H, v_cache.shape[-1]))
    lse = np.zeros((B, H))
    for b in range(B):
        slots = window_positions(int(pos[b]), window) % C
        for h in range(H):
            s = scale * (k_cache[b, slots, h] @ qn[b, h])
            m = np.max(s)
            L = m + np.log(np.sum(np.exp(s - m)))
            o[b, h] = np.exp(s - L) @ v_cache[b, slots, h]
            lse[b, h] = L
    return o, lse
