"""Oracle for the attention prologue: RoPE, then parameter-free RMS QK-norm.

TEST INFRASTRUCTURE (see the package docstring).

Passages followed:

* "从4万美元到73美元：GPT-2复现的成本革命" (intelliparadigm.com), §2.2: q and k
  are normalised after RoPE, ``q, k = normalize(apply_rope(q)), normalize(apply_rope(k))``;
  §2.1: the normalisation is an RMSNorm with no learnable gamma/beta.
* "NanoGPT Speedrun：大模型训练效率的极限竞速指南" (kongchang.com), "模型架构层面的改进":
  RoPE rotates q and k by a position-dependent rotation so that scores depend
  on relative position. The pages give no formula; the reading used here is
  the rotate-half pairing (i, i + D/2) with angle t * theta_i,
  theta_i = base^(-2i/D), applied to all D dims, positions t = 0..T-1 in every
  sequence ("GPT-2 124M 复现" §9: each row of a batch is an independent sequence).
* eps = 1e-6 inside the square root.

Arrays are (B, T, H, D) float64.
"""

from __future__ import annotations

import numpy as np


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), via float32; returns float64.

    Used only to model the places where the library stores bf16 tensors
    (its inputs and the normalised q, k it writes), so that the oracle sees the
    same operands as the kernels.
    """
    f = np.asarray(a, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def rope_angles(T: int, D: int, base: float) -> np.ndarray:
    """Angle table a[t, i] = t * base^(-2i/D) for t < T, i < D/2 (float64)."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    t = np.arange(T, dtype=np.float64)
    return t[:, None] * theta[None, :]


def rope(x: np.ndarray, base: float) -> np.ndarray:
    """Rotate each pair (x_i, x_{i+D/2}) of every (b, t, h) row by angle t*theta_i."""
    B, T, H, D = x.shape
    ang = rope_angles(T, D, base)[None, :, None, :]   # (1, T, 1, D/2)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_transpose(dy: np.ndarray, base: float) -> np.ndarray:
    """Apply the transpose of the RoPE rotation (rotation by -t*theta_i): its backward."""
    B, T, H, D = dy.shape
    ang = rope_angles(T, D, base)[None, :, None, :]
    c, s = np.cos(ang), np.sin(ang)
    d1, d2 = dy[..., : D // 2], dy[..., D // 2:]
    return np.concatenate([d1 * c + d2 * s, -d1 * s + d2 * c], axis=-1)


def rms_norm(u: np.ndarray, eps: float):
    """x_hat = u / sqrt(mean_d u^2 + eps) per row; also returns r = 1/sqrt(mean u^2 + eps)."""
    r = 1.0 / np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    return u * r, r


def rms_norm_bwd(x_hat: np.ndarray, r: np.ndarray, dx_hat: np.ndarray) -> np.ndarray:
    """Backward of x_hat = u * r(u): du = r * (dx_hat - x_hat * mean_d(x_hat * dx_hat)).

    Derivation: d r / d u_j = -r^3 u_j / D, so
    du_j = r dx_j - (r^3 u_j / D) sum_d u_d dx_d = r (dx_j - x_hat_j (x_hat . dx) / D).
    """
    D = x_hat.shape[-1]
    dot = np.sum(x_hat * dx_hat, axis=-1, keepdims=True)
    return r * (dx_hat - x_hat * dot / D)


def rope_qknorm(x: np.ndarray, base: float, eps: float):
    """Prologue of one of q or k: x_hat = RMSNorm(RoPE(x)). Returns (x_hat, r)."""
    return rms_norm(rope(x, base), eps)


def rope_qknorm_bwd(x: np.ndarray, dx_hat: np.ndarray, base: float, eps: float) -> np.ndarray:
    """Gradient of the prologue w.r.t. the pre-RoPE input x, given d(x_hat)."""
    x_hat, r = rope_qknorm(x, base, eps)
    du = rms_norm_bwd(x_hat, r, dx_hat)
    return rope_transpose(du, base)
