"""Oracle for the gated value embedding added to V.

TEST INFRASTRUCTURE (see the package docstring).

Passage followed: lanjinlin.com.cn repost of the nanochat d24 write-up,
sub-head "3. Value Embeddings": ``ve = value_embeds[layer](token_ids)``,
``gate = 2 * sigmoid(ve_gate(x[:, :, :32]))`` with range (0, 2), ``v = v + gate * ve``.
Reading: ve_gate is a bias-free 32 -> H projection (one gate per head, broadcast
over the head's D channels); ve channel c belongs to head c // D.
The intelliparadigm.com page's §4.1 snippet (no projection, adds to x) is
taken as garbled.
"""

from __future__ import annotations

import numpy as np


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def ve_gate(x32: np.ndarray, Wg: np.ndarray) -> np.ndarray:
    """g[b, t, h] = 2 * sigmoid(sum_c x32[b, t, c] * Wg[c, h]); x32 is (B, T, 32), Wg (32, H)."""
    z = np.einsum("btc,ch->bth", x32, Wg)
    return 2.0 * _sigmoid(z)


def apply_gate(v: np.ndarray, g: np.ndarray, ve: np.ndarray) -> np.ndarray:
    """v_eff = v + g * ve with v (B, T, H, D), g (B, T, H), ve (B, T, H*D)."""
    B, T, H, D = v.shape
    return v + g[..., None] * ve.reshape(B, T, H, D)


def ve_gate_bwd(x32: np.ndarray, Wg: np.ndarray, g: np.ndarray, dv_eff: np.ndarray,
                ve: np.ndarray):
    """Backward of v_eff = v + g * ve, g = 2 sigmoid(x32 Wg).

    Returns (dv, dve, dg, dWg, dx32):
    dv = dv_eff; dve = g * dv_eff; dg = sum_d dv_eff * ve;
    dz = dg * g * (1 - g / 2)   (d/dz of 2 sigmoid(z) = 2 s (1 - s) = g (1 - g/2));
    dWg = sum_{b,t} x32^T dz; dx32 = dz Wg^T.
    """
    B, T, H, D = dv_eff.shape
    ve4 = ve.reshape(B, T, H, D)
    dv = dv_eff.copy()
    dve = (g[..., None] * dv_eff).reshape(B, T, H * D)
    dg = np.sum(dv_eff * ve4, axis=-1)
    dz = dg * g * (1.0 - g / 2.0)
    dWg = np.einsum("btc,bth->ch", x32, dz)
    dx32 = np.einsum("bth,ch->btc", dz, Wg)
    return dv, dve, dg, dWg, dx32


def ve_lookup(table: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """ve[b, t] = table[ids[b, t]]: the value-embedding row of each token (B, T, H*D).

    The write-up's ``value_embeds[layer_idx](token_ids)`` is an embedding lookup; reading:
    ids outside [0, rows) contribute a zero row (they never occur for valid tokens).
    """
    ids = np.asarray(ids)
    ok = (ids >= 0) & (ids < table.shape[0])
    out = table[np.where(ok, ids, 0)]
    return np.where(ok[..., None], out, 0.0)


def ve_table_grad(dve: np.ndarray, ids: np.ndarray, rows: int) -> np.ndarray:
    """Gradient of the table from the per-token gradients: dtable[v] = sum of dve[b, t] over the
    tokens with ids[b, t] == v (invalid ids contribute nothing)."""
    ids = np.asarray(ids).reshape(-1)
    flat = dve.reshape(ids.shape[0], -1)
    out = np.zeros((rows, flat.shape[1]))
    ok = (ids >= 0) & (ids < rows)
    np.add.at(out, ids[ok], flat[ok])
    return out
