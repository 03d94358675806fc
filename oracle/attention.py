"""Oracle for causal sliding-window softmax attention, forward and backward.

TEST INFRASTRUCTURE (see the package docstring).

Passages followed:

* "GPT-2 124M 复现" (notes.cassieliang.com), §3: scores = (q k^T) / sqrt(D);
  the causal mask is lower-triangular including the diagonal (position t never
  sees t+1 ...); softmax over the key axis; y = att @ v; heads are a batch axis.
* "从4万美元到73美元：GPT-2复现的成本革命" (intelliparadigm.com), §3.2: layers use
  a local window of 1024 tokens or the full 2048-token window. Reading: a window
  W admits keys j with i - W + 1 <= j <= i (W keys including the query itself);
  W >= T is plain causal attention.
* "GPT-2 124M 复现" §19: FlashAttention computes the same function exactly; the
  online softmax keeps a running row max m and normaliser l,
  m' = max(m, max s), l' = exp(m - m') l + sum exp(s - m'), and rescales the
  V accumulator by the same factor; the backward recomputes intermediates.
  ``attention_fwd_online`` follows that recurrence block by block; it is a
  second statement of the forward used to pin the dense one.
* Document masking (optional ``doc_id``): "从4万美元到73美元" §6.1 packs several
  documents into one BOS-aligned row, and §7 of that page ("避坑指南") lists
  variable-length (per-document) attention among the alternatives tried; "神级项目训练GPT-2仅需5分钟" notes that
  longer rows with FlexAttention split fewer documents. Reading: a token attends
  only inside its own document, a document being a maximal run of equal
  ``doc_id`` values along the row; the causal window applies as well.
* The backward is the chain rule through softmax written out by hand:
  dV = P^T dO, dP = dO V^T, dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
  dq = scale dS K, dk = scale dS^T Q.

Layout: q, k, v, dO and outputs are (B, T, H, D) float64; lse is (B, H, T),
natural log. All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np


def window_mask(T: int, window: int) -> np.ndarray:
    """Boolean (T, T) mask, True where key j is visible to query i: i - W < j <= i."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & (j > i - window)


def segment_ids(doc_id: np.ndarray) -> np.ndarray:
    """(B, T) index of the maximal run of equal doc_id values each token lies in (per row)."""
    doc_id = np.asarray(doc_id)
    change = np.ones(doc_id.shape, dtype=bool)
    change[:, 1:] = doc_id[:, 1:] != doc_id[:, :-1]
    return np.cumsum(change, axis=1) - 1


def visible_mask(T: int, window: int, seg_row: np.ndarray | None = None) -> np.ndarray:
    """(T, T) mask of visible pairs: the causal window and, with a segment row, the same run."""
    m = window_mask(T, window)
    if seg_row is not None:
        m = m & (seg_row[:, None] == seg_row[None, :])
    return m


def _masks(B: int, T: int, window: int, doc_id):
    if doc_id is None:
        m = window_mask(T, window)
        return [m] * B
    seg = segment_ids(doc_id)
    return [visible_mask(T, window, seg[b]) for b in range(B)]


def pair_count(T: int, window: int) -> int:
    """Number of visible (query, key) pairs per sequence and head: sum_i min(i + 1, W)."""
    return int(sum(min(i + 1, window) for i in range(T)))


def _scores(qh: np.ndarray, kh: np.ndarray, scale: float, mask: np.ndarray) -> np.ndarray:
    s = scale * (qh @ kh.T)
    return np.where(mask, s, -np.inf)


def attention_probs(qh: np.ndarray, kh: np.ndarray, window: int, scale: float,
                    doc_id=None) -> np.ndarray:
    """Dense softmax matrix P (B, H, T, T) (zeros outside the window). Small inputs only."""
    B, T, H, D = qh.shape
    masks = _masks(B, T, window, doc_id)
    P = np.zeros((B, H, T, T))
    for b in range(B):
        for h in range(H):
            s = _scores(qh[b, :, h], kh[b, :, h], scale, masks[b])
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            P[b, h] = e / np.sum(e, axis=1, keepdims=True)
    return P


def attention_fwd(qh: np.ndarray, kh: np.ndarray, v: np.ndarray, window: int, scale: float,
                  doc_id=None):
    """Dense forward: O (B, T, H, D) and lse (B, H, T).

    lse_i = m_i + log sum_j exp(s_ij - m_i), m_i = max_j s_ij; O_i = sum_j exp(s_ij - lse_i) v_j.
    """
    B, T, H, D = qh.shape
    masks = _masks(B, T, window, doc_id)
    O = np.zeros((B, T, H, v.shape[-1]))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            s = _scores(qh[b, :, h], kh[b, :, h], scale, masks[b])
            m = np.max(s, axis=1, keepdims=True)
            l = np.sum(np.exp(s - m), axis=1, keepdims=True)
            L = m + np.log(l)
            P = np.exp(s - L)
            O[b, :, h] = P @ v[b, :, h]
            lse[b, h] = L[:, 0]
    return O, lse


def attention_fwd_online(qh: np.ndarray, kh: np.ndarray, v: np.ndarray, window: int, scale: float,
                         block: int = 16, doc_id=None):
    """Forward by the online-softmax recurrence over key blocks of ``block`` keys."""
    B, T, H, D = qh.shape
    masks = _masks(B, T, window, doc_id)
    O = np.zeros((B, T, H, v.shape[-1]))
    lse = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            q, k, vv = qh[b, :, h], kh[b, :, h], v[b, :, h]
            mask = masks[b]
            m = np.full((T, 1), -np.inf)
            l = np.zeros((T, 1))
            acc = np.zeros((T, vv.shape[-1]))
            for j0 in range(0, T, block):
                j1 = min(j0 + block, T)
                s = scale * (q @ k[j0:j1].T)
                s = np.where(mask[:, j0:j1], s, -np.inf)
                m_new = np.maximum(m, np.max(s, axis=1, keepdims=True))
                # rows whose keys so far are all masked keep m = -inf; leave them untouched
                live = np.isfinite(m_new)
                alpha = np.where(live, np.exp(np.where(live, m, 0.0) - np.where(live, m_new, 0.0)), 1.0)
                e = np.where(live, np.exp(s - np.where(live, m_new, 0.0)), 0.0)
                l = alpha * l + np.sum(e, axis=1, keepdims=True)
                acc = alpha * acc + e @ vv[j0:j1]
                m = m_new
            O[b, :, h] = acc / l
            lse[b, h] = (m + np.log(l))[:, 0]
    return O, lse


def attention_bwd(qh: np.ndarray, kh: np.ndarray, v: np.ndarray, dO: np.ndarray, window: int,
                  scale: float, lse: np.ndarray | None = None, doc_id=None):
    """Backward: (dq, dk, dv) w.r.t. the attention inputs, given the upstream dO.

    P is recomputed from the scores and lse (computed here when not given).
    """
    B, T, H, D = qh.shape
    if lse is None:
        _, lse = attention_fwd(qh, kh, v, window, scale, doc_id=doc_id)
    masks = _masks(B, T, window, doc_id)
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            q, k, vv, do = qh[b, :, h], kh[b, :, h], v[b, :, h], dO[b, :, h]
            s = _scores(q, k, scale, masks[b])
            P = np.exp(s - lse[b, h][:, None])
            dv[b, :, h] = P.T @ do
            dP = do @ vv.T
            rowdot = np.sum(P * dP, axis=1, keepdims=True)
            dS = P * (dP - rowdot)
            dq[b, :, h] = scale * (dS @ k)
            dk[b, :, h] = scale * (dS.T @ q)
    return dq, dk, dv
