"""Pins of the oracle's document masking (attention restricted to a token's own document).

Independent references: hand-evaluated segment ids; torch SDPA and autograd in float64 with a
document mask built by explicit loops over the rows; the no-document path (one document per
row must give the same numbers); separate calls on each document (documents do not see one
another); the online recurrence; central finite differences through the whole layer. CPU only.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _doc_ids(B, T, lengths_seed, mean_len):
    """Random document layout: consecutive runs with lengths 1 + Poisson(mean_len - 1)."""
    rng = np.random.default_rng(lengths_seed)
    ids = np.zeros((B, T), dtype=np.int64)
    for b in range(B):
        t, d = 0, 100 * b
        while t < T:
            n = 1 + int(rng.poisson(mean_len - 1))
            ids[b, t:t + n] = d
            t += n
            d += 1 + int(rng.integers(0, 3))   # ids need not be consecutive
    return ids


def _loop_mask(ids_row, W):
    """Visible pairs by direct loops: j <= i, i - j < W, and no change of id between j and i."""
    T = len(ids_row)
    m = torch.zeros(T, T, dtype=torch.bool)
    for i in range(T):
        j = i
        while j >= 0 and i - j < W:
            m[i, j] = True
            if j > 0 and ids_row[j - 1] != ids_row[j]:
                break
            j -= 1
    return m


def test_segment_ids_hand_values():
    ids = np.array([[5, 5, 7, 7, 7, 5, 9], [1, 1, 1, 1, 1, 1, 1]])
    np.testing.assert_array_equal(oracle.segment_ids(ids),
                                  [[0, 0, 1, 1, 1, 2, 3], [0, 0, 0, 0, 0, 0, 0]])


@pytest.mark.parametrize("T,W,mean_len", [(40, 40, 6), (40, 7, 10), (64, 64, 1), (33, 5, 20)])
def test_doc_attention_matches_torch_sdpa(T, W, mean_len):
    B, H, D = 2, 2, 16
    q, k, v, do = (_rand((B, T, H, D), s) for s in (11, 12, 13, 14))
    ids = _doc_ids(B, T, 7 + T + W, mean_len)
    scale = 1.0 / math.sqrt(D)
    O, lse = oracle.attention_fwd(q, k, v, W, scale, doc_id=ids)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, scale, doc_id=ids)
    qt, kt, vt = (torch.from_numpy(x).transpose(1, 2).requires_grad_(True) for x in (q, k, v))
    mask = torch.stack([_loop_mask(ids[b], W) for b in range(B)])[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(O, o.transpose(1, 2).detach().numpy(), rtol=1e-12, atol=1e-12)
    s = scale * torch.einsum("bihd,bjhd->bhij", torch.from_numpy(q), torch.from_numpy(k))
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)
    o.backward(torch.from_numpy(do).transpose(1, 2))
    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(mine, ref.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_one_document_is_the_plain_path():
    B, T, H, D, W = 2, 37, 2, 8, 9
    q, k, v, do = (_rand((B, T, H, D), s) for s in (21, 22, 23, 24))
    ids = np.full((B, T), 3)
    O0, l0 = oracle.attention_fwd(q, k, v, W, 0.3)
    O1, l1 = oracle.attention_fwd(q, k, v, W, 0.3, doc_id=ids)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(l0, l1)
    g0 = oracle.attention_bwd(q, k, v, do, W, 0.3)
    g1 = oracle.attention_bwd(q, k, v, do, W, 0.3, doc_id=ids)
    for a, b in zip(g0, g1):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("W", [4, 100])
def test_documents_are_independent_sequences(W):
    """Each document gives what attention on that document alone gives (positions restart)."""
    H, D = 2, 8
    lens = [5, 1, 17, 9]
    T = sum(lens)
    q, k, v, do = (_rand((1, T, H, D), s) for s in (31, 32, 33, 34))
    ids = np.concatenate([np.full(n, i) for i, n in enumerate(lens)])[None]
    O, lse = oracle.attention_fwd(q, k, v, W, 0.25, doc_id=ids)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, W, 0.25, doc_id=ids)
    t0 = 0
    for n in lens:
        sl = slice(t0, t0 + n)
        Os, ls = oracle.attention_fwd(q[:, sl], k[:, sl], v[:, sl], W, 0.25)
        gs = oracle.attention_bwd(q[:, sl], k[:, sl], v[:, sl], do[:, sl], W, 0.25)
        np.testing.assert_allclose(O[:, sl], Os, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, sl], ls, rtol=1e-12, atol=1e-13)
        for a, b in zip((dq, dk, dv), gs):
            np.testing.assert_allclose(a[:, sl], b, rtol=1e-11, atol=1e-12)
        t0 += n


def test_online_recurrence_with_documents():
    B, T, H, D, W = 2, 45, 2, 8, 13
    q, k, v = (_rand((B, T, H, D), s) for s in (41, 42, 43))
    ids = _doc_ids(B, T, 5, 8)
    O, lse = oracle.attention_fwd(q, k, v, W, 0.35, doc_id=ids)
    O2, lse2 = oracle.attention_fwd_online(q, k, v, W, 0.35, block=7, doc_id=ids)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_layer_finite_differences_with_documents():
    """Loss = sum(O * dO) through RoPE, QK-norm and document-masked attention."""
    B, T, H, D, W = 1, 12, 2, 8, 6
    q, k, v, dO = (_rand((B, T, H, D), s) for s in (51, 52, 53, 54))
    ids = np.array([[0, 0, 0, 0, 1, 1, 1, 1, 1, 2, 3, 3]])
    fwd = oracle.layer_fwd(q, k, v, W, doc_id=ids)
    bwd = oracle.layer_bwd(q, k, v, dO, W, fwd, doc_id=ids)

    def loss(q_, k_, v_):
        return float(np.sum(oracle.layer_fwd(q_, k_, v_, W, doc_id=ids)["O"] * dO))

    h = 1e-6
    rng = np.random.default_rng(3)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - bwd[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, bwd[name][idx])
