"""Pins of the decoding oracle against the training-path oracle: a decoding step at position p
is row p of the full-sequence layer (RoPE, QK-norm, windowed attention), whatever the ring
capacity, and the positional prologue equals the sequence prologue's row p. CPU only."""

import numpy as np
import pytest

import oracle
from oracle.decode import decode_fwd, rope_qknorm_at, window_positions


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_window_positions():
    np.testing.assert_array_equal(window_positions(0, 4), [0])
    np.testing.assert_array_equal(window_positions(2, 4), [0, 1, 2])
    np.testing.assert_array_equal(window_positions(9, 4), [6, 7, 8, 9])


def test_positional_prologue_is_the_sequence_prologue_row():
    B, T, H, D = 2, 40, 3, 16
    x = _rand((B, T, H, D), 1)
    full, _ = oracle.rope_qknorm(x, 10000.0, 1e-6)
    for p in (0, 1, 17, 39):
        got = rope_qknorm_at(x[:, p], np.full(B, p), 10000.0, 1e-6)
        np.testing.assert_allclose(got, full[:, p], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("W,C", [(8, 40), (8, 8), (8, 11), (40, 40), (3, 5)])
def test_decoding_step_is_the_training_row(W, C):
    """Fill a ring of C slots with the normalised keys / raw values of positions 0..p (later
    positions overwrite earlier slots) and decode position p; compare with the layer's row p."""
    B, T, H, D = 2, 40, 2, 16
    q, k, v = (_rand((B, T, H, D), s) for s in (2, 3, 4))
    fwd = oracle.layer_fwd(q, k, v, W)
    kn_all, _ = oracle.rope_qknorm(k, 10000.0, 1e-6)
    for p in (0, 5, W - 1, 23, T - 1):
        kc = np.full((B, C, H, D), np.nan)
        vc = np.full((B, C, H, D), np.nan)
        for j in range(p + 1):
            kc[:, j % C] = kn_all[:, j]
            vc[:, j % C] = v[:, j]
        pos = np.full(B, p)
        qn = rope_qknorm_at(q[:, p], pos, 10000.0, 1e-6)
        o, lse = decode_fwd(qn, kc, vc, pos, W, 1.0 / np.sqrt(D))
        np.testing.assert_allclose(o, fwd["O"][:, p], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, fwd["lse"][:, :, p], rtol=1e-12, atol=1e-12)


def test_sequences_at_different_positions():
    B, T, H, D, W = 3, 30, 2, 8, 6
    q, k, v = (_rand((B, T, H, D), s) for s in (5, 6, 7))
    fwd = oracle.layer_fwd(q, k, v, W)
    kn_all, _ = oracle.rope_qknorm(k, 10000.0, 1e-6)
    pos = np.array([3, 29, 11])
    C = 7
    kc = np.zeros((B, C, H, D))
    vc = np.zeros((B, C, H, D))
    for b in range(B):
        for j in range(pos[b] + 1):
            kc[b, j % C] = kn_all[b, j]
            vc[b, j % C] = v[b, j]
    qn = rope_qknorm_at(q[np.arange(B), pos], pos, 10000.0, 1e-6)
    o, lse = decode_fwd(qn, kc, vc, pos, W, 1.0 / np.sqrt(D))
    for b in range(B):
        np.testing.assert_allclose(o[b], fwd["O"][b, pos[b]], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], fwd["lse"][b, :, pos[b]], rtol=1e-12, atol=1e-12)
