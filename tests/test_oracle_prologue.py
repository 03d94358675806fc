"""Pins of the oracle's RoPE and RMS QK-norm against facts that do not come from the oracle.

Runs on the CPU only (no ``gpu`` marker).
"""

import math

import numpy as np
import pytest
import scipy.linalg
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- RoPE

def test_rope_hand_values_pairing_and_frequencies():
    """Hand-evaluated case, D=4, base=100: theta_0 = 1, theta_1 = 100^(-2/4) = 0.1.

    Pairs are (0, 2) and (1, 3); at position t the pair (x_i, x_{i+2}) turns by
    t * theta_i counter-clockwise. A wrong pairing (interleaved), a wrong sign or
    a wrong frequency exponent fails here.
    """
    x = np.zeros((1, 4, 1, 4))
    x[0, 3, 0] = [1.0, 2.0, 3.0, 4.0]          # t = 3: angles 3 and 0.3
    y = oracle.rope(x, base=100.0)[0, 3, 0]
    c3, s3, c03, s03 = math.cos(3.0), math.sin(3.0), math.cos(0.3), math.sin(0.3)
    want = [1.0 * c3 - 3.0 * s3, 2.0 * c03 - 4.0 * s03, 1.0 * s3 + 3.0 * c3, 2.0 * s03 + 4.0 * c03]
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-14)
    # position 0 is the identity, rows at other positions are untouched by position 3's angles
    np.testing.assert_array_equal(oracle.rope(x, base=100.0)[0, :3], 0.0)


def test_rope_equals_matrix_exponential_of_generator():
    """R_t = expm(t * G) with G the block-diagonal generator of the pair rotations.

    scipy's expm is an independent routine; this pins cos/sin placement for all D/2 pairs.
    """
    D, T, base = 8, 6, 10000.0
    x = _rand((1, T, 1, D), 1)
    y = oracle.rope(x, base)
    for t in range(T):
        G = np.zeros((D, D))
        for i in range(D // 2):
            th = base ** (-2.0 * i / D)
            G[i + D // 2, i] = th      # d/dt y_{i+D/2} = +theta * y_i
            G[i, i + D // 2] = -th
        R = scipy.linalg.expm(t * G)
        np.testing.assert_allclose(y[0, t, 0], R @ x[0, t, 0], rtol=0, atol=1e-12)


def test_rope_norm_preserving_and_relative_position():
    D, T = 16, 40
    x = _rand((2, T, 3, D), 2)
    y = oracle.rope(x, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])
    # q at position t and k at position s: the rotated dot product depends on t - s only
    q, k = _rand(D, 3), _rand(D, 4)
    X = np.zeros((1, T, 2, D))
    X[0, :, 0] = q
    X[0, :, 1] = k
    Y = oracle.rope(X, 10000.0)[0]
    for (t, s, c) in [(5, 2, 7), (10, 10, 20), (3, 9, 30)]:
        a = Y[t, 0] @ Y[s, 1]
        b = Y[t + c, 0] @ Y[s + c, 1]
        assert abs(a - b) < 1e-11


def test_rope_transpose_is_inverse_and_adjoint():
    x, g = _rand((1, 20, 2, 8), 5), _rand((1, 20, 2, 8), 6)
    np.testing.assert_allclose(oracle.rope_transpose(oracle.rope(x, 1e4), 1e4), x, atol=1e-13)
    # <R x, g> = <x, R^T g>
    assert abs(np.sum(oracle.rope(x, 1e4) * g) - np.sum(x * oracle.rope_transpose(g, 1e4))) < 1e-11


# ---------------------------------------------------------------- RMS norm

def test_rms_norm_matches_torch_rms_norm():
    u = _rand((2, 7, 3, 16), 7) * 3.0
    xh, r = oracle.rms_norm(u, 1e-6)
    ref = F.rms_norm(torch.from_numpy(u), (16,), eps=1e-6).numpy()
    np.testing.assert_allclose(xh, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r[..., 0], 1.0 / np.sqrt(np.mean(u * u, -1) + 1e-6), rtol=1e-14)


def test_qknorm_unit_rms_per_head():
    """mean_d(x_hat^2) = m / (m + eps) with m = mean_d(u^2): ~1 per (token, head)."""
    u = _rand((2, 9, 4, 64), 8)
    xh, _ = oracle.rope_qknorm(u, 10000.0, 1e-6)
    m = np.mean(oracle.rope(u, 10000.0) ** 2, -1)
    np.testing.assert_allclose(np.mean(xh ** 2, -1), m / (m + 1e-6), rtol=1e-13)
    assert np.all(np.abs(np.mean(xh ** 2, -1) - 1.0) < 1e-5)


def test_rms_norm_bwd_matches_torch_autograd():
    u = _rand((1, 5, 2, 16), 9)
    g = _rand((1, 5, 2, 16), 10)
    ut = torch.from_numpy(u).requires_grad_(True)
    F.rms_norm(ut, (16,), eps=1e-6).backward(torch.from_numpy(g))
    xh, r = oracle.rms_norm(u, 1e-6)
    np.testing.assert_allclose(oracle.rms_norm_bwd(xh, r, g), ut.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_rope_then_norm_commutes_with_norm_then_rope():
    u = _rand((1, 11, 2, 32), 11)
    a, _ = oracle.rms_norm(oracle.rope(u, 1e4), 1e-6)
    b = oracle.rope(oracle.rms_norm(u, 1e-6)[0], 1e4)
    np.testing.assert_allclose(a, b, atol=1e-14)


@pytest.mark.parametrize("seed", [12, 13])
def test_prologue_bwd_finite_differences(seed):
    B, T, H, D = 1, 5, 2, 8
    x = _rand((B, T, H, D), seed)
    g = _rand((B, T, H, D), seed + 100)
    grad = oracle.rope_qknorm_bwd(x, g, 1e4, 1e-6)
    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fp = np.sum(oracle.rope_qknorm(xp, 1e4, 1e-6)[0] * g)
        fm = np.sum(oracle.rope_qknorm(xm, 1e4, 1e-6)[0] * g)
        fd[idx] = (fp - fm) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


def test_round_bf16_matches_torch_cast():
    a = np.concatenate([_rand(10000, 14) * 10.0 ** k for k in range(-3, 4)])
    # exact ties: a bf16 value plus half an ulp must round to even
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7)])
    a = np.concatenate([a, ties])
    want = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(a), want)
