"""Pins of the fp8 oracle: the e4m3 decoder and encoder against torch's float8_e4m3fn (the OCP
E4M3 format) over every code and over random and halfway values, saturation and NaN handling
(the reading where torch differs), the calibrated quantiser, and the attention on fp8 inputs
against the plain attention of the decoded values. CPU only."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    assert np.sum(np.isnan(got)) == 2                         # 0x7F and 0xFF
    assert fp8.e4m3_decode(np.uint8(0x7E)) == 448.0           # largest finite
    assert fp8.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6       # smallest normal
    assert fp8.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9       # smallest subnormal


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_encode_matches_torch_on_random_and_halfway_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x[np.abs(x) < 440].astype(np.float32)
    np.testing.assert_array_equal(fp8.e4m3_encode(x), _torch_codes(x))
    # exact midpoints between neighbouring finite codes: ties go to the even mantissa
    pos = fp8.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    nxt = fp8.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    mid = (pos + nxt) / 2
    got = fp8.e4m3_encode(mid)
    np.testing.assert_array_equal(got, _torch_codes(mid))
    assert np.all(got % 2 == 0)
    np.testing.assert_array_equal(fp8.e4m3_encode(-mid), got | 0x80)


def test_saturation_nan_and_zero():
    """Reading: finite values beyond 448 saturate (torch's cast gives NaN there instead)."""
    assert fp8.e4m3_encode(np.array([449.0, 463.9, 1e9, np.inf])).tolist() == [0x7E] * 4
    assert fp8.e4m3_encode(np.array([-500.0, -np.inf])).tolist() == [0xFE] * 2
    assert fp8.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F
    assert fp8.e4m3_encode(np.array([0.0, -0.0])).tolist() == [0x00, 0x80]
    # below half the smallest subnormal rounds to zero, exactly half rounds to even (zero)
    assert fp8.e4m3_encode(np.array([2.0 ** -11, 2.0 ** -10, 1.5 * 2.0 ** -10])).tolist() == [0, 0, 1]


def test_quantize_is_float32_product_then_one_rounding():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(5000).astype(np.float32) * 3
    s = 0.037
    want = _torch_codes(x * (np.float32(1) / np.float32(s)))
    np.testing.assert_array_equal(fp8.quantize(x, s), want)
    back = fp8.dequantize(fp8.quantize(x, s), s)
    # within half an e4m3 ulp (2^-4 relative) of x, away from the subnormal range
    big = np.abs(x / s) > 2.0 ** -6
    assert np.all(np.abs(back - x)[big] <= 2.0 ** -4 * np.abs(x)[big] + 1e-12)


@pytest.mark.parametrize("W", [1, 7, 40])
def test_fp8_attention_is_attention_of_the_decoded_inputs(W):
    B, T, H, D = 2, 40, 2, 16
    rng = np.random.default_rng(W)
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    sq, sk, sv = 0.02, 0.03, 0.05
    q8, k8, v8 = fp8.quantize(q, sq), fp8.quantize(k, sk), fp8.quantize(v, sv)
    o, lse = fp8.attention_fwd_fp8(q8, k8, v8, sq, sk, sv, W, 0.25)
    # independent statement: decode by torch, dense softmax written out here
    dec = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).double() * float(np.float32(s))
    qt, kt, vt = dec(q8, sq), dec(k8, sk), dec(v8, sv)
    s_ = torch.einsum("bihd,bjhd->bhij", qt, kt) * 0.25
    i = torch.arange(T)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    s_ = s_.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s_, -1).numpy(), rtol=1e-12, atol=1e-12)
    ot = torch.einsum("bhij,bjhd->bihd", torch.softmax(s_, -1), vt)
    np.testing.assert_allclose(o, ot.numpy(), rtol=1e-12, atol=1e-12)
    if W == 1:   # a single visible key: O is that key's decoded value row
        np.testing.assert_allclose(o, vt.numpy(), rtol=0, atol=1e-15)
