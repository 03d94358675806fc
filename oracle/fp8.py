"""Oracle for the fp8 forward variant: the e4m3 format and attention on fp8 inputs.

TEST INFRASTRUCTURE (see the package docstring).

Passages followed:

* "NanoGPT Speedrun：大模型训练效率的极限竞速指南" (kongchang.com), section "工程与硬件优化",
  its paragraph on bf16 and fp8: fp8 is an 8-bit floating-point format that can double
  matrix throughput over bf16 but needs finer calibration (scales) to stay accurate. The pages fix no fp8 encoding; reading: the OCP
  E4M3 format that gfx950's fp8 matrix instructions read (1 sign, 4 exponent bits with bias
  7, 3 mantissa bits; subnormals; no infinities; S.1111.111 is NaN; largest finite 448).
* Reading (calibration): each of q_hat, k_hat, v is stored as e4m3 codes of x / s with one
  float32 scale s per tensor, x ~= s * decode(code). Encoding rounds to nearest, ties to
  even, and saturates: finite values beyond 448 (and infinities) become +-448, NaN stays NaN.
  The division by s is a float32 multiply by the float32 reciprocal of s, rounded once,
  then one rounding to e4m3.
* The attention itself is the plain definition ("GPT-2 124M 复现" §3) on the decoded,
  rescaled inputs; the fp8 rounding of the probabilities inside a kernel is that kernel's own
  rounding (like the bf16 rounding of P in the bf16 kernels), not part of the definition.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_fwd

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3 code (uint8) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code (ties to even mantissa), saturating to +-448; NaN -> 0x7F | sign."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # exponent of the binade holding a (normal range starts at 2^-6)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e = np.where(np.exp2(e.astype(np.float64)) > a, e - 1, e)
    e = np.where(np.exp2(e + 1.0) <= a, e + 1, e)
    sub = e < -6
    # subnormal: integer multiple of 2^-9 (8 of them is the smallest normal, code 0x08)
    qs = np.rint(a * 2.0 ** 9).astype(np.int64)
    # normal: 8 + mantissa = a / 2^e * 8, rounded to nearest even
    qn = np.rint(a * np.exp2(3.0 - e)).astype(np.int64)
    carry = qn == 16
    e_n = np.where(carry, e + 1, e)
    m_n = np.where(carry, 0, qn - 8)
    code_n = ((e_n + 7) << 3) | m_n
    code = np.where(sub, qs, code_n)
    code = np.where(a == 0, 0, code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of x / scale: float32 product with the float32 reciprocal, then e4m3 rounding."""
    inv = np.float32(1.0) / np.float32(scale)
    y = np.asarray(x, dtype=np.float32) * inv
    return e4m3_encode(y.astype(np.float64))


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    return e4m3_decode(codes) * float(np.float32(scale))


def attention_fwd_fp8(q8: np.ndarray, k8: np.ndarray, v8: np.ndarray, q_scale: float,
                      k_scale: float, v_scale: float, window: int, scale: float, doc_id=None):
    """O (B, T, H, D) and lse (B, H, T) of the attention on the decoded, rescaled codes
    (q8, k8, v8 in the (B, T, H, D) layout)."""
    return attention_fwd(dequantize(q8, q_scale), dequantize(k8, k_scale),
                         dequantize(v8, v_scale), window, scale, doc_id=doc_id)
