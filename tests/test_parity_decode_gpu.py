"""GPU parity of sliding-window decoding from a ring K/V cache against the oracle, through the
C ABI: the positional prologue and its cache writes (bitwise the training prologue's rows),
the attention over the cached window (with and without ring wrap, with one and with several
splits of the window), the agreement of a decoding step with the training forward's row, and
invalid positions."""

import numpy as np
import pytest
import torch

from oracle.decode import decode_fwd, rope_qknorm_at
import oracle
from causal_sliding_window_rope_amd import binding as sw
from gpu_helpers import BF16_LSE_ABS, announce, check, dev, host

pytestmark = pytest.mark.gpu


def _rb(a, dtype):
    """Values as the library stores them (bf16 rounding for bf16 runs)."""
    return oracle.round_bf16(a) if dtype == "bf16" else a.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_prologue(dtype, D):
    B, H, cap = 5, 3, 7
    announce("decode prologue", dtype, D)
    rng = np.random.default_rng(D)
    q, k, v = (rng.standard_normal((B, H, D)) for _ in range(3))
    pos = np.array([0, 6, 7, 30, 2], dtype=np.int32)
    cs = sw.rope_table(40, D, 10000.0)
    kc = torch.full((B, cap, H, D), 7.0, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                    device="cuda")
    vc = kc.clone()
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    qn = sw.swa_decode_prologue(tq, tk, tv, cs, torch.from_numpy(pos).cuda(), kc, vc)
    torch.cuda.synchronize()
    qr, kr, vr = host(tq), host(tk), host(tv)
    check("qn", host(qn), rope_qknorm_at(qr, pos, 10000.0, 1e-6), dtype)
    kn = rope_qknorm_at(kr, pos, 10000.0, 1e-6)
    kch, vch = host(kc), host(vc)
    for b in range(B):
        s = pos[b] % cap
        check("k_cache", kch[b, s], kn[b], dtype)
        np.testing.assert_array_equal(vch[b, s], vr[b])
        others = [j for j in range(cap) if j != s]
        assert np.all(kch[b, others] == 7.0) and np.all(vch[b, others] == 7.0)


CASES = [  # B, H, D, cap, W, positions, dtype
    (2, 3, 128, 64, 64, [0, 63], "bf16"),
    (3, 2, 128, 96, 40, [5, 200, 95], "bf16"),        # ring wrap, window < cap
    (4, 12, 128, 1024, 1024, [2047, 1500, 1023, 700], "bf16"),   # several splits
    (2, 2, 64, 300, 300, [1000, 150], "bf16"),
    (2, 3, 64, 50, 17, [3, 120], "f32"),
    (2, 2, 128, 2048, 2048, [2047, 10], "f32"),
    (2, 12, 64, 300, 256, [299, 600], "bf16"),       # all-heads kernel, second load half used
    (2, 16, 128, 200, 128, [150, 7], "bf16"),        # all-heads kernel, four loads per row
    (2, 12, 128, 128, 128, [127, 300], "f32"),       # row of six loads: per-head kernel
    # the d24 decoding step's shape (32 sequences, 12 heads, window 1024 of a 2048-slot ring)
    (32, 12, 128, 2048, 1024, [2047] * 24 + [1023, 1024, 3000, 4095, 0, 15, 16, 17], "bf16"),
]


@pytest.mark.parametrize("B,H,D,cap,W,positions,dtype", CASES)
def test_decode_attention(B, H, D, cap, W, positions, dtype):
    announce("decode", B, H, D, cap, W, positions, dtype)
    rng = np.random.default_rng(B * 100 + cap + W)
    qn = _rb(rng.standard_normal((B, H, D)), dtype)
    kc = _rb(rng.standard_normal((B, cap, H, D)), dtype)
    vc = _rb(rng.standard_normal((B, cap, H, D)), dtype)
    pos = np.array(positions, dtype=np.int32)
    scale = 1.0 / np.sqrt(D)
    o, lse = sw.swa_decode(dev(qn, dtype), dev(kc, dtype), dev(vc, dtype),
                           torch.from_numpy(pos).cuda(), W, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = decode_fwd(qn, kc, vc, pos, W, scale)
    check("o", host(o), o_ref, dtype)
    check("lse", host(lse), lse_ref, dtype, lse=True)


def test_decode_step_matches_training_row():
    """Fill the cache step by step with the decode prologue and decode at several positions;
    the results are row p of the oracle's full-sequence layer (and of swa_fwd)."""
    B, T, H, D, W, cap = 2, 300, 2, 128, 100, 128
    announce("decode vs training row")
    rng = np.random.default_rng(11)
    q, k, v = (oracle.round_bf16(rng.standard_normal((B, T, H, D))) for _ in range(3))
    fwd = oracle.layer_fwd(q, k, v, W, round_boundary=True)
    cs = sw.rope_table(T, D, 10000.0)
    kc = torch.zeros((B, cap, H, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    checked = 0
    for p in range(T):
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        qn = sw.swa_decode_prologue(tq[:, p].contiguous(), tk[:, p].contiguous(),
                                    tv[:, p].contiguous(), cs, pos, kc, vc)
        if p in (0, 1, 99, 100, 200, 299):
            o, lse = sw.swa_decode(qn, kc, vc, pos, W)
            torch.cuda.synchronize()
            check("o", host(o), fwd["O"][:, p], "bf16")
            assert np.max(np.abs(host(lse) - fwd["lse"][:, :, p])) <= BF16_LSE_ABS
            checked += 1
    assert checked == 6


def test_decode_invalid_positions():
    B, H, D, cap = 3, 2, 64, 16
    announce("decode invalid positions")
    cs = sw.rope_table(20, D, 10000.0)
    x = torch.ones((B, H, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.full((B, cap, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    pos = torch.tensor([-1, 25, 4], dtype=torch.int32, device="cuda")   # negative, past the table
    qn = sw.swa_decode_prologue(x, x, x, cs, pos, kc, vc)
    torch.cuda.synchronize()
    assert torch.isnan(qn[0].float()).all() and torch.isnan(qn[1].float()).all()
    assert torch.isfinite(qn[2].float()).all()
    assert (kc[0] == 3.0).all() and (kc[1] == 3.0).all()      # untouched
    assert not (kc[2, 4] == 3.0).all()                         # written
    o, lse = sw.swa_decode(x, kc, vc, torch.tensor([-5, 3, 4], dtype=torch.int32, device="cuda"), 8)
    torch.cuda.synchronize()
    assert torch.isnan(o[0].float()).all() and torch.isfinite(o[1:].float()).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_prologue_matches_training_prologue(dtype, D):
    """The decode prologue's q-hat and k-hat rows are bitwise rope_qknorm_fwd's rows at the same
    positions (a decoding step is row p of the training forward)."""
    B, H, T, cap = 4, 3, 40, 64
    announce("decode prologue vs training prologue", dtype, D)
    rng = np.random.default_rng(100 + D)
    q, k, v = (rng.standard_normal((B, H, D)) for _ in range(3))
    pos = np.array([0, 17, 39, 5], dtype=np.int32)
    cs = sw.rope_table(T, D, 10000.0)
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    kc = torch.zeros((B, cap, H, D), dtype=tq.dtype, device="cuda")
    vc = torch.zeros_like(kc)
    qn = sw.swa_decode_prologue(tq, tk, tv, cs, torch.from_numpy(pos).cuda(), kc, vc)
    xq = torch.zeros((B, T, H, D), dtype=tq.dtype, device="cuda")
    xk = torch.zeros_like(xq)
    for b in range(B):
        xq[b, pos[b]] = tq[b]
        xk[b, pos[b]] = tk[b]
    tqn, tkn = sw.rope_qknorm_fwd(xq, xk, cs)
    torch.cuda.synchronize()
    for b in range(B):
        assert torch.equal(qn[b], tqn[b, pos[b]])
        assert torch.equal(kc[b, pos[b] % cap], tkn[b, pos[b]])
        assert torch.equal(vc[b, pos[b] % cap], tv[b])

