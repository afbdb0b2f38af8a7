"""Pins of the oracle's contraction, bias, GELU-tanh epilogue, bf16 rounding
and acceptance rule.

Sources: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
section "Quantization Details" (W8A8 MXFP8 linears with F16 biases);
"Model Quantization Techniques", Conv3D mode table (FP32 accumulation).
Independent references: exact rational arithmetic over codes decoded by
torch, special cases that reduce to the quantizer, torch's GELU (tanh form)
and its float32 -> bfloat16 cast.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def torch_dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def rand_bf16(rng, shape, scale=1.0):
    v = rng.standard_normal(shape) * scale
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 5, 64), (5, 2, 96), (4, 4, 32)])
def test_exact_rational_contraction(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = rand_bf16(rng, (M, K))
    w = rand_bf16(rng, (N, K), 0.02)
    b = torch.from_numpy(rng.standard_normal(N) * 0.01).to(torch.float16).to(torch.float64).numpy()
    xq, xs = oracle.quantize_mx(x)
    wq, ws = oracle.quantize_mx(w)
    y, S = oracle.linear_ref(xq, xs, wq, ws, bias=b)
    xd, wd = torch_dec(xq), torch_dec(wq)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            sabs = Fraction(0)
            for k in range(K):
                sa = Fraction(2) ** (int(xs[m, k // 32]) - 127)
                sb = Fraction(2) ** (int(ws[n, k // 32]) - 127)
                t = Fraction(float(xd[m, k])) * sa * Fraction(float(wd[n, k])) * sb
                acc += t
                sabs += abs(t)
            exact = acc + Fraction(float(b[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= K * Fraction(2) ** -52 * (sabs + abs(Fraction(float(b[n]))))
            assert abs(Fraction(float(S[m, n])) - sabs) <= K * Fraction(2) ** -52 * sabs


def test_identity_weight_returns_dequantized_input():
    # W = I: each weight row is one-hot; its group holding the 1 has amax 1,
    # scale 2**-8 (code 119) and the 1 encodes as 0x78 (256); other groups are zero.
    # Then y = xhat exactly, and xhat has at most 4 significant bits.
    rng = np.random.default_rng(3)
    K = 128
    x = rand_bf16(rng, (7, K)) * np.exp2(rng.integers(-8, 8, size=(7, 1)))
    wq, ws = oracle.quantize_mx(np.eye(K))
    diag_group = (np.arange(K)[:, None] // 32) == np.arange(K // 32)[None, :]
    assert np.all(ws[diag_group] == 119) and np.all(ws[~diag_group] == 0)
    assert np.all(wq[np.eye(K, dtype=bool)] == 0x78)
    xq, xs = oracle.quantize_mx(x)
    y, S = oracle.linear_ref(xq, xs, wq, ws)
    xh = oracle.dequantize_mx(xq, xs)
    assert np.array_equal(y, xh)
    assert np.array_equal(S, np.abs(xh))
    assert np.array_equal(oracle.bf16_round(xh), xh)


def test_single_group_closed_form():
    # K = 32: y = 2**(ea + ew) * sum_j dec(qa_j) * dec(qw_j).
    rng = np.random.default_rng(4)
    x = rand_bf16(rng, (2, 32), 3.0)
    w = rand_bf16(rng, (3, 32), 0.05)
    xq, xs = oracle.quantize_mx(x)
    wq, ws = oracle.quantize_mx(w)
    y, _ = oracle.linear_ref(xq, xs, wq, ws)
    for m in range(2):
        for n in range(3):
            dot = float(np.sum(torch_dec(xq[m]) * torch_dec(wq[n])))  # exact: few bits
            want = np.ldexp(dot, int(xs[m, 0]) + int(ws[n, 0]) - 254)
            assert y[m, n] == want


def test_zero_rows_give_bias():
    rng = np.random.default_rng(8)
    x = rand_bf16(rng, (4, 64))
    x[2:] = 0.0
    w = rand_bf16(rng, (5, 64), 0.02)
    b = torch.from_numpy(rng.standard_normal(5) * 0.01).to(torch.float16).to(torch.float64).numpy()
    y, S = oracle.linear_ref(*oracle.quantize_mx(x), *oracle.quantize_mx(w), bias=b)
    assert np.array_equal(y[2:], np.broadcast_to(b, (2, 5)))
    assert np.all(S[2:] == 0)
    yg, _ = oracle.linear_ref(*oracle.quantize_mx(x), *oracle.quantize_mx(w), bias=b, epilogue="gelu_tanh")
    assert np.allclose(yg[2:], oracle.gelu_tanh(np.broadcast_to(b, (2, 5))), rtol=0, atol=0)


def test_gelu_tanh_matches_torch_and_identities():
    v = np.linspace(-12, 12, 100001)
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    assert np.allclose(oracle.gelu_tanh(v), ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(0.0) == 0.0
    # gelu(v) - gelu(-v) = v for the tanh form.
    assert np.allclose(oracle.gelu_tanh(v) - oracle.gelu_tanh(-v), v, rtol=1e-13, atol=1e-13)
    # Largest slope is about 1.1290, below the 1.13 used in the tolerance.
    slope = np.diff(oracle.gelu_tanh(v)) / np.diff(v)
    assert 1.128 < slope.max() < oracle.mx_oracle.GELU_SLOPE_MAX


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(21)
    v = (rng.standard_normal(200_000) * np.exp2(rng.integers(-140, 120, size=200_000))).astype(np.float32)
    v = v[np.isfinite(v)].astype(np.float64)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v), ref)


def test_bf16_ulp_closed_forms():
    u = oracle.bf16_ulp
    assert u(1.0) == 2.0**-7
    assert u(1.99) == 2.0**-7
    assert u(2.0) == 2.0**-6
    assert u(-3.0) == 2.0**-6
    assert u(0.0) == 2.0**-133
    assert u(2.0**-126) == 2.0**-133
    assert u(2.0**-130) == 2.0**-133


def test_tolerance_rule():
    S = np.array([0.0, 100.0])
    y = np.array([0.5, 0.5])
    t = oracle.tolerance(S, y)
    assert t[0] == 2.0**-8 and t[1] == 0.1 + 2.0**-8
    tg = oracle.tolerance(S, y, "gelu_tanh")
    assert np.isclose(tg[1], 0.113 + 2.0**-8)
