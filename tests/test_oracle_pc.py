"""Pins of the oracle's per-output-channel FP8 scheme (oracle/pc_oracle.py):
hand-worked rows, exact rational checks of both FP32 divisions, invariants,
special rows, and the contraction against exact arithmetic.

Sources: "Wan2.2 I2V A14B, four-step 720p: native LightX2V FP8 and NVFP4",
section "Conversion and compatibility" (E4M3 weights, per-output-channel FP32
scales, nearest rounding); "Model Quantization Techniques" (LightX2V), mode
table (channel-symmetric FP8 weights, channel-dynamic-symmetric FP8
activations), the row rule scale = max(abs(x)) / qmax, and qmax 448 with FP32
accumulation (Conv3D mode table).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def nearest_f32(q, value):
    """True if float32 q is a float32 nearest to the exact rational value."""
    q = np.float32(q)
    lo, hi = np.nextafter(q, np.float32(-np.inf)), np.nextafter(q, np.float32(np.inf))
    d = abs(Fraction(float(q)) - value)
    return d <= abs(Fraction(float(lo)) - value) and d <= abs(Fraction(float(hi)) - value)


def test_worked_row_power_of_two_scale():
    # amax 3.5: scale 3.5 / 448 = 2**-7 exactly. 1.0 * 2**7 = 128 = 2**7:
    # exponent field 14, mantissa 0 -> 0x70. -0.5 -> -64 = -2**6 -> 0x68 | 0x80.
    # 3.5 -> 448 = 1.75 * 2**8 -> 0x7E. 0 -> 0x00.
    q, s = oracle.quantize_pc(np.array([[1.0, -0.5, 3.5, 0.0]]))
    assert s[0] == np.float32(2.0**-7)
    assert list(q[0]) == [0x70, 0xE8, 0x7E, 0x00]


def test_worked_row_general_scale():
    # amax 1.0: scale = fp32(1/448). 1.0 / scale is 448 within an fp32 ulp ->
    # 448 (or saturated) -> 0x7E. 0.3 / scale = 134.4 (within fp32 rounding):
    # E4M3 spacing in [128, 256) is 16, 134.4 is nearer 128 -> 0x70.
    q, s = oracle.quantize_pc(np.array([[1.0, 0.3]], dtype=np.float32))
    assert s[0] == np.float32(1.0) / np.float32(448.0)
    assert list(q[0]) == [0x7E, 0x70]


def test_scale_and_quotient_are_the_nearest_float32():
    # Both divisions are checked against exact rational arithmetic, not
    # against numpy's float32 division.
    x = synth.make_activation(6, 64, seed=3).float().numpy()
    w = synth.make_weight(4, 64, seed=3).numpy()
    for a in (x, w):
        q, s = oracle.quantize_pc(a)
        for r in range(a.shape[0]):
            amax = max(abs(Fraction(float(v))) for v in a[r])
            assert nearest_f32(s[r], amax / 448)
            for k in range(0, a.shape[1], 7):
                quot = Fraction(float(a[r, k])) / Fraction(float(s[r]))
                # the code is the E4M3 encoding of the nearest float32 quotient
                cands = [np.float32(float(quot))]
                cands += [np.nextafter(cands[0], np.float32(-np.inf)), np.nextafter(cands[0], np.float32(np.inf))]
                best = [c for c in cands if nearest_f32(c, quot)]
                assert int(q[r, k]) in {int(oracle.e4m3_encode(np.float64(c))) for c in best}


def test_row_maximum_encodes_to_448():
    x = synth.make_activation(64, 256, seed=5).float().numpy()
    q, s = oracle.quantize_pc(x)
    i = np.argmax(np.abs(x), axis=1)
    assert np.all((q[np.arange(64), i] & 0x7F) == 0x7E)
    assert np.all(s > 0)


def test_power_of_two_equivariance_and_sign_symmetry():
    x = synth.make_activation(8, 128, seed=7).float().numpy()
    q, s = oracle.quantize_pc(x)
    for k in (-20, -3, 5, 30):
        q2, s2 = oracle.quantize_pc(x * np.float32(2.0**k))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0**k))
    qn, sn = oracle.quantize_pc(-x)
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)


def test_error_bound():
    # |dec(q) s - x| <= (half an E4M3 step at |x/s| + the quotient's fp32
    # rounding) * s; E4M3 steps: 2**(floor(log2 v) - 3) for v >= 2**-6, 2**-9 below.
    w = synth.make_weight(16, 512, seed=9).numpy()
    q, s = oracle.quantize_pc(w)
    v = np.abs(w / s[:, None].astype(np.float64))
    step = np.where(v >= 2.0**-6, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0**-6))) - 3), 2.0**-9)
    err = np.abs(oracle.dequantize_pc(q, s) - w)
    assert np.all(err <= (step / 2 + v * 2.0**-23) * s[:, None])


def test_special_rows():
    x = np.array([[0.0, -0.0, 0.0, 0.0], [1.0, np.inf, 0.0, 2.0], [1.0, np.nan, 0.0, 2.0], [1e-45, -1e-45, 0, 0]],
                 dtype=np.float32)
    q, s = oracle.quantize_pc(x)
    assert list(q[0]) == [0x00, 0x80, 0x00, 0x00] and s[0] == 0
    assert np.all(q[1] == 0x7F) and np.isnan(s[1])
    assert np.all(q[2] == 0x7F) and np.isnan(s[2])
    # amax 2**-149 / 448 underflows to a zero scale: signed zeros
    assert list(q[3]) == [0x00, 0x80, 0x00, 0x00] and s[3] == 0


def test_linear_exact_on_tiny_shapes():
    rng = np.random.default_rng(11)
    xq = rng.integers(0, 256, (3, 64)).astype(np.uint8)
    wq = rng.integers(0, 256, (2, 64)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x01  # no NaN codes
    wq[(wq & 0x7F) == 0x7F] = 0x02
    xs = np.array([0.5, 2.0**-7, 3.0], dtype=np.float32)
    ws = np.array([np.float32(1 / 448), np.float32(0.25)], dtype=np.float32)
    bias = np.array([0.5, -1.25])
    y, S = oracle.linear_pc_ref(xq, xs, wq, ws, bias=bias)
    dec = lambda c: Fraction(float(oracle.e4m3_decode(np.uint8(c))))  # noqa: E731
    for m in range(3):
        for n in range(2):
            exact = sum(dec(xq[m, k]) * dec(wq[n, k]) for k in range(64))
            want = Fraction(float(xs[m])) * Fraction(float(ws[n])) * exact + Fraction(bias[n])
            assert abs(Fraction(y[m, n]) - want) <= Fraction(2.0**-40) * (1 + abs(want))
            sabs = sum(abs(dec(xq[m, k]) * dec(wq[n, k])) for k in range(64))
            assert abs(Fraction(S[m, n]) - abs(Fraction(float(xs[m])) * Fraction(float(ws[n]))) * sabs) <= Fraction(
                2.0**-40) * (1 + sabs)


def test_linear_diagonal_weights():
    # W = diag(c): row n's only nonzero is c_n, so its scale is c_n / 448 and
    # its code 0x7E (448). Then y[m, n] = xs[m] dec(xq[m, n]) * 448 * ws[n].
    c = np.array([0.5, -2.0, 3.0, 0.125] * 16, dtype=np.float32)
    W = np.diag(c)
    wq, ws = oracle.quantize_pc(W)
    assert np.all((wq[np.arange(64), np.arange(64)] & 0x7F) == 0x7E)
    x = synth.make_activation(5, 64, seed=2).float().numpy()
    xq, xs = oracle.quantize_pc(x)
    y, _ = oracle.linear_pc_ref(xq, xs, wq, ws)
    want = oracle.dequantize_pc(xq, xs) * (448.0 * ws.astype(np.float64) * np.sign(c))[None, :]
    assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_gelu_epilogue_and_bias():
    x = synth.make_activation(4, 128, seed=4).float().numpy()
    w = synth.make_weight(8, 128, seed=4).numpy()
    b = synth.make_bias(8, seed=4).double().numpy()
    xq, xs = oracle.quantize_pc(x)
    wq, ws = oracle.quantize_pc(w)
    y0, S = oracle.linear_pc_ref(xq, xs, wq, ws, bias=b)
    y1, S1 = oracle.linear_pc_ref(xq, xs, wq, ws, bias=b, epilogue="gelu_tanh")
    assert np.array_equal(S, S1)
    assert np.allclose(y1, oracle.gelu_tanh(y0), rtol=0, atol=0)
    assert np.all(S >= np.abs(y0 - b[None, :]) * (1 - 1e-12))
    with pytest.raises(ValueError):
        oracle.linear_pc_ref(xq, xs, wq, ws, epilogue="relu")
