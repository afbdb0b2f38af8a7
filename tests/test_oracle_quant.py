"""Pins of the oracle's MX group quantization (shared E8M0 scale per 32
elements along K, E4M3 elements), from closed forms, hand-worked groups,
invariants and exact brute force.

Source: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
section "Quantization Details" (group_size 32, sym, E4M3 + E8M0). The shared
exponent rule floor(log2 amax) - 8 is the OCP MX conversion (external).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def group(vals):
    g = np.zeros(32)
    g[: len(vals)] = vals
    return g[None, :]


def test_worked_group_three():
    # amax 3.0: floor(log2 3) = 1, e = 1 - 8 = -7, scale code 120.
    # 3.0 * 2**7 = 384 = 1.5 * 2**8 -> exponent field 15, mantissa 4 -> 0x7C.
    # -0.3 * 2**7 = -38.4 = -1.2 * 2**5; 1.2 lies between 1.125 and 1.25 and
    # is nearer 1.25 -> exponent field 12, mantissa 2 -> 0x62 | 0x80 = 0xE2.
    q, s = oracle.quantize_mx(group([3.0, -0.3, 0.0, -0.0]))
    assert s.tolist() == [[120]]
    assert q[0, :4].tolist() == [0x7C, 0xE2, 0x00, 0x80]
    assert np.all(q[0, 4:] == 0)


def test_worked_group_saturating():
    # amax 500: floor(log2 500) = 8, e = 0, scale code 127; 500 > 448 so it
    # saturates to 0x7E; 1.0 stays 0x38.
    q, s = oracle.quantize_mx(group([500.0, 1.0]))
    assert s.tolist() == [[127]]
    assert q[0, :2].tolist() == [0x7E, 0x38]


def test_worked_group_subnormal_input_is_not_flushed():
    # bf16 2**-130 alone: floor(log2) - 8 = -138 clamps to -127 (code 0);
    # 2**-130 * 2**127 = 2**-3 = 1.0 * 2**-3 -> exponent field 4 -> 0x20.
    q, s = oracle.quantize_mx(group([2.0**-130]))
    assert s.tolist() == [[0]]
    assert q[0, 0] == 0x20


def test_zero_group_maps_to_zero():
    q, s = oracle.quantize_mx(np.zeros((3, 64)))
    assert np.all(s == 0) and np.all(q == 0)
    z = np.zeros((1, 32))
    z[0, 5] = -0.0
    q, s = oracle.quantize_mx(z)
    assert q[0, 5] == 0x80 and s[0, 0] == 0
    assert np.all(oracle.dequantize_mx(q, s) == 0)


def test_nonfinite_group_fails_closed_and_stays_local():
    x = np.ones((2, 96))
    x[0, 40] = np.nan
    x[1, 70] = -np.inf
    q, s = oracle.quantize_mx(x)
    assert s.tolist() == [[127 - 8, 255, 127 - 8], [127 - 8, 127 - 8, 255]]
    assert np.all(q[0, 32:64] == 0x7F) and np.all(q[1, 64:96] == 0x7F)
    assert np.all(q[0, :32] == 0x78) and np.all(q[1, :64] == 0x78)
    assert np.all(np.isnan(oracle.dequantize_mx(q, s)[0, 32:64]))


def _bf16_like(rng, shape, outliers=True):
    v = rng.standard_normal(shape)
    if outliers:
        v = np.where(rng.random(shape) < 1e-3, v * 50, v)
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()


def test_scale_rule_by_exact_search():
    # Independent of frexp: the shared exponent e is the unique integer with
    # 2**(e+8) <= amax < 2**(e+9), found by search in exact rationals, then
    # clamped to [-127, 127].
    rng = np.random.default_rng(5)
    x = _bf16_like(rng, (64, 32 * 8)) * np.exp2(rng.integers(-140, 120, size=(64, 1)))
    _, s = oracle.quantize_mx(x)
    amax = np.max(np.abs(x.reshape(64, 8, 32)), axis=-1)
    for (i, j), a in np.ndenumerate(amax):
        fa = Fraction(float(a))
        e = 0
        while Fraction(2) ** (e + 8) > fa:
            e -= 1
        while Fraction(2) ** (e + 9) <= fa:
            e += 1
        assert s[i, j] == max(e, -127) + 127


def test_invariants_random_groups():
    rng = np.random.default_rng(7)
    x = _bf16_like(rng, (512, 1024)) * np.exp2(rng.integers(-30, 30, size=(512, 1)))
    q, s = oracle.quantize_mx(x)
    xh = oracle.dequantize_mx(q, s)
    assert np.all(s != 0xFF) and np.all(s > 0)
    g = x.reshape(512, 32, 32)
    gh = xh.reshape(512, 32, 32)
    amax = np.max(np.abs(g), axis=-1)
    # |xhat| <= 2 * amax everywhere; scale is a power of two by construction.
    assert np.all(np.abs(gh) <= 2 * amax[..., None])
    # The group max lands in the top E4M3 binade: magnitude code 0x78..0x7E,
    # and its dequantized value is within [0.875, 1.0625] * amax.
    i = np.argmax(np.abs(g), axis=-1)
    qg = q.reshape(512, 32, 32)
    top = np.take_along_axis(qg, i[..., None], -1)[..., 0] & 0x7F
    assert np.all((top >= 0x78) & (top <= 0x7E))
    ratio = np.abs(np.take_along_axis(gh, i[..., None], -1)[..., 0]) / amax
    assert np.all((ratio >= 0.875) & (ratio <= 1.0625))
    # Per-element error: at most half an E4M3 step at the element's binade,
    # i.e. 2**-4 relative in the normal range, 2**-10 * 2**e below it.
    e = s.astype(np.int64)[..., None] - 127
    err = np.abs(gh - g)
    bound = np.maximum(np.abs(g) * 2.0**-4, np.ldexp(1.0, e - 10))
    # Saturated elements (above 448 * 2**e, below 512 * 2**e) lose < 1/8.
    bound = np.where(np.abs(g) > np.ldexp(448.0, e), np.abs(g) / 8, bound)
    assert np.all(err <= bound)
    # Signs survive (zeros aside).
    nz = gh != 0
    assert np.all(np.sign(gh[nz]) == np.sign(g[nz]))


def test_power_of_two_equivariance():
    rng = np.random.default_rng(11)
    x = _bf16_like(rng, (64, 256))
    q0, s0 = oracle.quantize_mx(x)
    for k in (-20, -3, 1, 17):
        qk, sk = oracle.quantize_mx(np.ldexp(x, k))
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_sign_symmetry():
    rng = np.random.default_rng(13)
    x = _bf16_like(rng, (32, 128))
    q, s = oracle.quantize_mx(x)
    qn, sn = oracle.quantize_mx(-x)
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ 0x80)


def test_rows_are_independent():
    rng = np.random.default_rng(17)
    x = _bf16_like(rng, (40, 160))
    q, s = oracle.quantize_mx(x)
    for r in (0, 13, 39):
        qr, sr = oracle.quantize_mx(x[r : r + 1])
        assert np.array_equal(qr[0], q[r]) and np.array_equal(sr[0], s[r])


def test_bad_k_rejected():
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.zeros((2, 48)))
