"""Pins of the oracle's E4M3 / E8M0 codecs against things other than itself.

Sources: the model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
OptRTN)", section "Quantization Details" (FP8 E4M3 elements, E8M0 scales),
and "Model Quantization Techniques", the Conv3D mode table (E4M3 range 448).
Independent references used here: torch's own float8_e4m3fn / float8_e8m0fnu
dtypes (a library decoder and a library round-to-nearest-even encoder), exact
rational arithmetic, and closed-form values.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_constants.json")
ALL = np.arange(256, dtype=np.uint8)


def torch_e4m3_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(v):
    """torch's float64 -> float8_e4m3fn cast: round to nearest even, no
    saturation (so only valid for |v| <= 448)."""
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_all_codes():
    mine = oracle.e4m3_decode(ALL)
    ref = torch_e4m3_decode(ALL)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_closed_forms():
    d = oracle.e4m3_decode
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0
    assert d(0x08) == 2.0**-6  # smallest normal
    assert d(0x07) == 0.013671875  # largest subnormal, 7/8 * 2**-6
    assert d(0x01) == 2.0**-9  # smallest subnormal
    assert d(0x78) == 256.0  # bottom of the top binade
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    pos = oracle.e4m3_decode(np.arange(127))
    assert np.all(np.diff(pos) > 0)
    finite = oracle.e4m3_decode(ALL)
    finite = finite[~np.isnan(finite)]
    assert len(set(finite.tolist())) == 253  # 126 positive, 126 negative, zero


def test_e4m3_max_is_the_pages_qmax():
    g = json.load(open(GOLDEN))
    assert oracle.E4M3_MAX == g["e4m3_fp32_accum"]["weight_qmax"] == g["e4m3_fp32_accum"]["activation_qmax"]
    assert np.nanmax(oracle.e4m3_decode(ALL)) == oracle.E4M3_MAX
    assert oracle.GROUP == g["quantization_config"]["group_size"] == g["quantization_config"]["act_group_size"]
    assert g["formats"]["scale_every"] == oracle.GROUP


def test_e8m0_decode_matches_torch_all_codes():
    mine = oracle.e8m0_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])
    assert oracle.e8m0_decode(127) == 1.0
    assert oracle.e8m0_decode(0) == 2.0**-127
    assert oracle.e8m0_decode(254) == 2.0**127


def test_e4m3_encode_roundtrip_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert len(codes) == 254
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_e4m3_encode_midpoints_go_to_even_code():
    pos = torch_e4m3_decode(np.arange(127))
    mids = (pos[:-1] + pos[1:]) / 2  # exact in float64
    lo_codes = np.arange(126)
    want = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1).astype(np.uint8)
    assert np.array_equal(oracle.e4m3_encode(mids), want)
    assert np.array_equal(oracle.e4m3_encode(-mids), want | 0x80)
    # The library encoder agrees on all 252 ties.
    assert np.array_equal(torch_e4m3_encode(mids), want)
    assert np.array_equal(torch_e4m3_encode(-mids), want | 0x80)


def test_e4m3_encode_worked_ties():
    # 272 lies halfway between 256 (0x78) and 288 (0x79): even code 0x78.
    # 304 lies halfway between 288 (0x79) and 320 (0x7A): even code 0x7A.
    # 2**-10 is halfway between 0 and 2**-9: even code 0x00.
    # 3 * 2**-10 is halfway between 2**-9 (0x01) and 2**-8 (0x02): 0x02.
    got = oracle.e4m3_encode([272.0, 304.0, 2.0**-10, 3 * 2.0**-10])
    assert got.tolist() == [0x78, 0x7A, 0x00, 0x02]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1234)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), size=200_000))
    v = mag * rng.choice([-1.0, 1.0], size=mag.shape)
    # torch casts float64 through float32 first, so keep to values that are
    # exact in float32 (the layer's inputs are bf16 or fp32 anyway).
    v = np.clip(v, -448.0, 448.0).astype(np.float32).astype(np.float64)
    assert np.array_equal(oracle.e4m3_encode(v), torch_e4m3_encode(v))


def test_e4m3_encode_saturates_and_keeps_sign():
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 511.0, 1e30, np.inf])
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(np.nan) == 0x7F


def _fraction_encode(v):
    """Independent encoder: exhaustive nearest search in exact rationals
    over the magnitudes that torch decodes, ties to the even code."""
    a = min(abs(Fraction(v)), Fraction(448))
    mags = [Fraction(float(m)) for m in torch_e4m3_decode(np.arange(127))]
    best = None
    for code, m in enumerate(mags):
        d = abs(a - m)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    code = best[1]
    if np.signbit(v):
        code |= 0x80
    return code


def test_e4m3_encode_fraction_bruteforce():
    rng = np.random.default_rng(99)
    vals = list(np.exp2(rng.uniform(-12, 9.5, size=300)) * rng.choice([-1, 1], size=300))
    vals += [0.0, -0.0, 2.0**-10, 2.0**-9 * 1.5, 0.0146484375, 447.9, 448.1, 500.0]
    mine = oracle.e4m3_encode(np.array(vals))
    for v, c in zip(vals, mine):
        assert c == _fraction_encode(v), v


@pytest.mark.parametrize("k", range(-20, 20))
def test_e8m0_code_is_exponent_of_power_of_two(k):
    # A group whose largest magnitude is exactly 2**(k+8) has shared
    # exponent k, i.e. code k + 127, and its max element maps to 256.
    assert oracle.mx_scale_code(2.0 ** (k + 8)) == k + 127
