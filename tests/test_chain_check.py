"""Pins of the chain check the GPU tests use for ffn.net.0.proj -> requantize
-> ffn.net.2 (tests/helpers.py: requant_range, assert_requant_valid,
assert_chain_close).

The check must accept every result a correct device could give (an fp32
result within the stated radius of the exact value, then bf16 rounding, then
the MX rule) and reject plausible mistakes: a changed code the oracle fixes, a
wrong scale, a second linear off by more than its allowance, or wrong weights.
The "device" here is simulated on the CPU from the oracle itself.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import CHAIN_RADIUS, assert_chain_close, assert_requant_valid, quant_ref, requant_range


def chain_case(seed=3, M=6, K=256, N1=128, N2=64):
    x = synth.make_activation(M, K, seed)
    w1, b1 = synth.make_weight(N1, K, seed), synth.make_bias(N1, seed).double().numpy()
    w2, b2 = synth.make_weight(N2, N1, seed + 1), synth.make_bias(N2, seed + 1).double().numpy()
    y1, S1 = oracle.linear_ref(*quant_ref(x), *quant_ref(w1), bias=b1, epilogue="gelu_tanh")
    return y1, S1, quant_ref(w2), b2


def device_like(y1, S1, w2, b2, seed=0, frac=0.9):
    """A result a correct device could give: each fp32 output within
    frac * radius of the exact value, rounded to bf16, quantized by the MX
    rule; the second linear within half its tolerance, rounded to bf16."""
    rng = np.random.default_rng(seed)
    r = CHAIN_RADIUS * oracle.GELU_SLOPE_MAX * S1
    h = oracle.bf16_round(y1 + rng.uniform(-frac, frac, y1.shape) * r)
    hq, hs = oracle.quantize_mx(h)
    y2, S2 = oracle.linear_ref(hq, hs, *w2, bias=b2)
    y2 = oracle.bf16_round(y2 + rng.uniform(-0.5, 0.5, y2.shape) * 1e-3 * S2)
    return hq, hs, y2


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_accepts_results_within_the_radius(seed):
    y1, S1, w2, b2 = chain_case()
    hq, hs, y2 = device_like(y1, S1, w2, b2, seed=seed)
    rng = requant_range(y1, S1, "gelu_tanh")
    assert_requant_valid(hq, hs, rng)
    assert_chain_close(y2, y1, S1, "gelu_tanh", *w2, b2)


def test_exact_result_gives_the_oracle_codes():
    y1, S1, w2, b2 = chain_case()
    rng = requant_range(y1, S1, "gelu_tanh")
    hq, hs = oracle.quantize_mx(oracle.bf16_round(y1))
    assert np.array_equal(hq, rng["codes"]) and np.array_equal(hs, rng["scales"])
    assert ((rng["slo"] <= hs) & (hs <= rng["shi"])).all()
    # most codes are fixed, and a fixed code's range is its own value
    assert rng["fixed"].mean() > 0.3
    v = oracle.dequantize_mx(hq, hs)
    assert np.array_equal(rng["qlo"][rng["fixed"]], v[rng["fixed"]])


def test_rejects_a_changed_fixed_code():
    y1, S1, w2, b2 = chain_case()
    rng = requant_range(y1, S1, "gelu_tanh")
    hq, hs, _ = device_like(y1, S1, w2, b2)
    i = np.argwhere(rng["fixed"] & (np.abs(oracle.dequantize_mx(hq, hs)) > 0))[0]
    hq = hq.copy()
    hq[tuple(i)] ^= 1  # neighbouring code: one E4M3 step
    with pytest.raises(AssertionError, match="oracle fixes differ"):
        assert_requant_valid(hq, hs, rng)


def test_rejects_a_wrong_scale():
    y1, S1, w2, b2 = chain_case()
    rng = requant_range(y1, S1, "gelu_tanh")
    hq, hs, _ = device_like(y1, S1, w2, b2)
    hs = hs.copy()
    hs[0, 1] += 1
    with pytest.raises(AssertionError, match="scale"):
        assert_requant_valid(hq, hs, rng)


def test_rejects_an_output_off_by_more_than_its_allowance():
    y1, S1, w2, b2 = chain_case()
    _, _, y2 = device_like(y1, S1, w2, b2)
    rng = requant_range(y1, S1, "gelu_tanh")
    qc = oracle.dequantize_mx(rng["codes"], rng["scales"])
    delta = np.maximum(rng["qhi"] - qc, qc - rng["qlo"])
    allow = delta @ np.abs(oracle.dequantize_mx(*w2)).T
    _, S2 = oracle.linear_ref(rng["codes"], rng["scales"], *w2, bias=b2)
    y2 = y2.copy()
    y2[2, 5] += 2 * allow[2, 5] + 3e-3 * S2[2, 5] + 1.0
    with pytest.raises(AssertionError, match="1 of"):
        assert_chain_close(y2, y1, S1, "gelu_tanh", *w2, b2)


def test_rejects_wrong_weights_in_the_second_linear():
    y1, S1, w2, b2 = chain_case()
    other = quant_ref(synth.make_weight(64, 128, 99))
    _, _, y2 = device_like(y1, S1, other, b2)
    with pytest.raises(AssertionError):
        assert_chain_close(y2, y1, S1, "gelu_tanh", *w2, b2)


def test_rejects_a_dropped_group_in_the_first_linear():
    # The device forgets the last 32-group of K in ffn.net.0.proj.
    x = synth.make_activation(6, 256, 3)
    w1, b1 = synth.make_weight(128, 256, 3), synth.make_bias(128, 3).double().numpy()
    xq, xs = quant_ref(x)
    xq_bad = xq.copy()
    xq_bad[:, -32:] = 0
    y1, S1 = oracle.linear_ref(xq, xs, *quant_ref(w1), bias=b1, epilogue="gelu_tanh")
    y1_bad, _ = oracle.linear_ref(xq_bad, xs, *quant_ref(w1), bias=b1, epilogue="gelu_tanh")
    hq, hs = oracle.quantize_mx(oracle.bf16_round(y1_bad))
    with pytest.raises(AssertionError):
        assert_requant_valid(hq, hs, requant_range(y1, S1, "gelu_tanh"))
