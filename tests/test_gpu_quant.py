"""GPU parity of the standalone MX quantizer (mx_quantize_act,
mx_quantize_weight) against the oracle: codes and scales bit-exact.

Source of the rule: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
OptRTN)", section "Quantization Details" (dynamic MXFP8 activations, E4M3
weights with per-32 E8M0 scales); OCP MX conversion for the shared exponent.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import dev, f64, mx, quant_ref, u8

pytestmark = pytest.mark.gpu


def bf16_from_bits(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def exhaustive_bf16_groups(K=1024):
    """Every finite bf16 pattern, in groups built to hit every reachable
    E8M0 code: for code c (e = c - 127) a group holds an anchor of magnitude
    2**(e+8) (so its scale is exactly c; for c = 0 the anchor is 2**-119)
    and 31 patterns whose magnitude stays below 2**(e+9)."""
    bits = np.arange(0x10000, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    mag_exp = (bits >> 7) & 0xFF  # biased exponent of each pattern
    groups = []
    for c in range(0, 247):
        e = c - 127
        if c == 0:
            anchor_exp, limit_exp = 8, 9  # 2**-119 has biased exponent 8; keep below 2**-118
        else:
            anchor_exp, limit_exp = e + 8 + 127, e + 9 + 127
        vals = bits[finite & (mag_exp < limit_exp)].astype(np.uint16)
        n = (len(vals) + 30) // 31
        pad = np.zeros(n * 31, dtype=np.uint16)
        pad[: len(vals)] = vals
        body = pad.reshape(n, 31)
        anchor = np.full((n, 1), anchor_exp << 7, dtype=np.uint16)
        anchor[1::2] |= 0x8000  # alternate the anchor's sign
        groups.append(np.concatenate([anchor, body], axis=1))
    g = np.concatenate(groups)
    per_row = K // 32
    rows = (len(g) + per_row - 1) // per_row
    out = np.zeros((rows * per_row, 32), dtype=np.uint16)
    out[: len(g)] = g
    return bf16_from_bits(out.reshape(rows, K))


def test_act_quantizer_exhaustive_bf16_sweep():
    x = exhaustive_bf16_groups()
    print(f"exhaustive sweep: {tuple(x.shape)} bf16", flush=True)
    q, s = mx().mx_quantize_act(x.to(dev()))
    torch.cuda.synchronize()
    rq, rs = quant_ref(x)
    assert np.unique(rs).size >= 247  # every reachable scale code occurs
    assert np.array_equal(u8(s), rs)
    assert np.array_equal(u8(q), rq)


def test_act_quantizer_nonfinite_groups():
    x = synth.make_activation(4, 256, seed=3)
    x[0, 5] = float("nan")
    x[1, 40] = float("inf")
    x[2, 255] = float("-inf")
    x[3, 64:96] = float("nan")
    q, s = mx().mx_quantize_act(x.to(dev()))
    rq, rs = quant_ref(x)
    assert np.array_equal(u8(s), rs) and np.array_equal(u8(q), rq)
    assert u8(s)[0, 0] == 0xFF and np.all(u8(q)[0, :32] == 0x7F)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (300, 5120), (129, 13824)])
def test_act_quantizer_synthetic(M, K):
    x = synth.make_activation(M, K, seed=M + K)
    q, s = mx().mx_quantize_act(x.to(dev()))
    rq, rs = quant_ref(x)
    assert np.array_equal(u8(s), rs) and np.array_equal(u8(q), rq)


def test_act_quantizer_text_context_zero_rows():
    x = synth.make_text_context(512, 5120, seed=0)
    q, s = mx().mx_quantize_act(x.to(dev()))
    rq, rs = quant_ref(x)
    assert np.array_equal(u8(s), rs) and np.array_equal(u8(q), rq)
    assert np.all(u8(s)[410:] == 0) and np.all(u8(q)[410:] == 0)


def test_act_quantizer_strided_rows():
    base = synth.make_activation(70, 384, seed=9).to(dev())
    x = base[:, 64:320]  # pitch 384, K 256
    q, s = mx().mx_quantize_act(x)
    rq, rs = quant_ref(x.cpu())
    assert np.array_equal(u8(s), rs) and np.array_equal(u8(q), rq)


def test_act_quantizer_empty():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev())
    q, s = mx().mx_quantize_act(x)
    assert q.shape == (0, 256) and s.shape == (0, 8)


def test_act_quantizer_full_size_sampled_rows():
    M, K = synth.VIDEO_TOKENS, synth.HIDDEN
    x = synth.make_activation(M, K, seed=0)
    print(f"full-size act quantize {M}x{K}", flush=True)
    q, s = mx().mx_quantize_act(x.to(dev()))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 100, M), rng.integers(0, M, 1024)]))
    rq, rs = oracle.quantize_mx(f64(x[rows]))
    assert np.array_equal(u8(s[rows]), rs) and np.array_equal(u8(q[rows]), rq)


def f32_tie_groups(n_groups, seed):
    """f32 groups whose elements sit on, and one f32 ulp either side of, the
    E4M3 rounding midpoints, at random shared exponents; plus denormal and
    huge groups."""
    rng = np.random.default_rng(seed)
    mags = oracle.e4m3_decode(np.arange(127))
    mids = (mags[:-1] + mags[1:]) / 2
    e = rng.integers(-125, 119, size=(n_groups, 1))
    t = rng.choice(mids, size=(n_groups, 32)).astype(np.float32)
    nudge = rng.integers(-1, 2, size=t.shape)
    t = np.nextafter(t, np.where(nudge > 0, np.inf, -np.inf).astype(np.float32)) * (nudge != 0) + t * (nudge == 0)
    t[:, 0] = 448.0 + 30.0  # anchor in [256, 512): scale is exactly e; saturates
    t *= rng.choice([-1.0, 1.0], size=t.shape).astype(np.float32)
    v = (t.astype(np.float64) * np.exp2(e.astype(np.float64))).astype(np.float32)
    # denormal-only groups (scale code 0) and groups near the f32 maximum
    v[0, :] = (rng.standard_normal(32) * 2.0**-135).astype(np.float32)
    v[1, :] = (rng.standard_normal(32) * 2.0**-146).astype(np.float32)
    v[2, :] = (rng.standard_normal(32) * 1e38).astype(np.float32)
    v[3, :] = 0.0
    v[3, 7] = -0.0
    return torch.from_numpy(v.reshape(-1, 256))


def test_weight_quantizer_f32_ties_denormals_extremes():
    w = f32_tie_groups(4096, seed=1)
    q, s = mx().mx_quantize_weight(w.to(dev()))
    rq, rs = quant_ref(w)
    assert np.array_equal(u8(s), rs)
    assert np.array_equal(u8(q), rq)


def test_weight_quantizer_f32_nonfinite():
    w = synth.make_weight(2, 128, seed=4)
    w[0, 3] = float("nan")
    w[1, 100] = float("inf")
    q, s = mx().mx_quantize_weight(w.to(dev()))
    rq, rs = quant_ref(w)
    assert np.array_equal(u8(s), rs) and np.array_equal(u8(q), rq)


@pytest.mark.parametrize("N,K", [(256, 5120), (15360, 5120), (5120, 13824)])
def test_weight_quantizer_f32_wan_shapes(N, K):
    w = synth.make_weight(N, K, seed=N)
    q, s = mx().mx_quantize_weight(w.to(dev()))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N), np.random.default_rng(N).integers(0, N, 512)]))
    rq, rs = oracle.quantize_mx(f64(w[rows]))
    assert np.array_equal(u8(s[rows]), rs) and np.array_equal(u8(q[rows]), rq)


def test_weight_quantizer_bf16():
    w = synth.make_weight(512, 1024, seed=2).to(torch.bfloat16)
    q, s = mx().mx_quantize_weight(w.to(dev()))
    rq, rs = quant_ref(w)
    assert np.array_equal(u8(s), rs) and np.array_equal(u8(q), rq)
