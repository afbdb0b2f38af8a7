"""GPU parity of the MXFP8 W8A8 linear (mx_linear with the fused activation
quantization, mx_linear_q on pre-quantized activations) against the oracle:
every output within 1e-3 g sum|a||b| + one bf16 ulp (g = 1, or 1.13 through
GELU-tanh), and bit-exact where the result is exact.

Source: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound OptRTN)",
section "Quantization Details" (W8A8 MXFP8 linears with F16 biases); FP32
accumulation per "Model Quantization Techniques", Conv3D mode table.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_chain_close, assert_linear_close, dev, f64, mx, quant_ref

pytestmark = pytest.mark.gpu


def run_case(M, K, N, seed, bias=True, gelu=False, fused=True, x=None):
    d = dev()
    x = synth.make_activation(M, K, seed) if x is None else x
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed) if bias else None
    wq, ws = mx().mx_quantize_weight(w.to(d))
    if fused:
        y = mx().mx_linear_fused(x.to(d), wq, ws, None if b is None else b.to(d), gelu=gelu)
    else:
        xq, xs = mx().mx_quantize_act(x.to(d))
        y = mx().mx_linear_q(xq, xs, wq, ws, None if b is None else b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    return x, w, b, wq, ws, y


def oracle_linear(x, w, b, gelu, wref=None):
    """The oracle's linear on the seeded inputs (wref: the oracle's codes and
    scales of w, when the caller has them already)."""
    xq, xs = quant_ref(x)
    wq, ws = quant_ref(w) if wref is None else wref
    return oracle.linear_ref(xq, xs, wq, ws, bias=None if b is None else f64(b),
                             epilogue="gelu_tanh" if gelu else "none")


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize(
    "M,K,N",
    [(1, 32, 16), (5, 64, 32), (77, 96, 256), (256, 128, 256), (300, 160, 512), (513, 512, 272), (70, 5120, 768)],
)
def test_linear_small_shapes(M, K, N, fused):
    print(f"linear M={M} K={K} N={N} fused={fused}", flush=True)
    x, w, b, wq, ws, y = run_case(M, K, N, seed=M * 7 + K + N, fused=fused)
    yref, S = oracle_linear(x, w, b, False)
    assert_linear_close(y, yref, S, what=f"M{M} K{K} N{N}")


@pytest.mark.parametrize("fused", [True, False])
def test_linear_gelu_no_bias(fused):
    x, w, b, wq, ws, y = run_case(300, 256, 512, seed=5, bias=False, gelu=True, fused=fused)
    yref, S = oracle_linear(x, w, None, True)
    assert_linear_close(y, yref, S, "gelu_tanh", what="gelu")


def test_fused_equals_prequantized_bitwise():
    d = dev()
    x = synth.make_activation(600, 1024, seed=11).to(d)
    w = synth.make_weight(512, 1024, seed=11).to(d)
    b = synth.make_bias(512, seed=11).to(d)
    wq, ws = mx().mx_quantize_weight(w)
    y1 = mx().mx_linear_fused(x, wq, ws, b, gelu=True)
    xq, xs = mx().mx_quantize_act(x)
    y2 = mx().mx_linear_q(xq, xs, wq, ws, b, gelu=True)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_identity_weight_reproduces_quantized_input_bitwise():
    # W = I (N = K): y = xhat exactly (products with 256 * 2**-8, sums of one
    # nonzero term), so y == bf16(xhat) bit for bit. This ties the fused
    # prologue's codes and scales to the oracle quantizer.
    d = dev()
    K = 1024
    rng = np.random.default_rng(3)
    x = synth.make_activation(1000, K, seed=3)
    x = (x.double() * torch.from_numpy(np.exp2(rng.integers(-60, 60, size=(1000, 1))))).to(torch.bfloat16)
    eye = torch.eye(K, dtype=torch.float32)
    wq, ws = mx().mx_quantize_weight(eye.to(d))
    y = mx().mx_linear_fused(x.to(d), wq, ws)
    xq, xs = mx().mx_quantize_act(x.to(d))
    y2 = mx().mx_linear_q(xq, xs, wq, ws)
    torch.cuda.synchronize()
    rq, rs = quant_ref(x)
    want = oracle.mx_oracle.bf16_round(oracle.dequantize_mx(rq, rs))
    assert np.array_equal(f64(y), want)
    assert np.array_equal(f64(y2), want)


def test_zero_rows_give_bias():
    d = dev()
    ctx = synth.make_text_context(512, 5120, seed=0)
    x, w, b, wq, ws, y = run_case(512, 5120, 1024, seed=0, x=ctx)
    yg = f64(y)
    want = f64(b.float().to(torch.bfloat16))  # bf16(f32(bias))
    assert np.array_equal(yg[410:], np.broadcast_to(want, (102, 1024)))
    yref, S = oracle_linear(x, w, b, False)
    assert_linear_close(y, yref, S, what="text ctx")


def test_deterministic_and_fully_written():
    d = dev()
    x = synth.make_activation(333, 512, seed=21).to(d)
    w = synth.make_weight(768, 512, seed=21).to(d)
    wq, ws = mx().mx_quantize_weight(w)
    y1 = torch.full((333, 768), float("nan"), dtype=torch.bfloat16, device=d)
    y2 = torch.full((333, 768), float("nan"), dtype=torch.bfloat16, device=d)
    mx().mx_linear_fused(x, wq, ws, y=y1)
    mx().mx_linear_fused(x, wq, ws, y=y2)
    torch.cuda.synchronize()
    assert not torch.isnan(y1).any()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_empty_batch():
    d = dev()
    w = synth.make_weight(256, 128, seed=1).to(d)
    wq, ws = mx().mx_quantize_weight(w)
    y = mx().mx_linear_fused(torch.empty((0, 128), dtype=torch.bfloat16, device=d), wq, ws)
    assert y.shape == (0, 256)


def sampled_rows(M, n=96, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(4), np.arange(M - 84, M), rng.integers(0, M, n)]))


@pytest.mark.parametrize("cfg", ["single_128x5120x5120", "qkv_75348x5120x15360", "xattn_512x5120x10240"])
def test_workload_configs(cfg):
    d = dev()
    for li, shp in enumerate(synth.CONFIGS[cfg]):
        print(f"{cfg} {shp}", flush=True)
        seed = 100 + li
        x = (synth.make_text_context(shp.M, shp.K, seed) if shp.M == synth.TEXT_TOKENS
             else synth.make_activation(shp.M, shp.K, seed))
        w = synth.make_weight(shp.N, shp.K, seed)
        b = synth.make_bias(shp.N, seed)
        wq, ws = mx().mx_quantize_weight(w.to(d))
        xd = x.to(d)
        y = mx().mx_linear_fused(xd, wq, ws, b.to(d), gelu=shp.gelu)
        torch.cuda.synchronize()
        rows = np.arange(shp.M) if shp.M <= 512 else sampled_rows(shp.M)
        yref, S = oracle_linear(x[rows], w, b, shp.gelu)
        assert_linear_close(y[rows], yref, S, "gelu_tanh" if shp.gelu else "none", what=f"{cfg}/{shp.name}")
        del y, xd


def test_ffn_chain_requantizes_intermediate():
    # ffn.net.0.proj (GELU) then ffn.net.2 on the bf16 intermediate h, which
    # the second call quantizes on the fly. h is held to the oracle's first
    # linear; the down-projection to the oracle's whole chain from the seeded
    # inputs (assert_chain_close).
    d = dev()
    up, down = synth.CONFIGS["ffn_75348x5120x13824"]
    M = 2048 + 84  # several token tiles and the same ragged tail as 75348
    x = synth.make_activation(M, up.K, 7)
    w1, b1 = synth.make_weight(up.N, up.K, 7), synth.make_bias(up.N, 7)
    w2, b2 = synth.make_weight(down.N, down.K, 8), synth.make_bias(down.N, 8)
    w1q, w1s = mx().mx_quantize_weight(w1.to(d))
    w2q, w2s = mx().mx_quantize_weight(w2.to(d))
    h = mx().mx_linear_fused(x.to(d), w1q, w1s, b1.to(d), gelu=True)
    y = mx().mx_linear_fused(h, w2q, w2s, b2.to(d))
    torch.cuda.synchronize()
    rows = sampled_rows(M, 64, seed=1)
    href, S1 = oracle_linear(x[rows], w1, b1, True)
    assert_linear_close(h[rows], href, S1, "gelu_tanh", what="ffn up")
    assert_chain_close(y[rows], href, S1, "gelu_tanh", *quant_ref(w2), f64(b2), what="ffn down")
