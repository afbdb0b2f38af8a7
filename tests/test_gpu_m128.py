"""GPU parity of the slab GEMM on 256 (weight rows) x 128 (tokens) tiles
(mx_linear_slab_m128): every output is the same chain of scaled MFMAs from
the bias as in mx_linear_slab, so the two must agree bit for bit; both are
checked against the oracle on every element (within 1e-3 g sum|a||b| + one
bf16 ulp). Shapes cover one 64-K slab and odd slab counts, ragged M (an odd
number of 128-token tiles, so the last one ends inside the slab's 256-row
padding) and ragged N, several rounds of tiles, and the 512-token text k|v
linear at full size.

Source of the rule: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
OptRTN)", section "Quantization Details".
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx, quant_ref

pytestmark = pytest.mark.gpu


def oracle_linear(x, w, b, gelu):
    xq, xs = quant_ref(x)
    wq, ws = quant_ref(w)
    return oracle.linear_ref(xq, xs, wq, ws, bias=None if b is None else f64(b),
                             epilogue="gelu_tanh" if gelu else "none")


def operands(M, K, N, seed, bias=True, x=None):
    d = dev()
    x = synth.make_activation(M, K, seed) if x is None else x
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed) if bias else None
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    return x, w, b, xs, ws, None if b is None else b.to(d)


CASES = [
    (1, 64, 16, False, True),
    (77, 128, 272, True, True),
    (128, 192, 256, False, False),
    (129, 64, 512, True, True),
    (300, 640, 528, False, True),
    (384, 320, 4112, True, False),
    (513, 1984, 1024, False, True),
    (700, 960, 784, True, True),
]


@pytest.mark.parametrize("M,K,N,gelu,bias", CASES)
def test_m128_equals_slab_and_oracle(M, K, N, gelu, bias):
    print(f"m128 M={M} K={K} N={N} gelu={gelu} bias={bias}", flush=True)
    x, w, b, xs, ws, bd = operands(M, K, N, seed=M + 7 * N + K, bias=bias)
    y128 = mx().mx_linear_slab_m128(xs, ws, bd, gelu=gelu)
    y = mx().mx_linear_slab(xs, ws, bd, gelu=gelu)
    yp = mx().mx_linear_slab_planned(("slab_m128", 1), xs, ws, bd, gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y128.view(torch.int16), y.view(torch.int16))
    assert torch.equal(yp.view(torch.int16), y.view(torch.int16))
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y128, yref, S, "gelu_tanh" if gelu else "none", what=f"m128 {M}x{K}x{N}")


def test_m128_more_tiles_than_cus():
    # 33 token tiles x 17 weight tiles: several rounds, a ragged last round.
    M, K, N = 4097, 192, 4112
    print(f"m128 many tiles M={M} K={K} N={N}", flush=True)
    x, w, b, xs, ws, bd = operands(M, K, N, seed=41)
    y128 = mx().mx_linear_slab_m128(xs, ws, bd, gelu=True)
    y = mx().mx_linear_slab(xs, ws, bd, gelu=True)
    torch.cuda.synchronize()
    assert torch.equal(y128.view(torch.int16), y.view(torch.int16))
    yref, S = oracle_linear(x, w, b, True)
    assert_linear_close(y128, yref, S, "gelu_tanh", what="m128 many tiles")


def test_m128_text_kv_full_size():
    # attn2 k|v on the 512 text tokens (zero-padded rows give bf16(bias)).
    shp = synth.CONFIGS["xattn_512x5120x10240"][0]
    ctx = synth.make_text_context(shp.M, shp.K, 35)
    print(f"m128 text k|v {shp}", flush=True)
    x, w, b, xs, ws, bd = operands(shp.M, shp.K, shp.N, 35, x=ctx)
    y128 = mx().mx_linear_slab_m128(xs, ws, bd, gelu=shp.gelu)
    y = mx().mx_linear_slab(xs, ws, bd, gelu=shp.gelu)
    torch.cuda.synchronize()
    assert torch.equal(y128.view(torch.int16), y.view(torch.int16))
    yref, S = oracle_linear(x, w, b, shp.gelu)
    assert_linear_close(y128, yref, S, "gelu_tanh" if shp.gelu else "none", what="m128 text k|v")
    pad = ~np.asarray(ctx.abs().sum(dim=1) > 0)
    assert pad.any()
    want = f64(b.float().to(torch.bfloat16))
    assert np.array_equal(f64(y128)[pad], np.broadcast_to(want, (int(pad.sum()), shp.N)))
