"""Seeded random shapes through every slab-GEMM kernel kind against the
oracle: the slab GEMM, split-K, the few-token kernel (one and several K
ranges) and the balanced GEMM, with ragged M and N, K from one 64-K slab up,
GELU or not, bias or not; and two shapes with more tiles than CUs (several
rounds of tiles, a ragged last round). Each case: every output element
within 1e-3 g sum|a||b| + one bf16 ulp of the oracle, and the run repeated
(or the one-call path run) for bit-identical output.

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


def _cases(n=18, seed=2026):
    rng = np.random.default_rng(seed)
    kinds = ["slab", "splitk", "small", "balanced"]
    out = []
    for i in range(n):
        kind = kinds[i % len(kinds)]
        M = int(rng.integers(1, 700))
        N = 16 * int(rng.integers(1, 48))
        K = 64 * int(rng.integers(1, 16))
        splits = 1
        if kind in ("splitk", "small"):
            splits = int(rng.integers(1, min(8, K // 64) + 1))
        out.append((kind, splits, M, K, N, bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), 100 + i))
    return out


@pytest.mark.parametrize("kind,splits,M,K,N,gelu,bias,seed", _cases())
def test_random_shapes_every_kernel(kind, splits, M, K, N, gelu, bias, seed):
    print(f"{kind} s={splits} M={M} K={K} N={N} gelu={gelu} bias={bias}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed)
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed) if bias else None
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    bd = None if b is None else b.to(d)
    plan = (kind, splits)
    y1 = mx().mx_linear_slab_planned(plan, xs, ws, bd, gelu=gelu)
    y2 = mx().mx_linear_slab_planned(plan, xs, ws, bd, gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    xq, xsc = quant_ref(x)
    wq, wsc = quant_ref(w)
    yref, S = oracle.linear_ref(xq, xsc, wq, wsc, bias=None if b is None else f64(b),
                                epilogue="gelu_tanh" if gelu else "none")
    assert_linear_close(y1, yref, S, "gelu_tanh" if gelu else "none", what=f"{kind}{splits} {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,gelu", [(4365, 192, 4144, False), (4097, 320, 4112, True)])
def test_many_tiles_every_element(M, K, N, gelu):
    """More 256 x 256 tiles than CUs (several rounds, a ragged last round,
    ragged rows and columns), every output element against the oracle,
    through the slab GEMM and the one-call linear."""
    print(f"many tiles M={M} K={K} N={N} gelu={gelu}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, 71)
    w = synth.make_weight(N, K, 72)
    b = synth.make_bias(N, 73)
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    y1 = mx().mx_linear_slab(xs, ws, b.to(d), gelu=gelu)
    y2 = mx().mx_linear(x.to(d), ws, b.to(d), gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    xq, xsc = quant_ref(x)
    wq, wsc = quant_ref(w)
    yref, S = oracle.linear_ref(xq, xsc, wq, wsc, bias=f64(b), epilogue="gelu_tanh" if gelu else "none")
    assert_linear_close(y1, yref, S, "gelu_tanh" if gelu else "none", what=f"many tiles {M}x{K}x{N}")
