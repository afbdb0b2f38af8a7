"""The slab linear at its documented size limits, K = 2^20 and N = 2^20
(in-tile byte offsets stay below 2^30), through the slab GEMM, split-K and
the few-token kernel, every output element against the oracle.

Source of the rule: model card "Wan2.2-I2V-A14B-Lightning · MXFP8 (AutoRound
OptRTN)", section "Quantization Details".
"""

import pytest
import torch

import oracle
import synth
from helpers import assert_linear_close, dev, f64, mx, quant_ref

pytestmark = pytest.mark.gpu


def _run(M, K, N, plans, seed):
    d = dev()
    x = synth.make_activation(M, K, seed)
    w = synth.make_weight(N, K, seed)
    b = synth.make_bias(N, seed)
    xs = mx().mx_quantize_act_slab(x.to(d))
    ws = mx().mx_quantize_weight_slab(w.to(d))
    xq, xsc = quant_ref(x)
    wq, wsc = quant_ref(w)
    yref, S = oracle.linear_ref(xq, xsc, wq, wsc, bias=f64(b))
    for plan in plans:
        print(f"M={M} K={K} N={N} plan={plan}", flush=True)
        y = mx().mx_linear_slab_planned(plan, xs, ws, b.to(d))
        torch.cuda.synchronize()
        assert_linear_close(y, yref, S, what=f"{plan} {M}x{K}x{N}")
        del y
    del xs, ws
    torch.cuda.empty_cache()


def test_largest_k():
    _run(16, 1 << 20, 64, [("splitk", 8), ("small", 8), ("slab", 1)], seed=71)


def test_largest_n():
    _run(16, 64, 1 << 20, [("slab", 1), ("small", 1)], seed=72)
