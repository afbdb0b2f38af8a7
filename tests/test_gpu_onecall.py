"""The one-call linear (mx_linear): quantizer into the caller's workspace,
then the GEMM through the shape's plan (tuned, else the default rule).

Each case: the output equals the two-call path with the same plan
(mx_quantize_act_slab + mx_linear_slab_planned) bit for bit, and the oracle
within 1e-3 g sum|a||b| + one bf16 ulp on every element. The workspace needs
no initial value, so it is filled with 0xFF first and the call is repeated.

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
    return oracle.linear_ref(*quant_ref(x), *quant_ref(w), bias=None if b is None else f64(b),
                             epilogue="gelu_tanh" if gelu else "none")


CASES = [
    # M, K, N, gelu, bias: the default plan is the few-token kernel with
    # several K ranges up to 256 tokens; above, the 128-token tiles (640 x
    # 512 x 4096: 48 tiles of 256 x 256), split-K or the slab GEMM.
    (128, 5120, 5120, False, True),
    (77, 640, 272, True, True),
    (200, 256, 512, False, False),
    (1, 1024, 16, True, True),
    (256, 13824, 1024, False, True),
    (300, 512, 768, True, True),
    (1000, 512, 512, False, True),
    (640, 512, 4096, True, False),
]


@pytest.mark.parametrize("M,K,N,gelu,bias", CASES)
def test_one_call_matches_plan_and_oracle(M, K, N, gelu, bias):
    mx().mx_linear_plan_clear()
    plan = mx().plan_linear(M, K, N)
    print(f"one-call M={M} K={K} N={N} gelu={gelu} bias={bias} plan={plan}", flush=True)
    d = dev()
    x = synth.make_activation(M, K, seed=M + K + N)
    w = synth.make_weight(N, K, seed=M + 1)
    b = synth.make_bias(N, seed=M + 2) if bias else None
    xd, bd = x.to(d), None if b is None else b.to(d)
    wsl = mx().mx_quantize_weight_slab(w.to(d))
    ws = torch.full((mx().mx_linear_ws_bytes(M, K, N),), 0xFF, dtype=torch.uint8, device=d)
    y1 = mx().mx_linear(xd, wsl, bd, gelu=gelu, workspace=ws)
    y2 = mx().mx_linear(xd, wsl, bd, gelu=gelu, workspace=ws)
    y3 = mx().mx_linear_slab_planned(plan, mx().mx_quantize_act_slab(xd), wsl, bd, gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "repeat differs"
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16)), "differs from the two-call path"
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y1, yref, S, "gelu_tanh" if gelu else "none", what=f"one-call {plan}")


def test_one_call_takes_the_tuned_plan():
    """After mx_linear_tune caches a plan for the shape, mx_linear runs that
    plan (bit-identical to it); a workspace too small for the cached plan's
    partial sums makes it fall back to the default plan."""
    M, K, N = 128, 1024, 2048
    d = dev()
    x = synth.make_activation(M, K, seed=31).to(d)
    wsl = mx().mx_quantize_weight_slab(synth.make_weight(N, K, seed=31).to(d))
    b = synth.make_bias(N, seed=31).to(d)
    xs = mx().mx_quantize_act_slab(x)
    mx().mx_linear_plan_clear()
    default = mx().plan_linear(M, K, N)
    tuned = mx().mx_linear_tune(xs, wsl, b, reps=3)
    assert mx().plan_lookup(M, K, N) == tuned
    y = mx().mx_linear(x, wsl, b)
    ref = mx().mx_linear_slab_planned(tuned, xs, wsl, b)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    # Force a cached plan with large partials, then give only the minimum.
    mx().mx_linear_plan_clear()
    big = ("small", 8)
    base = mx().mx_linear_ws_bytes(M, K, N) - mx().mx_linear_tune_ws_bytes(M, K, N)
    ws_min = torch.empty((base + mx().plan_ws_bytes(default, M, N, K),), dtype=torch.uint8, device=d)
    if mx().plan_ws_bytes(big, M, N, K) > mx().plan_ws_bytes(default, M, N, K):
        y_min = mx().mx_linear(x, wsl, b, workspace=ws_min)
        ref_d = mx().mx_linear_slab_planned(default, xs, wsl, b)
        torch.cuda.synchronize()
        assert torch.equal(y_min.view(torch.int16), ref_d.view(torch.int16))
    mx().mx_linear_plan_clear()


def test_one_call_nonfinite_few_token_ranges():
    """NaN / Inf groups on the few-token plan with K ranges: NaN rows and
    columns exactly where the oracle has them."""
    M, K, N = 100, 640, 272
    d = dev()
    x = synth.make_activation(M, K, seed=71)
    w = synth.make_weight(N, K, seed=71)
    b = synth.make_bias(N, seed=71)
    x[3, 70], x[60, 600], x[M - 1, 0] = float("nan"), float("inf"), -float("inf")
    w[7, 9], w[N - 1, 320] = float("inf"), float("nan")
    plan = mx().plan_linear(M, K, N)
    assert plan[0] == "small" and plan[1] > 1
    y = mx().mx_linear(x.to(d), mx().mx_quantize_weight_slab(w.to(d)), b.to(d))
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        yref, S = oracle_linear(x, w, b, False)
    assert_linear_close(y, yref, S, what="one-call nonfinite")


def test_one_call_graph_replays_match_eager():
    """The one-call linear on the few-token plan (quantizer, GEMM over K
    ranges, ordered reduction) captured in a HIP graph: replays with eager
    work between them equal the eager call bit for bit."""
    M, K, N = 128, 1024, 1024
    d = dev()
    inputs = [synth.make_activation(M, K, seed=s).to(d) for s in (81, 82, 83)]
    wsl = mx().mx_quantize_weight_slab(synth.make_weight(N, K, seed=84).to(d))
    b = synth.make_bias(N, seed=84).to(d)
    mx().mx_linear_plan_clear()
    assert mx().plan_linear(M, K, N)[0] == "small"
    x = inputs[0].clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    ws = torch.empty((mx().mx_linear_ws_bytes(M, K, N),), dtype=torch.uint8, device=d)

    def step():
        mx().mx_linear(x, wsl, b, y=y, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep, xin in enumerate(inputs + inputs[:1]):
        x.copy_(xin)
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), y.view(torch.int16)), f"replay {rep}"
    del g
