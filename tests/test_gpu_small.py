"""GPU parity of the few-token GEMM (mx_linear_slab_small: 128-token x
64-weight-row tiles, K split into ranges) against the oracle, on the same
seeded inputs as the slab tests: within 1e-3 g sum|a||b| + one bf16 ulp,
every element; with one range bit-identical to mx_linear_slab (the same
MFMA chain over K and the same epilogue); deterministic with several ranges.

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


@pytest.mark.parametrize(
    "M,K,N,splits,gelu,bias",
    [(1, 64, 16, 1, False, True), (5, 64, 64, 1, True, False), (77, 192, 272, 3, False, True),
     (128, 512, 512, 4, True, True), (256, 128, 256, 2, False, True), (300, 320, 512, 5, True, True),
     (513, 512, 272, 8, False, False), (129, 5120, 768, 80, False, True), (70, 5120, 768, 1, True, True)],
)
def test_small_matches_oracle(M, K, N, splits, gelu, bias):
    print(f"small M={M} K={K} N={N} splits={splits} gelu={gelu}", flush=True)
    x, w, b, xs, ws, bd = operands(M, K, N, seed=M * 7 + K + N, bias=bias)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
    mx().mx_linear_slab_small(xs, ws, bd, gelu=gelu, y=y, splits=splits)
    y2 = mx().mx_linear_slab_small(xs, ws, bd, gelu=gelu, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed order, every element written
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y, yref, S, "gelu_tanh" if gelu else "none", what=f"small {M}x{K}x{N} s{splits}")


@pytest.mark.parametrize("M,K,N", [(128, 512, 512), (300, 320, 272), (1, 64, 16), (513, 256, 1024), (128, 5120, 1280)])
def test_small_single_range_equals_slab(M, K, N):
    x, w, b, xs, ws, bd = operands(M, K, N, seed=M + K)
    for gelu in (False, True):
        y1 = mx().mx_linear_slab(xs, ws, bd, gelu=gelu)
        y2 = mx().mx_linear_slab_small(xs, ws, bd, gelu=gelu, splits=1)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("cfg", ["single_128x5120x5120", "xattn_512x5120x10240"])
def test_small_token_configs(cfg):
    # The few-token linears at their full sizes with the chosen split count;
    # every output element against the oracle.
    shp = synth.CONFIGS[cfg][0]
    x = synth.make_text_context(shp.M, shp.K, 33) if shp.M == synth.TEXT_TOKENS else None
    x, w, b, xs, ws, bd = operands(shp.M, shp.K, shp.N, 33, x=x)
    splits = mx().mx_linear_small_choose(shp.M, shp.K, shp.N)
    print(f"small {cfg} {shp} splits={splits}", flush=True)
    y = mx().mx_linear_slab_small(xs, ws, bd, gelu=shp.gelu)
    torch.cuda.synchronize()
    yref, S = oracle_linear(x, w, b, shp.gelu)
    assert_linear_close(y, yref, S, "gelu_tanh" if shp.gelu else "none", what=cfg)


def test_small_zero_text_rows_give_bias():
    # Zero-padded text rows: every code 0, so the output is bf16(bias).
    ctx = synth.make_text_context(512, 1024, seed=8)
    x, w, b, xs, ws, bd = operands(512, 1024, 512, 8, x=ctx)
    y = mx().mx_linear_slab_small(xs, ws, bd, splits=4)
    torch.cuda.synchronize()
    want = f64(b.float().to(torch.bfloat16))
    assert np.array_equal(f64(y)[410:], np.broadcast_to(want, (102, 512)))


def test_small_bad_arguments():
    M, K, N = 128, 256, 256
    _, _, _, xs, ws, bd = operands(M, K, N, 3)
    with pytest.raises(RuntimeError, match="splits"):
        mx().mx_linear_slab_small(xs, ws, bd, splits=5)  # K/64 = 4
    small_ws = torch.empty(16, dtype=torch.uint8, device=dev())
    with pytest.raises(RuntimeError, match="workspace"):
        mx().mx_linear_slab_small(xs, ws, bd, splits=2, workspace=small_ws)


@pytest.mark.parametrize("M,K,N,kind", [(128, 512, 512, "small"), (512, 1024, 1024, "splitk"), (4096, 128, 4096, "slab")])
def test_planned_linear_matches_oracle(M, K, N, kind):
    # The per-shape choice (few-token kernel, split-K or the slab GEMM)
    # computes the same linear: every element against the oracle.
    plan = mx().plan_linear(M, K, N)
    assert plan[0] == kind
    x, w, b, xs, ws, bd = operands(M, K, N, seed=M + N + 1)
    nb = mx().plan_ws_bytes(plan, M, N)
    wsp = torch.empty((nb,), dtype=torch.uint8, device=dev()) if nb > 0 else None
    y = mx().mx_linear_slab_planned(plan, xs, ws, bd, gelu=True, workspace=wsp)
    torch.cuda.synchronize()
    yref, S = oracle_linear(x, w, b, True)
    assert_linear_close(y, yref, S, "gelu_tanh", what=f"planned {kind}")


@pytest.mark.parametrize("M,K,N,gelu", [(128, 5120, 5120, False), (512, 1024, 1024, True), (300, 640, 2048, False)])
def test_tuned_plan_is_cached_and_matches_oracle(M, K, N, gelu):
    # Warm-up tuning picks one of the candidate kernels for the shape, caches
    # it, and the auto entry point then runs that plan: same bits as calling
    # the plan directly, and the oracle's result within the tolerance.
    print(f"tune M={M} K={K} N={N}", flush=True)
    mx().mx_linear_plan_clear()
    assert mx().plan_lookup(M, K, N, gelu) == mx().plan_linear(M, K, N)
    x, w, b, xs, ws, bd = operands(M, K, N, seed=M + K + 7)
    plan = mx().mx_linear_tune(xs, ws, bd, gelu=gelu, reps=3)
    assert plan[0] in ("slab", "splitk", "small", "balanced", "slab_m128")
    assert mx().plan_lookup(M, K, N, gelu) == plan
    y_auto = mx().mx_linear_slab_auto(xs, ws, bd, gelu=gelu)
    y_plan = mx().mx_linear_slab_planned(plan, xs, ws, bd, gelu=gelu)
    torch.cuda.synchronize()
    assert torch.equal(y_auto.view(torch.int16), y_plan.view(torch.int16))
    yref, S = oracle_linear(x, w, b, gelu)
    assert_linear_close(y_auto, yref, S, "gelu_tanh" if gelu else "none", what=f"auto {plan}")
    mx().mx_linear_plan_clear()
    assert mx().plan_lookup(M, K, N, gelu) == mx().plan_linear(M, K, N)


def test_tune_without_workspace_keeps_to_plans_that_need_none():
    M, K, N = 128, 1024, 1024
    x, w, b, xs, ws, bd = operands(M, K, N, seed=5)
    empty = torch.empty((0,), dtype=torch.uint8, device=dev())
    plan = mx().mx_linear_tune(xs, ws, bd, workspace=empty, reps=2)
    assert plan in (("slab", 1), ("small", 1))
    y = mx().mx_linear_slab_auto(xs, ws, bd)
    torch.cuda.synchronize()
    yref, S = oracle_linear(x, w, b, False)
    assert_linear_close(y, yref, S, what=f"auto {plan}")
    mx().mx_linear_plan_clear()


def test_mfma_probe_sums_exactly():
    # Codes 0x38 (1.0) everywhere with unit block scales: each MFMA adds 64 to
    # each of its 32 x 32 accumulators, so a thread's sum of its 16 blocks of
    # 16 accumulators after `iters` rounds is 256 * 64 * iters, exact in fp32.
    d = dev()
    ones = torch.full((4096,), 0x38, dtype=torch.uint8, device=d)
    sink = torch.full((2 * 256,), float("nan"), dtype=torch.float32, device=d)
    flop = mx().mx_probe_mfma(ones, ones, 3, 2, sink)
    torch.cuda.synchronize()
    assert flop == 2 * 4 * 16 * 3 * 2 * 32 * 32 * 64
    assert torch.equal(sink.cpu(), torch.full((512,), 256.0 * 64 * 3))
    zeros = torch.zeros(4096, dtype=torch.uint8, device=d)
    mx().mx_probe_mfma(zeros, ones, 3, 2, sink)
    torch.cuda.synchronize()
    assert not sink.any()
